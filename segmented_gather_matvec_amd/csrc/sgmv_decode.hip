// sgmv_decode.hip - one-launch SGMV for decode-shaped segments (gfx950).
//
// Computes the LoRA term of the Punica README (page "Punica：多 LoRA 模型统一服务框架",
// LoRA and multi-LoRA paragraphs), Y[i] += (X[i] @ A_k) @ B_k, for segments of
// at most RB rows per unit, in a single launch:
//
//   * `splits` workgroups share a unit; split g owns input rows
//     [g*kc, (g+1)*kc) of A_k and output columns [g*cw, (g+1)*cw) of B_k.
//   * Every workgroup issues all of its HBM loads (its A_k chunk, X values,
//     its B_k chunk and Y values) up front in straight-line code, so the whole
//     call is in flight at once.
//   * Shrink partial sums are reduced inside each wave, then published as
//     64-bit words {fp32 value, launch tag}: one device-coherent atomic store
//     carries both the datum and its validity, so no counter, fence or cache
//     flush is needed.  Each workgroup polls the partials of its unit until
//     every tag matches, sums them in a fixed order (bitwise reproducible),
//     and expands its column chunk with the B_k values it already holds in
//     registers (each thread consumes exactly the B_k vectors it loaded).
//   * The launch tag mixes the dispatch packet id with the queue address, so it
//     changes on every launch, including replays of a captured graph; it is
//     always odd, so a zero-filled workspace never matches.
//   * Workgroups are dispatched round-robin over the 8 XCDs.  With one-row
//     segments the splits of a unit are placed on one XCD; when segments
//     hold several rows that share a LoRA, split-major order instead places
//     equal splits of neighbouring units (the same A_k / B_k slice) on one
//     XCD, so those slices are fetched from HBM once per XCD.
//   * The grid is sized by the host to be co-resident, so every wait ends when
//     the launch has the device to itself.  Each wait is still bounded: past a
//     deadline on the constant-rate real-time counter the workgroup gives up,
//     sets a bit in the device error word and exits without touching Y (the
//     case of another kernel holding the CUs that the unit's other workgroups
//     need).
#include <mutex>

#include "sgmv_device.h"
#include "sgmv_plan.h"
#include "sgmv_units.h"

namespace sgmv {

// Sticky error bits of the decode route on this device (SGMV_DEVICE_ERR_*),
// read and cleared by sgmv_take_device_errors.
__device__ __align__(256) uint32_t decode_errors;

namespace {

constexpr int kXcds = 8;
// Tagged words each thread polls per round: enough for the unit's outputs of
// V times 16 splits (every plan of H1 up to 8192 at rank 16), at most 8; a
// plan with more splits takes several rounds.  Fewer poll registers leave
// more of the register budget to the streamed A_k and B_k.
constexpr int poll_per_thread(int rb, int r) {
  return rb * r * 16 / kThreads < 1 ? 1 : rb * r * 16 / kThreads > 4 ? 4 : rb * r * 16 / kThreads;
}


// Value of a 64-bit lane variable in lane `l` (l uniform over the wave).
__device__ inline uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Lane exchanges inside a quad of lanes (DPP, no LDS traffic).
__device__ inline float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ inline float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

template <int H>
__device__ inline void halve(float (&v)[8], int lane, int mask) {
  const bool upper = (lane & mask) != 0;
#pragma unroll
  for (int q = 0; q < H; ++q) {
    const float send = upper ? v[q] : v[q + H];
    const float keep = upper ? v[q + H] : v[q];
    v[q] = keep + shfl_xor(send, mask);
  }
}

template <int R>
constexpr int log2_groups() {
  return R == 8 ? 0 : R == 16 ? 1 : R == 32 ? 2 : 3;
}

// SMALL: at most 64 LoRAs (pointer tables fetched one entry per lane).
// MAP: rows of X / Y are looked up in a row map.
// HET: per-LoRA ranks (compact A_k [h_in, r_k], B_k [r_k, h_out]; ranks
// r_k..R-1 are zero) and / or per-LoRA scales may be given.
// INL: the segment bounds and each segment's A_k / B_k come in the kernel
// arguments (m) instead of device tables, so they arrive with the other
// arguments rather than one dependent memory trip later.
// Each feature is a template flag, so a call pays only for what it uses.
template <class T, int R, int RB, bool SMALL, bool MAP, bool HET, bool INL>
__device__ __forceinline__ void decode_body(const DecodeParams& p, const InlineMeta* m) {
  constexpr int JG = R / 8;                  // 128-bit vectors per row of A_k
  constexpr int B0 = log2_groups<R>();
  constexpr int HS = kThreads / JG;          // A_k rows covered by one sweep of the workgroup
  constexpr int NA = decode_rows_per_thread(R);  // A_k rows per thread
  constexpr int KCMAX = NA * HS;             // = decode_max_kc(R)
  constexpr int JQ = kDecodeLanesPerColumn;  // lanes sharing one 8-column vector of B_k
  constexpr int NB = R / JQ;                 // B_k vectors per thread
  constexpr int NY = (RB + JQ - 1) / JQ;     // Y vectors per thread
  constexpr int PW = 1;                      // published partials per workgroup
  constexpr int NXV = RB == 1 ? 1 : (RB * KCMAX / 8 + kThreads - 1) / kThreads;
  constexpr int kPollPerThread = poll_per_thread(RB, R);
  constexpr int kStage = kThreads * kPollPerThread;
  static_assert(RB * R <= kThreads, "one output of V per thread");

  __shared__ __attribute__((aligned(16))) uint16_t lds_x[RB == 1 ? 8 : RB * KCMAX];
  __shared__ float lds_red[kWaves * RB * R];
  __shared__ float lds_stage[kStage];
  __shared__ float lds_v[RB * R];
  __shared__ int lds_gave_up;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  // INL: lane l fetches segment l's bounds and pointers from the kernel
  // arguments before anything else (entries past num_segs are not used), so
  // these loads depend on nothing and go out with the first argument loads.
  int lo_l = 0, hi_l = 0;
  uint64_t a_lane = 0, b_lane = 0;
  if constexpr (INL) {
    lo_l = m->seg[lane];
    hi_l = m->seg[lane + 1];
    a_lane = m->a[lane];
    b_lane = m->b[lane];
    // Consumed here, the loads stay ahead of the first branch and overlap the
    // argument loads; otherwise the compiler sinks them past the argument
    // checks, one memory trip later.
    asm volatile("" ::"v"(lo_l), "v"(hi_l), "v"(a_lane), "v"(b_lane));
  }
  const int G = p.splits;
  // Every projection's entry is loaded at a constant offset and blockIdx.y
  // selects one: loads at an offset computed from blockIdx.y were issued only
  // after the first argument loads had returned, a second trip before the
  // first metadata load.
  // With the rank and scale tables, the whole-struct copy under a condition
  // went through a stack copy of all entries (private memory on the critical
  // path: mixed-rank batch 13.9 us instead of 9.2 us), so those kernels select
  // field by field; the others keep the struct copy, which the compiler turns
  // into one load at a selected offset (0.2 us faster than selecting fields).
  Projection pr = p.proj[0];
  if constexpr (!INL) {  // (INL launches one projection)
#pragma unroll
    for (int i = 1; i < kMaxProjections; ++i) {
      if constexpr (HET) {
        const bool s = (int)blockIdx.y == i;
        pr.A_ptrs = s ? p.proj[i].A_ptrs : pr.A_ptrs;
        pr.B_ptrs = s ? p.proj[i].B_ptrs : pr.B_ptrs;
        pr.Y = s ? p.proj[i].Y : pr.Y;
        pr.ranks = s ? p.proj[i].ranks : pr.ranks;
        pr.scales = s ? p.proj[i].scales : pr.scales;
      } else if ((int)blockIdx.y == i) {
        pr = p.proj[i];
      }
    }
  }
  // A negative size or a null table is a malformed launch (the host rejects
  // both).  Testing every uniform argument here also makes the compiler fetch
  // them all in the first batch of loads instead of one round trip per
  // argument where it is first used.
  const bool bad_size = (p.num_units | p.splits | p.kc | p.cw | p.direct_units | p.split_major | p.n_rows |
                         p.h_in | p.h_out | p.num_segs | p.num_loras | p.unit_base | (p.round_units - 1) |
                         (int32_t)(p.slot_stride >> 32)) < 0;
  bool bad_ptr = (p.X == nullptr) | (p.slots == nullptr) | (pr.Y == nullptr) | (p.errors == nullptr);
  if constexpr (!INL)
    bad_ptr |= (p.seg_indptr == nullptr) | (p.lora_idx == nullptr) | (pr.A_ptrs == nullptr) |
               (pr.B_ptrs == nullptr);
  // The optional int32 / fp32 tables are 4-byte aligned (the rank and scale
  // tables are nullable).
  if constexpr (MAP) bad_ptr |= (reinterpret_cast<uintptr_t>(p.row_idx) & 3) != 0 || p.row_idx == nullptr;
  if constexpr (HET)
    bad_ptr |= ((reinterpret_cast<uintptr_t>(pr.ranks) | reinterpret_cast<uintptr_t>(pr.scales)) & 3) != 0;
  if (bad_size | bad_ptr) return;
  // Workgroups go round-robin over the XCDs.  This launch covers units
  // unit_base .. unit_base + round_units - 1 (one launch unless the units do
  // not all fit on the device at once; the host then launches passes).
  int unit, g;
  if (p.split_major) {
    unit = blockIdx.x / G;
    g = blockIdx.x - unit * G;
  } else {  // keep the splits of a unit on one XCD
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    unit = (slot / G) * kXcds + xcd;
    g = slot - (slot / G) * G;
  }
  unit += p.unit_base;
  // Workgroups past the last unit (the grid is padded to whole XCD rounds)
  // resolve a unit past every segment and exit after the metadata loads: an
  // exit before them would split the kernel-argument loads into serial rounds.
  if (unit >= p.num_units) unit = 0x3fffffff;
  // With at most 64 LoRAs, fetch both pointer tables (one entry per lane) in
  // parallel with the segment metadata instead of after it: the LoRA id then
  // selects its pointers from registers, saving one dependent memory trip.
  int rk_lane = R;
  float sk_lane = 1.f;
  if (SMALL && !INL && lane < p.num_loras) {
    a_lane = pr.A_ptrs[lane];
    b_lane = pr.B_ptrs[lane];
    if constexpr (HET) {
      if (pr.ranks) rk_lane = pr.ranks[lane];
      if (pr.scales) sk_lane = pr.scales[lane];
    }
  }
  Unit un;
  if constexpr (INL)  // the unit's k is its segment
    un = resolve_unit_lanes<RB>(lo_l, hi_l, p.num_segs, p.n_rows, p.direct_units, unit);
  else
    un = resolve_unit<RB>(p.seg_indptr, p.lora_idx, p.num_segs, p.num_loras, p.n_rows, p.direct_units, unit);
  if (un.L <= 0) return;  // uniform over the workgroup (and over the unit)
  const int L = un.L;
  const int r0 = un.r0;
  const uint32_t tag = launch_tag();

  const uint16_t* Ak;
  const uint16_t* Bk;
  int rk = R;      // rank of this unit's LoRA (row stride of A_k)
  float sk = 1.f;  // scale of its term
  if constexpr (INL) {
    Ak = reinterpret_cast<const uint16_t*>(readlane_u64(a_lane, un.k));
    Bk = reinterpret_cast<const uint16_t*>(readlane_u64(b_lane, un.k));
  } else if constexpr (SMALL) {
    Ak = reinterpret_cast<const uint16_t*>(readlane_u64(a_lane, un.k));
    Bk = reinterpret_cast<const uint16_t*>(readlane_u64(b_lane, un.k));
    if constexpr (HET) {
      rk = __builtin_amdgcn_readlane(rk_lane, un.k);
      sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sk_lane), un.k));
    }
  } else {
    Ak = reinterpret_cast<const uint16_t*>(pr.A_ptrs[un.k]);
    Bk = reinterpret_cast<const uint16_t*>(pr.B_ptrs[un.k]);
    if constexpr (HET) {
      if (pr.ranks) rk = pr.ranks[un.k];
      if (pr.scales) sk = pr.scales[un.k];
    }
  }
  if constexpr (HET) {
    rk = lora_rank<R>(rk);
    if (rk == 0) return;  // the LoRA adds nothing (uniform over the unit)
  }
  const int h0 = g * p.kc;
  const int h1 = p.h_in < h0 + p.kc ? p.h_in : h0 + p.kc;
  const int c0 = g * p.cw;
  const int c1 = p.h_out < c0 + p.cw ? p.h_out : c0 + p.cw;
  // Rows of X / Y.  With a row map, lane l looks up the row behind sorted row
  // r0 + l once, ahead of the streaming loads (L <= RB <= 64 rows), and every
  // other lane takes it from there.
  int prow = r0 + lane;
  if constexpr (MAP) prow = p.row_idx[r0 + (lane < L ? lane : L - 1)];
  const uint16_t* Xr = p.X + (int64_t)(MAP ? __builtin_amdgcn_readfirstlane(prow) : r0) * p.h_in;

  // ---------------- all loads, issued up front ----------------
  // Shrink: thread t owns ranks (t % JG)*8..+7 of rows h0 + t/JG + q*HS.
  // With a rank below R, A_k rows are rk wide and the lanes of ranks >= rk
  // load nothing new (their address is clamped) and compute nothing.
  const int jg = t % JG;
  const bool jg_ok = !HET || jg * 8 < rk;
  const int a_stride = HET ? rk : R;
  u32x4 av[NA];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    const int h = h0 + t / JG + q * HS;
    av[q] = load_stream(Ak + (h < h1 && jg_ok ? (int64_t)h * a_stride + jg * 8 : 0));
  }
  uint16_t xs[RB == 1 ? NA : 1];
  u32x4 xv[NXV];
  if constexpr (RB == 1) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int h = h0 + t / JG + q * HS;
      xs[q] = load_stream_u16(Xr + (h < h1 ? h : 0));
    }
  } else {
    const int xvr = (h1 - h0) / 8;  // 128-bit vectors per row of the chunk
#pragma unroll
    for (int q = 0; q < NXV; ++q) {
      const int x = t + kThreads * q;
      const int i = xvr > 0 ? x / xvr : 0, c = x - i * xvr;
      const int xi = x < L * xvr ? i : 0;
      const int64_t row = MAP ? __shfl(prow, xi) : r0 + xi;
      xv[q] = load_stream(p.X + row * p.h_in + (x < L * xvr ? h0 + c * 8 : 0));
    }
  }
  // Expand: thread t owns the 8 columns c0 + (t / JQ)*8 .. +7 and ranks
  // jq, jq + JQ, ... of B_k; lane jq also carries the Y rows i = jq + n*JQ.
  const int jq = t % JQ;
  const int col = c0 + (t / JQ) * 8;
  const bool col_ok = col < c1;
  u32x4 bv[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const bool ok = col_ok && (!HET || jq + JQ * m < rk);  // rows of B_k past rk do not exist
    bv[m] = load_stream(Bk + (ok ? (int64_t)(jq + JQ * m) * p.h_out + col : 0));
  }
  u32x4 yv[NY];
  int yrow[NY];  // row of Y of the rows i = jq + n*JQ (kept for the stores)
#pragma unroll
  for (int n = 0; n < NY; ++n) {
    const int i = jq + JQ * n;
    const int yi = col_ok && i < L ? i : 0;
    yrow[n] = MAP ? __shfl(prow, yi) : r0 + yi;
    yv[n] = load_stream(pr.Y + (int64_t)yrow[n] * p.h_out + (col_ok && i < L ? col : 0));
  }

  // ---------------- shrink ----------------
  float acc[RB][8];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  if constexpr (RB > 1) {
    const int xvr = (h1 - h0) / 8;
#pragma unroll
    for (int q = 0; q < NXV; ++q) {
      const int x = t + kThreads * q;
      if (x < L * xvr) {
        const int i = x / xvr, c = x - i * xvr;
        store_vec(&lds_x[i * KCMAX + c * 8], xv[q]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    const int hl = t / JG + q * HS;  // row inside the chunk
    if (h0 + hl < h1 && jg_ok) {
      float af[8];
      unpack8<T>(av[q], af);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (i < L) {
          const float xf = RB == 1 ? T::one(xs[q]) : T::one(lds_x[i * KCMAX + hl]);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][e] = __builtin_fmaf(xf, af[e], acc[i][e]);
        }
      }
    }
  }
  // Reduce each row's partial ranks over the lanes that share them (lane bits
  // B0..5); afterwards lane l < R of every wave holds rank
  // (l % JG)*8 + e(l) of the wave's partial.
  const int j_of_lane = (lane & (JG - 1)) * 8 + ((lane >> B0) & 1) * 4 + ((lane >> (B0 + 1)) & 1) * 2 +
                        ((lane >> (B0 + 2)) & 1);
  const bool rank_lane = (lane >> (B0 + 3)) == 0;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (i < L) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = acc[i][e];
      halve<4>(v, lane, 1 << B0);
      halve<2>(v, lane, 1 << (B0 + 1));
      halve<1>(v, lane, 1 << (B0 + 2));
#pragma unroll
      for (int b = B0 + 3; b < 6; ++b) v[0] += shfl_xor(v[0], 1 << b);
      acc[i][0] = v[0];
    }
  }

  // ---------------- publish ----------------
  // Per-unit slot layout: [G][PW][RB*R] tagged words.
  uint64_t* unit_slots = p.slots + (int64_t)blockIdx.y * p.slot_stride + (int64_t)unit * G * PW * (RB * R);
  // The waves' partials are summed in LDS first: one word per output leaves
  // the workgroup, which keeps the device-scope exchange small.
  {
#pragma unroll
    for (int i = 0; i < RB; ++i)
      if (i < L && rank_lane) lds_red[(wave * RB + i) * R + j_of_lane] = acc[i][0];
    if (t == 0) lds_gave_up = 0;
    __syncthreads();
    if (t < L * R) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += lds_red[w * RB * R + t];
      publish_tagged(unit_slots + (int64_t)g * (RB * R) + t, s, tag);
    }
  }

  // ---------------- gather: wait for every split of the unit ----------------
  const int n_out = L * R;                    // outputs of V for this unit
  const int parts = G * PW;                   // partials per output
  const int per_round = kStage / n_out;       // partials staged per round (>= 1)
  float vsum = 0.f;
  // The wait ends at a deadline on the constant-rate real-time counter, read
  // right after each round of polls is issued so that its latency overlaps
  // theirs.  A limit of 0 (the host's test hook) waits for a tag no partial
  // carries, so every workgroup gives up after one round of polls.
  const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + p.wait_ticks;
  const uint32_t want = p.wait_ticks != 0 ? tag : ~tag;
  for (int p0 = 0; p0 < parts; p0 += per_round) {
    const int pn = parts - p0 < per_round ? parts - p0 : per_round;
    const int items = pn * n_out;
    uint64_t w[kPollPerThread];
    const uint64_t* src[kPollPerThread];
#pragma unroll
    for (int m = 0; m < kPollPerThread; ++m) {
      const int it = t + kThreads * m;
      const int pp = it / n_out, o = it - pp * n_out;
      src[m] = unit_slots + (it < items ? (int64_t)(p0 + pp) * (RB * R) + o : 0);
      // Only lanes with an item load (device-scope loads are the exchange's
      // cost); the others are never examined.
      w[m] = it < items ? fetch_tagged(src[m]) : 0;
    }
    bool done;
    uint64_t now = 0;  // read beside each round of polls, checked at the next
    for (;;) {
      done = true;
#pragma unroll
      for (int m = 0; m < kPollPerThread; ++m)
        if (t + kThreads * m < items && (uint32_t)(w[m] >> 32) != want) done = false;
      if (done || now > deadline) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int m = 0; m < kPollPerThread; ++m)
        if (t + kThreads * m < items && (uint32_t)(w[m] >> 32) != want) w[m] = fetch_tagged(src[m]);
      now = __builtin_amdgcn_s_memrealtime();
    }
#pragma unroll
    for (int m = 0; m < kPollPerThread; ++m) {
      const int it = t + kThreads * m;
      if (it < items) lds_stage[it] = __uint_as_float((uint32_t)w[m]);
    }
    if (!done) lds_gave_up = 1;
    __syncthreads();
    if (t < n_out)
      for (int pp = 0; pp < pn; ++pp) vsum += lds_stage[pp * n_out + t];
    const bool quit = lds_gave_up != 0;  // read beside the partials, tested after the barrier
    __syncthreads();
    // Every thread of the workgroup leaves together when any thread gave up.
    if (quit) {
      if (t == 0) __hip_atomic_fetch_or(p.errors, kDecodeErrWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  if (t < n_out) lds_v[t] = HET ? vsum * sk : vsum;
  __syncthreads();

  // ---------------- expand ----------------
  float bf[NB][8];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    unpack8<T>(bv[m], bf[m]);
    if (HET && jq + JQ * m >= rk)
#pragma unroll
      for (int e = 0; e < 8; ++e) bf[m][e] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (i < L) {
      float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        const float vj = lds_v[i * R + jq + JQ * m];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = __builtin_fmaf(vj, bf[m][e], s[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[e] += quad_xor1(s[e]);
        s[e] += quad_xor2(s[e]);
      }
      if (col_ok && jq == i % JQ) {
        float yf[8];
        unpack8<T>(yv[i / JQ], yf);
#pragma unroll
        for (int e = 0; e < 8; ++e) yf[e] += s[e];
        store_vec(pr.Y + (int64_t)yrow[i / JQ] * p.h_out + col, pack8<T>(yf));
      }
    }
  }
}

template <class T, int R, int RB, bool SMALL, bool MAP, bool HET>
__global__ __launch_bounds__(kThreads) void sgmv_decode_kernel(DecodeParams p) {
  decode_body<T, R, RB, SMALL, MAP, HET, false>(p, nullptr);
}

// One projection, no row map, no rank or scale tables; the metadata in m.
template <class T, int R, int RB>
__global__ __launch_bounds__(kThreads) void sgmv_decode_inline_kernel(DecodeParams p, InlineMeta m) {
  decode_body<T, R, RB, false, false, false, true>(p, &m);
}

template <class T, int R, int RB>
hipError_t launch_t(const DecodeParams& p, int num_proj, hipStream_t stream) {
  const unsigned grid = (unsigned)p.round_units * (unsigned)p.splits;
  if (grid == 0 || num_proj <= 0) return hipSuccess;
  const bool small = p.num_loras <= 64;
  const bool map = p.row_idx != nullptr;
  bool het = false;
  for (int i = 0; i < num_proj; ++i) het = het || p.proj[i].ranks || p.proj[i].scales;
  using K = void (*)(DecodeParams);
  // [small][map][het]
  static constexpr K kernels[2][2][2] = {
      {{sgmv_decode_kernel<T, R, RB, false, false, false>, sgmv_decode_kernel<T, R, RB, false, false, true>},
       {sgmv_decode_kernel<T, R, RB, false, true, false>, sgmv_decode_kernel<T, R, RB, false, true, true>}},
      {{sgmv_decode_kernel<T, R, RB, true, false, false>, sgmv_decode_kernel<T, R, RB, true, false, true>},
       {sgmv_decode_kernel<T, R, RB, true, true, false>, sgmv_decode_kernel<T, R, RB, true, true, true>}}};
  const K kernel = kernels[small][map][het];
  hipLaunchKernelGGL(kernel, dim3(grid, num_proj), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <class T, int R, int RB, bool SMALL, bool MAP, bool HET>
int per_cu_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&sgmv_decode_kernel<T, R, RB, SMALL, MAP, HET>), kThreads, 0) !=
      hipSuccess)
    return 0;
  return n;
}

template <class T, int R, int RB>
int per_cu_inline_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&sgmv_decode_inline_kernel<T, R, RB>), kThreads, 0) != hipSuccess)
    return 0;
  return n;
}

// Workgroups of one variant that fit on the device at once.  `variant` holds
// the pointer-pool, row-map and rank/scale flags as bits 0, 1, 2, or is
// kDecodeInlineVariant for the kernel with the metadata in its arguments.
template <class T, int R, int RB>
int capacity_t(int variant) {
  using F = int (*)();
  static constexpr F per_cu[9] = {
      per_cu_t<T, R, RB, false, false, false>, per_cu_t<T, R, RB, true, false, false>,
      per_cu_t<T, R, RB, false, true, false>,  per_cu_t<T, R, RB, true, true, false>,
      per_cu_t<T, R, RB, false, false, true>,  per_cu_t<T, R, RB, true, false, true>,
      per_cu_t<T, R, RB, false, true, true>,   per_cu_t<T, R, RB, true, true, true>,
      per_cu_inline_t<T, R, RB>};
  int dev = 0, cus = 0;
  if (variant < 0 || variant > kDecodeInlineVariant) return 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return per_cu[variant]() * cus;
}

// Instantiated (rank, rows per unit) pairs: rank * RB <= 256.
template <class T, int R, int RB>
hipError_t launch_inline_t(const DecodeParams& p, const InlineMeta& m, hipStream_t stream) {
  const unsigned grid = (unsigned)p.round_units * (unsigned)p.splits;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((sgmv_decode_inline_kernel<T, R, RB>), dim3(grid, 1), dim3(kThreads), 0, stream, p, m);
  return hipGetLastError();
}

// m: launch the kernel with the metadata in its arguments (one projection).
template <class T>
hipError_t dispatch(int rank, int rb, const DecodeParams& p, int num_proj, hipStream_t s, int* cap,
                    int variant, const InlineMeta* m = nullptr) {
#define SGMV_DECODE_CASE(R_, RB_)                          \
  if (rank == R_ && rb == RB_) {                           \
    if (cap) {                                             \
      *cap = capacity_t<T, R_, RB_>(variant);              \
      return hipSuccess;                                   \
    }                                                      \
    if (m) return launch_inline_t<T, R_, RB_>(p, *m, s);   \
    return launch_t<T, R_, RB_>(p, num_proj, s);           \
  }
  SGMV_DECODE_CASE(8, 1) SGMV_DECODE_CASE(8, 4) SGMV_DECODE_CASE(8, 16)
  SGMV_DECODE_CASE(16, 1) SGMV_DECODE_CASE(16, 4) SGMV_DECODE_CASE(16, 16)
  SGMV_DECODE_CASE(32, 1) SGMV_DECODE_CASE(32, 4)
  SGMV_DECODE_CASE(64, 1) SGMV_DECODE_CASE(64, 4)
#undef SGMV_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t decode_error_word(uint32_t** word) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint32_t* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(decode_errors));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<uint32_t*>(ptr);
  }
  *word = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(int dtype, int rank, int rb, const DecodeParams& p, int num_proj, hipStream_t stream) {
  return dtype == 1 ? dispatch<BF16>(rank, rb, p, num_proj, stream, nullptr, 0)
                    : dispatch<F16>(rank, rb, p, num_proj, stream, nullptr, 0);
}

hipError_t launch_decode_inline(int dtype, int rank, int rb, const DecodeParams& p, const InlineMeta& m,
                                hipStream_t stream) {
  return dtype == 1 ? dispatch<BF16>(rank, rb, p, 1, stream, nullptr, 0, &m)
                    : dispatch<F16>(rank, rb, p, 1, stream, nullptr, 0, &m);
}

int decode_resident_capacity(int dtype, int rank, int rb, int variant) {
  int cap = 0;
  if (dtype == 1)
    (void)dispatch<BF16>(rank, rb, DecodeParams{}, 0, nullptr, &cap, variant);
  else
    (void)dispatch<F16>(rank, rb, DecodeParams{}, 0, nullptr, &cap, variant);
  return cap;
}

}  // namespace sgmv
