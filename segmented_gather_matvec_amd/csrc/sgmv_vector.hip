// sgmv_vector.hip - split-K vector kernels for decode-shaped SGMV (gfx950).
//
// The LoRA term of the Punica README (page "Punica：多 LoRA 模型统一服务框架",
// LoRA and multi-LoRA paragraphs) for short segments is two tall-skinny
// products per segment, V = X_seg @ A_k ([L, H1] x [H1, r]) and
// Y_seg += V @ B_k ([L, r] x [r, H2]), with L a handful of rows.  At that shape
// each weight byte feeds L multiply-adds, far below the ALU/HBM ridge, so the
// kernels are built around HBM streaming: every A_k and B_k byte is read once
// with 128-bit loads spread over many workgroups, and the arithmetic is plain
// fp32 FMA (no matrix cores).
//
// Work split: a "unit" is one row block (<= RB rows) of one segment; `splits`
// workgroups share a unit.  Split g reads input rows [g*kc, (g+1)*kc) of A_k
// (shrink) and output columns [g*cw, (g+1)*cw) of B_k (expand).  Shrink
// partial sums are reduced in registers (halving exchange across lanes), then
// across the four waves in LDS, then across splits in a fixed order, so the
// result is bitwise reproducible.
//
// Modes: kModeShrink writes V (the last workgroup of a unit to arrive sums the
// split partials), kModeExpand reads V.  These serve sgmv_shrink, sgmv_expand
// and the two-launch form of sgmv_lora_apply for any segment length.
#include "sgmv_device.h"
#include "sgmv_plan.h"
#include "sgmv_units.h"

namespace sgmv {
namespace {

constexpr int kNA = 2;  // 128-bit A loads per thread per shrink pass
constexpr int kNB = 2;  // 128-bit B loads per thread per expand pass

template <int R>
constexpr int log2_groups() {
  return R == 8 ? 0 : R == 16 ? 1 : R == 32 ? 2 : 3;
}

// One halving exchange: lanes whose `mask` bit is set keep the upper H of
// their 2H values, the others keep the lower H; each adds its partner's copy.
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

// Sum the published split partials of one unit, [G][RB*R] at `base`, over
// the splits in ascending order into dst[o] for o < n (n = L*R).  All
// partials are fetched at once (each thread a slice, into LDS), so the fetch
// costs one round trip to the device-coherent level, not one per split.
template <int RB, int R>
__device__ inline void gather_partials(const float* base, int G, int n, float* stage, int stage_len,
                                       float* dst) {
  constexpr int kPF = 8;  // fetches per thread per round
  const int t = threadIdx.x;
  const int per_round = stage_len / n;  // splits fetched per round (>= 1)
  float acc = 0.f;
  for (int g0 = 0; g0 < G; g0 += per_round) {
    const int gn = G - g0 < per_round ? G - g0 : per_round;
    const int items = gn * n;
    float v[kPF];
#pragma unroll
    for (int m = 0; m < kPF; ++m) {
      const int it = t + kThreads * m;
      const int gg = it / n, o = it - gg * n;
      const bool ok = it < items;
      v[m] = fetch_published_f32(base + (ok ? (int64_t)(g0 + gg) * (RB * R) + o : 0));
    }
#pragma unroll
    for (int m = 0; m < kPF; ++m) {
      const int it = t + kThreads * m;
      if (it < items) stage[it] = v[m];
    }
    __syncthreads();
    if (t < n)
      for (int gg = 0; gg < gn; ++gg) acc += stage[gg * n + t];
    __syncthreads();
  }
  if (t < n) dst[t] = acc;
}

// EXT: the extended arguments may be set (row map, per-LoRA ranks and scales;
// see the decode kernel).  Without EXT the kernel carries none of it.
template <class T, int R, int RB, int MODE, bool EXT>
__global__ __launch_bounds__(kThreads) void sgmv_vec_kernel(VecParams p) {
  constexpr int JG = R / 8;                 // 128-bit vectors per row of A_k
  constexpr int B0 = log2_groups<R>();
  constexpr int HP = vec_rows_per_pass(R);  // A_k rows per shrink pass
  constexpr int CP = vec_cols_per_pass(R);  // B_k columns per expand pass
  constexpr bool kShrink = MODE != kModeExpand;
  constexpr bool kExpand = MODE != kModeShrink;
  constexpr int NXV = (RB * HP / 8 + kThreads - 1) / kThreads;  // X vectors / thread / pass
  constexpr int NYV = (RB * CP / 8 + kThreads - 1) / kThreads;  // Y vectors / thread / pass
  constexpr int kStage = kThreads * 8;                          // floats staged per partial round

  __shared__ __attribute__((aligned(16))) uint16_t lds_x[kShrink ? RB * HP : 8];
  __shared__ float lds_red[kShrink ? kWaves * RB * R : 1];
  __shared__ float lds_v[RB * R];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[kExpand ? R * CP : 8];
  // Expand output partials; the shrink reuses it to stage split partials.
  __shared__ __attribute__((aligned(16))) float lds_out[kStage];
  __shared__ int lds_flag;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int G = p.splits;
  const int unit = blockIdx.x / G;
  const int g = blockIdx.x - unit * G;
  const Unit un = resolve_unit<RB>(p.seg_indptr, p.lora_idx, p.num_segs, p.num_loras, p.n_rows,
                                    p.direct_units, unit);
  if (un.L <= 0) return;  // uniform over the workgroup
  const int L = un.L;
  const int r0 = un.r0;
  // Rank of the LoRA (A_k rows and B_k's row count; ranks >= rk are zero) and
  // the scale of its term.
  int rk = R;
  float sk = 1.f;
  if constexpr (EXT) {
    if (p.ranks) rk = lora_rank<R>(p.ranks[un.k]);
    if (p.scales) sk = p.scales[un.k];
    if (rk == 0) return;  // nothing to add: every split of the unit leaves here
  }
  auto row_of = [&](int j) -> int64_t { return EXT && p.row_idx ? (int64_t)p.row_idx[j] : (int64_t)j; };

  // ---- expand operands: B_k columns [c0, c1), Y rows [r0, r0+L) ----
  // Every thread issues the same number of loads in every pass (addresses of
  // lanes without work are clamped to a valid element and their data unused),
  // so the compiler can wait for exactly the loads a pass needs while later
  // passes stay in flight.
  const uint16_t* Bk = nullptr;
  int c0 = 0, c1 = 0;
  if constexpr (kExpand) {
    Bk = reinterpret_cast<const uint16_t*>(p.B_ptrs[un.k]);
    c0 = g * p.cw;
    c1 = p.h_out < c0 + p.cw ? p.h_out : c0 + p.cw;
  }
  auto issue_expand = [&](int cp0, u32x4 (&bv)[kNB], u32x4 (&yv)[NYV]) {
    const int left = c1 - cp0;
    const int cvr = (left < CP ? (left > 0 ? left : 0) : CP) / 8;
#pragma unroll
    for (int q = 0; q < kNB; ++q) {
      const int v = t + kThreads * q;
      const int j = cvr ? v / cvr : 0, cv = v - j * cvr;
      const bool ok = v < R * cvr && (!EXT || j < rk);
      bv[q] = load_stream(Bk + (ok ? (int64_t)j * p.h_out + cp0 + cv * 8 : 0));
    }
#pragma unroll
    for (int q = 0; q < NYV; ++q) {
      const int y = t + kThreads * q;
      const int i = cvr ? y / cvr : 0, cv = y - i * cvr;
      const bool ok = y < L * cvr;
      yv[q] = load_stream(p.Y + row_of(r0 + (ok ? i : 0)) * p.h_out + (ok ? cp0 + cv * 8 : 0));
    }
  };
  auto compute_expand = [&](int cp0, const u32x4 (&bv)[kNB], const u32x4 (&yv)[NYV]) {
    const int cvr = (c1 - cp0 < CP ? c1 - cp0 : CP) / 8;
    __syncthreads();  // lds_v ready / the previous pass is done with lds_b, lds_out
#pragma unroll
    for (int q = 0; q < kNB; ++q) {
      const int v = t + kThreads * q;
      if (v < R * cvr) {
        const int j = v / cvr, cv = v - j * cvr;
        const u32x4 z = {0u, 0u, 0u, 0u};
        store_vec(&lds_b[j * CP + cv * 8], !EXT || j < rk ? bv[q] : z);
      }
    }
    __syncthreads();
    const int OV = L * cvr;  // output vectors (8 columns of one row) in this pass
    int JQ = 1;              // threads sharing one output vector, each with R/JQ ranks
    while (JQ < R && OV * JQ * 2 <= kThreads) JQ *= 2;
    if (JQ > 1) {
      if (t < OV * JQ) {
        const int ov = t % OV, jq = t / OV;
        const int i = ov / cvr, cv = ov - i * cvr;
        const int jn = R / JQ;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = jq * jn; j < (jq + 1) * jn; ++j) {
          float bf[8];
          unpack8<T>(load_vec(&lds_b[j * CP + cv * 8]), bf);
          const float vj = lds_v[i * R + j];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(vj, bf[e], acc[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) lds_out[(jq * OV + ov) * 8 + e] = acc[e];
      }
      __syncthreads();
      if (t < OV) {
        const int i = t / cvr, cv = t - i * cvr;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int jq = 0; jq < JQ; ++jq)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += lds_out[(jq * OV + t) * 8 + e];
        float yf[8];
        unpack8<T>(yv[0], yf);
#pragma unroll
        for (int e = 0; e < 8; ++e) yf[e] += acc[e];
        store_vec(p.Y + row_of(r0 + i) * p.h_out + cp0 + cv * 8, pack8<T>(yf));
      }
    } else {
#pragma unroll
      for (int q = 0; q < NYV; ++q) {
        const int ov = t + kThreads * q;
        if (ov < OV) {
          const int i = ov / cvr, cv = ov - i * cvr;
          float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
          for (int j = 0; j < R; ++j) {
            float bf[8];
            unpack8<T>(load_vec(&lds_b[j * CP + cv * 8]), bf);
            const float vj = lds_v[i * R + j];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(vj, bf[e], acc[e]);
          }
          float yf[8];
          unpack8<T>(yv[q], yf);
#pragma unroll
          for (int e = 0; e < 8; ++e) yf[e] += acc[e];
          store_vec(p.Y + row_of(r0 + i) * p.h_out + cp0 + cv * 8, pack8<T>(yf));
        }
      }
    }
  };
  u32x4 bv0[kNB], yv0[NYV], bv1[kNB], yv1[NYV];

  if constexpr (kShrink) {
    const uint16_t* Ak = reinterpret_cast<const uint16_t*>(p.A_ptrs[un.k]);
    const int h0 = g * p.kc;
    const int h1 = p.h_in < h0 + p.kc ? p.h_in : h0 + p.kc;
    auto issue_shrink = [&](int hp0, u32x4 (&av)[kNA], u32x4 (&xv)[NXV]) {
      const int left = h1 - hp0;
      const int hpn = left < HP ? (left > 0 ? left : 0) : HP;  // multiple of 8
      const int xvr = hpn / 8;                                  // X vectors per row in this pass
#pragma unroll
      for (int q = 0; q < kNA; ++q) {
        const int v = t + kThreads * q;
        // Vector v holds ranks (v % JG)*8 .. +7 of row hp0 + v / JG.
        const bool ok = v < hpn * JG && (!EXT || (v % JG) * 8 < rk);
        av[q] = load_stream(Ak + (ok ? (int64_t)(hp0 + v / JG) * (EXT ? rk : R) + (v % JG) * 8 : 0));
      }
#pragma unroll
      for (int q = 0; q < NXV; ++q) {
        const int x = t + kThreads * q;
        const int i = xvr ? x / xvr : 0, c = x - i * xvr;
        const bool ok = x < L * xvr;
        xv[q] = load_stream(p.X + row_of(r0 + (ok ? i : 0)) * p.h_in + (ok ? hp0 + c * 8 : 0));
      }
    };
    float acc[RB][8];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    auto compute_shrink = [&](int hp0, const u32x4 (&av)[kNA], const u32x4 (&xv)[NXV]) {
      const int hpn = h1 - hp0 < HP ? h1 - hp0 : HP;
      const int xvr = hpn / 8;
      __syncthreads();  // the previous pass is done with lds_x
#pragma unroll
      for (int q = 0; q < NXV; ++q) {
        const int x = t + kThreads * q;
        if (x < L * xvr) {
          const int i = x / xvr, c = x - i * xvr;
          store_vec(&lds_x[i * HP + c * 8], xv[q]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kNA; ++q) {
        const int v = t + kThreads * q;
        if (v < hpn * JG && (!EXT || (v % JG) * 8 < rk)) {
          const int hl = v / JG;  // row of A_k inside the pass; ranks (t % JG)*8 .. +7
          float af[8];
          unpack8<T>(av[q], af);
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            if (i < L) {
              const float xf = T::one(lds_x[i * HP + hl]);
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[i][e] = __builtin_fmaf(xf, af[e], acc[i][e]);
            }
          }
        }
      }
    };

    // Ping-pong over passes: pass p+1 is in flight while pass p is computed.
    u32x4 av0[kNA], xv0[NXV], av1[kNA], xv1[NXV];
    issue_shrink(h0, av0, xv0);
    for (int hp0 = h0; hp0 < h1; hp0 += 2 * HP) {
      issue_shrink(hp0 + HP, av1, xv1);
      compute_shrink(hp0, av0, xv0);
      issue_shrink(hp0 + 2 * HP, av0, xv0);
      if (hp0 + HP < h1) compute_shrink(hp0 + HP, av1, xv1);
    }

    // Reduce each row's 8 partial ranks over the lanes that share them
    // (lane bits B0..5), then over the waves through LDS.
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
        if ((lane >> (B0 + 3)) == 0) {
          const int jg = lane & (JG - 1);
          const int e = ((lane >> B0) & 1) * 4 + ((lane >> (B0 + 1)) & 1) * 2 + ((lane >> (B0 + 2)) & 1);
          lds_red[(wave * RB + i) * R + jg * 8 + e] = v[0];
        }
      }
    }
    __syncthreads();

    if (MODE == kModeShrink && G == 1) {
      for (int o = t; o < L * R; o += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += lds_red[w * RB * R + o];
        p.V[(int64_t)(r0 + o / R) * R + (o % R)] = EXT ? s * sk : s;
      }
      return;
    }
    // Publish this split's partial sums, then count the arrival.
    float* part = p.partials + ((int64_t)unit * G + g) * (RB * R);
    for (int o = t; o < L * R; o += kThreads) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += lds_red[w * RB * R + o];
      publish_f32(&part[o], s);
    }
    wait_memory_ops();
    __syncthreads();
    uint32_t* arrive = p.counters + unit;
    const float* base = p.partials + (int64_t)unit * G * (RB * R);
    // The last split to arrive sums all partials (in split order) into V.
    if (t == 0) lds_flag = counter_add(arrive, 1u) == (uint32_t)(G - 1);
    __syncthreads();
    if (!lds_flag) return;
    for (int o0 = 0; o0 < L * R; o0 += kThreads) {
      const int n = L * R - o0 < kThreads ? L * R - o0 : kThreads;
      gather_partials<RB, R>(base + o0, G, n, lds_out, kStage, lds_v);
      __syncthreads();
      if (t < n) p.V[(int64_t)(r0 + (o0 + t) / R) * R + ((o0 + t) % R)] = EXT ? lds_v[t] * sk : lds_v[t];
      __syncthreads();
    }
    if (t == 0) counter_store(arrive, 0u);
    return;
  }

  if constexpr (kExpand) {
    for (int o = t; o < L * R; o += kThreads) lds_v[o] = p.V[(int64_t)(r0 + o / R) * R + (o % R)];
    issue_expand(c0, bv0, yv0);
    for (int cp0 = c0; cp0 < c1; cp0 += 2 * CP) {
      issue_expand(cp0 + CP, bv1, yv1);
      compute_expand(cp0, bv0, yv0);
      issue_expand(cp0 + 2 * CP, bv0, yv0);
      if (cp0 + CP < c1) compute_expand(cp0 + CP, bv1, yv1);
    }
  }
}

template <class T, int R, int RB, int MODE>
hipError_t launch_one(const VecParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.num_units * (unsigned)p.splits;
  if (grid == 0) return hipSuccess;
  if (p.row_idx || p.ranks || p.scales)
    hipLaunchKernelGGL((sgmv_vec_kernel<T, R, RB, MODE, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((sgmv_vec_kernel<T, R, RB, MODE, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <class T, int R, int RB>
hipError_t launch_mode(int mode, const VecParams& p, hipStream_t s) {
  switch (mode) {
    case kModeShrink: return launch_one<T, R, RB, kModeShrink>(p, s);
    case kModeExpand: return launch_one<T, R, RB, kModeExpand>(p, s);
  }
  return hipErrorInvalidValue;
}

template <class T, int R>
hipError_t launch_rb(int rb, int mode, const VecParams& p, hipStream_t s) {
  switch (rb) {
    case 1: return launch_mode<T, R, 1>(mode, p, s);
    case 4: return launch_mode<T, R, 4>(mode, p, s);
    case 16: return launch_mode<T, R, 16>(mode, p, s);
  }
  return hipErrorInvalidValue;
}

template <class T>
hipError_t launch_rank(int rank, int rb, int mode, const VecParams& p, hipStream_t s) {
  switch (rank) {
    case 8: return launch_rb<T, 8>(rb, mode, p, s);
    case 16: return launch_rb<T, 16>(rb, mode, p, s);
    case 32: return launch_rb<T, 32>(rb, mode, p, s);
    case 64: return launch_rb<T, 64>(rb, mode, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_vec(int dtype, int rank, int rb, int mode, const VecParams& p, hipStream_t stream) {
  return dtype == 1 ? launch_rank<BF16>(rank, rb, mode, p, stream)
                    : launch_rank<F16>(rank, rb, mode, p, stream);
}

namespace {
__global__ __launch_bounds__(kThreads) void clear_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t launch_clear_u32(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(clear_u32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace sgmv
