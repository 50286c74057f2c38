// sgmv_mfma.hip - matrix-core SGMV kernels for long (prefill) segments (gfx950).
//
// For a segment of L rows the LoRA term of the Punica README (page "Punica：多
// LoRA 模型统一服务框架", LoRA and multi-LoRA paragraphs) is two skinny GEMMs,
// V = X_seg @ A_k ([L, H1] x [H1, r]) and Y_seg += V @ B_k ([L, r] x [r, H2]).
// Each weight byte is reused by L rows; at L in the hundreds and r = 64 the
// arithmetic intensity (up to ~60 flop/B) is above what plain fp32 FMA can
// sustain against HBM, so both run on v_mfma_f32_16x16x32_{f16,bf16}
// (lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], D[4(l/16)+i][l%16]).
//
// Two launches (three for the standalone shrink, whose reduce writes V):
//  1. shrink: a workgroup (4 waves, 16 rows each) takes up to 64 rows of one
//     segment and one chunk of H1, streamed in stages of 128 H1 rows that are
//     pipelined two deep: the X rows and A_k rows of the next stage are in
//     flight (registers) while the current one is multiplied.  Both are
//     staged in LDS: X as loaded (whole rows per load instruction), A_k
//     transposed to [r][h] so that a lane reads the 8 consecutive h of one
//     rank with one 128-bit LDS read.  Each H1 chunk writes its own fp32 partial plane of V; workgroups
//     that read the same chunk of A_k run on one XCD.
//  2. V = sum of the partial planes, in chunk order (reproducible); the
//     LoRA's scale, if any, is applied to V by the expand.  With more than one
//     plane the expand launch begins with lead workgroups that sum them for
//     blocks of rows and publish V as words {fp32, launch tag}
//     (16-row expand tiles), or write V and flag each row block with the
//     launch's tag (larger tiles); the expand workgroups issue their first
//     loads, then poll the words or flags of their rows.  With one plane the
//     expand reads it as V.  The separate reduce launch serves the standalone
//     shrink.
//  3. expand: a workgroup takes 64 rows (16 when the segments are short) and a
//     group of 128-column chunks.  V is split into V_hi + V_lo (both in the
//     input format), consumed as a K of 2r against [B_k; B_k], which keeps
//     about twice the format's significand bits of V; its MFMA fragments stay
//     in registers for all chunks.  Each
//     chunk of B_k is staged transposed ([c][j]) in LDS while the next chunk's
//     B_k and Y are in flight; the result tile goes through LDS so that Y is
//     read and written with 128-bit accesses.
#include "sgmv_device.h"
#include "sgmv_mfma_ops.h"
#include "sgmv_plan.h"
#include "sgmv_units.h"

namespace sgmv {
namespace {

constexpr int kMT = kMfmaRowsPerTile;        // 64 rows per subtile: 16 per wave
constexpr int kCW = kMfmaColsPerTile;        // 128 output columns per expand chunk

constexpr int kXcds = 8;

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b on XCD
// b % 8), each with its own L2.  Give every XCD a contiguous run of the linear
// work order (grid = 8 * per_xcd), so that items adjacent in that order, which
// read the same weight slice, run on one XCD and share its L2.
// The first `skip` workgroups (a multiple of 8) are left out of the order.
__device__ inline int xcd_linear_index(int skip = 0) {
  const int per_xcd = (gridDim.x - skip) / kXcds;
  const int b = blockIdx.x - skip;
  return (b % kXcds) * per_xcd + b / kXcds;
}


// ---------------------------------------------------------------- shrink
// H1 rows per pipeline stage: while one stage's X fragments and A_k rows are
// multiplied, the next stage's loads are in flight.
constexpr int kKStage = 128;

// EXT: the extended arguments may be set (row map, per-LoRA ranks and scales;
// see the decode kernel).  Without EXT the kernel carries none of it.
// XL: X goes through LDS (below); else straight into the MFMA operand
// registers, which costs each stage less latency and suits short row tiles.
template <class T, int R, bool EXT, bool XL>
__global__ __launch_bounds__(kThreads) void sgmv_mfma_shrink_kernel(MfmaParams p) {
  constexpr int NT = R / 16;                // 16-wide rank tiles
  constexpr int JG = R / 8;                 // 128-bit vectors per row of A_k
  constexpr int PAIRS = kKStage / 2 * JG;   // (h, h+1) vector pairs of A_k per stage
  constexpr int NPAIR = (PAIRS + kThreads - 1) / kThreads;
  constexpr int MS = kKStage / 32;          // MFMA k-steps per stage
  // LDS row stride (halves) of transposed A_k: 72 dwords, which the 16 rank
  // rows of one 128-bit MFMA operand read cover without bank conflicts (a
  // stride of 68 dwords costs a second pass).
  constexpr int AST = kKStage + 16;
  // Within a rank row, the stage's h sit in groups of 8 (one 128-bit MFMA
  // operand read); group g of rank row r is stored at group g ^ swz(r).  The
  // xor changes every 4 rank rows, which the operand reads take without
  // conflicts, and it spreads the transposed stores of each half-wave (the
  // pair map below) over all banks.
  auto swz = [](int r) { return (r >> 2) & (kKStage / 8 - 1); };
  // (h-pair, rank group) item pr of a stage -> its h pair hp and its rank
  // group jg.  Each half-wave's 32 items are 4 rank groups x 8 h pairs
  // (r = 64, 32), or one rank group x 32 h pairs (r = 16): with the xor above
  // the transposed stores of a half-wave then meet every LDS bank once, and a
  // wave's loads still read whole rows of A_k.
  auto pair_of = [](int pr, int& hp, int& jg) {
    if constexpr (R == 64) {
      jg = (pr & 3) | (((pr >> 5) & 1) << 2);
      hp = ((pr >> 2) & 7) | ((pr >> 6) << 3);
    } else if constexpr (R == 32) {
      jg = pr & 3;
      hp = pr >> 2;
    } else {
      jg = (pr >> 5) & 1;
      hp = (pr & 31) | ((pr >> 6) << 5);
    }
  };
  static_assert(kMfmaKChunk % (2 * kKStage) == 0, "H1 chunks hold whole stage pairs");
  // XL: the X tile of a stage (64 rows x kKStage h, 128-bit vectors) is loaded
  // with whole rows per instruction (4 rows x 256 contiguous bytes), then
  // staged in LDS for the MFMA A operand, whose own layout (16 rows x 64 bytes
  // per instruction) asks L2 twice for every 128-byte line: streamed that way,
  // X arrives at about 3.2 TB/s.  Row stride 72 dwords: the operand reads
  // (16 rows x 4 k-groups) meet no bank twice.
  constexpr int XV = kKStage / 8;                  // 128-bit vectors per X row of a stage
  constexpr int NXV = XL ? kMT * XV / kThreads : MS;  // X vectors per thread and stage
  constexpr int XST = kKStage + 16;
  static_assert(!XL || NXV * kThreads == kMT * XV, "whole X tiles per stage");
  __shared__ __attribute__((aligned(16))) uint16_t lds_at[R * AST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[XL ? kMT * XST : 8];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int q = lane >> 4;   // k-group of the lane (8 k each)
  const int ml = lane & 15;  // row (A operand) / rank column (B operand) of the lane
  // Linear order: H1 chunk major, so the row units that read one chunk of A_k
  // share an XCD.
  const Projection pj = p.proj[blockIdx.y];
  // A negative size or a null table is a malformed launch (the host rejects
  // both).  Testing every uniform argument here also makes the compiler fetch
  // them all in the first batch of loads.
  const bool bad_size = (p.n_rows | p.h_in | p.num_segs | p.num_loras | p.num_units64 | p.direct_units64 |
                         p.ksplit | p.kc | (int32_t)(p.partial_stride >> 32) | (int32_t)(p.proj_stride >> 32)) < 0;
  const bool bad_ptr = (p.seg_indptr == nullptr) | (p.lora_idx == nullptr) | (p.X == nullptr) |
                       (p.partials == nullptr) | (pj.A_ptrs == nullptr);
  if (bad_size | bad_ptr) return;
  const int idx = xcd_linear_index();
  if (idx >= p.num_units64 * p.ksplit) return;
  const int g = idx / p.num_units64;
  const int unit = idx - g * p.num_units64;
  const Unit un = resolve_unit<kMT>(p.seg_indptr, p.lora_idx, p.num_segs, p.num_loras, p.n_rows,
                                    p.direct_units64, unit);
  if (un.L <= 0) return;
  const int L = un.L, r0 = un.r0;
  const uint16_t* Ak = reinterpret_cast<const uint16_t*>(pj.A_ptrs[un.k]);
  // Rank of the LoRA: A_k rows are rk wide; ranks >= rk are zero.
  int rk = R;
  if constexpr (EXT) {
    if (pj.ranks) rk = lora_rank<R>(pj.ranks[un.k]);
    if (rk == 0) return;  // nothing to add (the expand skips the unit too)
  }
  const int a_stride = EXT ? rk : R;
  const int k0 = g * p.kc;
  const int k1 = p.h_in < k0 + p.kc ? p.h_in : k0 + p.kc;
  // X rows of this thread.  XL: rows xr0 + 16m (m < NXV), h block xc of each
  // stage; otherwise the row the lane feeds into the MFMA A operand.  Rows
  // past the segment re-read its last row; they feed MFMA rows that are never
  // stored.
  const int xr0 = XL ? t / XV : wave * 16 + ml;
  const int xc = t % XV;
  constexpr int NXR = XL ? NXV : 1;
  const uint16_t* xrow[NXR];
#pragma unroll
  for (int m = 0; m < NXR; ++m) {
    const int rr = xr0 + m * (kThreads / XV);
    const int srow = r0 + (rr < L ? rr : L - 1);
    xrow[m] = p.X + (EXT && p.row_idx ? (int64_t)p.row_idx[srow] : (int64_t)srow) * p.h_in;
  }
  // X through the L1 at rank <= 16: with the direct layout, the next k-step's
  // load hits the other half of each line there; with either layout the
  // expand that follows ran faster (mixed r = 16, 4096 -> 11008: 60.5 -> 56.4
  // us) than after streaming X.  At rank 64 cached X costs the A_k stages
  // their L2 reuse (4096 -> 11008: 89.3 -> 92.7 us per call) and streams.
  auto load_x = [](const uint16_t* a) { return R <= 16 ? load_vec(a) : load_stream(a); };

  // All loads of one stage, at clamped (valid) addresses; values past k1 are
  // zeroed where they are consumed.
  auto issue = [&](int kk, u32x4 (&x)[NXV], u32x4 (&a)[NPAIR][2]) {
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) {
      const int pr = t + kThreads * m;
      int hp, jg;
      pair_of(pr, hp, jg);
      const int h = kk + hp * 2;
      const bool ok = pr < PAIRS && (!EXT || jg * 8 < rk);
      a[m][0] = load_stream(Ak + (ok && h < k1 ? (int64_t)h * a_stride + jg * 8 : 0));
      a[m][1] = load_stream(Ak + (ok && h + 1 < k1 ? (int64_t)(h + 1) * a_stride + jg * 8 : 0));
    }
    if constexpr (XL) {
      const int h = kk + xc * 8;
#pragma unroll
      for (int m = 0; m < NXV; ++m) x[m] = load_x(xrow[m] + (h < k1 ? h : 0));
    } else {
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        const int h = kk + s * 32 + q * 8;
        x[s] = load_x(xrow[0] + (h < k1 ? h : 0));
      }
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage the A_k rows transposed ([r][h]) so that a lane reads the 8
  // consecutive h of one rank with one 128-bit LDS read, then multiply.
  auto compute = [&](int kk, const u32x4 (&x)[NXV], const u32x4 (&a)[NPAIR][2]) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    __syncthreads();  // the previous stage is done with lds_at
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) {
      const int pr = t + kThreads * m;
      if (pr < PAIRS) {
        int hp, jg;
        pair_of(pr, hp, jg);
        const int h = hp * 2;
        const bool live = !EXT || jg * 8 < rk;
        // rank rows jg*8..+3 share one swz, rows jg*8+4..+7 the next
        const int hs0 = (((h >> 3) ^ swz(jg * 8)) << 3) | (h & 7);
        const int hs1 = (((h >> 3) ^ swz(jg * 8 + 4)) << 3) | (h & 7);
        store_pair_transposed_split(&lds_at[(jg * 8) * AST + hs0], &lds_at[(jg * 8 + 4) * AST + hs1], AST,
                                    live && kk + h < k1 ? a[m][0] : z, live && kk + h + 1 < k1 ? a[m][1] : z);
      }
    }
    if constexpr (XL) {
      const bool xlive = kk + xc * 8 < k1;  // ragged tail of H1: zeros
#pragma unroll
      for (int m = 0; m < NXV; ++m)
        store_vec(&lds_x[(xr0 + m * (kThreads / XV)) * XST + xc * 8], xlive ? x[m] : z);
    }
    __syncthreads();
    if (wave * 16 >= L) return;  // this wave's rows are all past the segment
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      u32x4 xa;
      if constexpr (XL)
        xa = load_vec(&lds_x[(wave * 16 + ml) * XST + s * 32 + q * 8]);
      else
        xa = kk + s * 32 + q * 8 < k1 ? x[s] : z;  // ragged tail of H1
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = mfma<T>(xa, load_vec(&lds_at[(n * 16 + ml) * AST + (((4 * s + q) ^ swz(n * 16 + ml)) << 3)]), acc[n]);
    }
  };

  // Ping-pong over stage pairs: each buffer is waited for only where it is
  // consumed.  A stage past k1 loads clamped addresses and contributes zeros.
  // The loop body issues its loads unconditionally (a load under a branch
  // makes the compiler wait for every load in flight at the loop head); the
  // last stage pair, which issues no loads beyond itself, is peeled.
  u32x4 xA[NXV], aA[NPAIR][2], xB[NXV], aB[NPAIR][2];
  issue(k0, xA, aA);
  int kk = k0;
  for (; kk + 2 * kKStage < k1; kk += 2 * kKStage) {
    issue(kk + kKStage, xB, aB);
    compute(kk, xA, aA);
    issue(kk + 2 * kKStage, xA, aA);
    compute(kk + kKStage, xB, aB);
  }
  issue(kk + kKStage, xB, aB);
  compute(kk, xA, aA);
  compute(kk + kKStage, xB, aB);

  // D[4q+i][ml] of rank tile n: row wave*16 + 4q + i, rank n*16 + ml.
  float* dst = p.partials + (int64_t)blockIdx.y * p.proj_stride + (int64_t)g * p.partial_stride;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = wave * 16 + q * 4 + i;
      if (rr < L) dst[(int64_t)(r0 + rr) * R + n * 16 + ml] = acc[n][i];
    }
}

// ---------------------------------------------------------------- reduce
// V[row] = sum over the ksplit partial planes, in plane order.  The segments
// tile the rows [0, seg_indptr[num_segs]) in order, so the rows to reduce
// are known without looking up any segment: a workgroup takes kThreads / (R/4)
// rows, every thread one float4 of one row, and all of the thread's plane
// loads are issued at once (together with the one load of the row bound).
// Rows outside all segments are left untouched.
template <int R>
// Few waves per SIMD are needed (the kernel is one round of loads), so the
// scheduler may use registers to keep every load of a batch in flight.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void sgmv_mfma_reduce_kernel(MfmaParams p) {
  constexpr int V4 = R / 4;                 // float4 per row of V
  constexpr int ROWS = kThreads / V4;       // rows per workgroup
  constexpr int kBatch = 32;                // plane loads in flight per thread
  const bool bad = (p.n_rows | p.num_segs | (p.ksplit - 1) | (int32_t)(p.partial_stride >> 32) |
                    (int32_t)(p.proj_stride >> 32)) < 0;
  const bool bad_ptr = (p.seg_indptr == nullptr) | (p.partials == nullptr) | (p.V == nullptr);
  if (bad | bad_ptr) return;
  const int t = threadIdx.x;
  const int row = blockIdx.x * ROWS + t / V4;
  const float* partials = p.partials + (int64_t)blockIdx.y * p.proj_stride;
  float* V = p.V + (int64_t)blockIdx.y * p.proj_stride;
  int end = p.seg_indptr[p.num_segs];
  end = end < p.n_rows ? end : p.n_rows;
  const int64_t off = (int64_t)(row < p.n_rows ? row : p.n_rows - 1) * R + (t % V4) * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  const int64_t span = (int64_t)p.ksplit * p.partial_stride * 4;  // bytes of all planes
  if (span <= (int64_t)UINT32_MAX) {
    // One uniform base address and a 32-bit offset per load: all of a
    // batch's loads are issued before the first add waits.
    const char* base = reinterpret_cast<const char*>(partials);
    const uint32_t pstride = (uint32_t)(p.partial_stride * 4);
    const uint32_t boff = (uint32_t)(off * 4);
    for (int k0 = 0; k0 < p.ksplit; k0 += kBatch) {
      f32x4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t k = (uint32_t)(k0 + u < p.ksplit ? k0 + u : p.ksplit - 1);
        v[u] = *reinterpret_cast<const f32x4*>(base + (k * pstride + boff));
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const f32x4 a = s + v[u];
        s = k0 + u < p.ksplit ? a : s;
      }
    }
  } else {
    for (int k = 0; k < p.ksplit; ++k) s += *reinterpret_cast<const f32x4*>(partials + k * p.partial_stride + off);
  }
  if (row < end) *reinterpret_cast<f32x4*>(V + off) = s;
}

// ---------------------------------------------------------------- lead reduce
// Lead workgroup b of projection y: V of rows [b * lead_rows, (b + 1) *
// lead_rows) = the sum of the partial planes in plane order from zero (the
// reduce launch's order and bits).  TAGGED: published as words {fp32, launch
// tag}; otherwise V is written through to the device-coherent level and, once
// every thread's stores have completed, flags[b] = tag.  Lead workgroups never
// wait, and they have the lowest workgroup ids of the launch, so they are
// dispatched ahead of every workgroup that waits for them.  Up to 16 planes a
// thread sums one float4 of a row (1024 / R rows per workgroup); beyond, one
// float2 (512 / R rows), so that every plane load of a thread is in flight at
// once up to 32 planes at the same register count (more would cost the expand
// occupancy).
template <int R, int W, bool TAGGED>
__device__ inline void lead_sum(const MfmaParams& p, int y, int b, uint32_t tag) {
  using VT = __attribute__((ext_vector_type(W))) float;
  constexpr int VW = R / W;               // vectors per row of V
  constexpr int ROWS = kThreads / VW;
  constexpr int kBatch = 64 / W;          // plane loads in flight per thread
  const int t = threadIdx.x;
  const int row = b * ROWS + t / VW;
  const float* partials = p.partials + (int64_t)y * p.proj_stride;
  char* area = static_cast<char*>(p.lead_area) + (int64_t)y * p.proj_stride * 4;
  int end = p.seg_indptr[p.num_segs];
  end = end < p.n_rows ? end : p.n_rows;
  const int64_t off = (int64_t)(row < p.n_rows ? row : p.n_rows - 1) * R + (t % VW) * W;
  VT s = {};
  for (int k0 = 0; k0 < p.ksplit; k0 += kBatch) {
    VT v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t k = k0 + u < p.ksplit ? k0 + u : p.ksplit - 1;
      v[u] = *reinterpret_cast<const VT*>(partials + k * p.partial_stride + off);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const VT a = s + v[u];
      s = k0 + u < p.ksplit ? a : s;
    }
  }
  if constexpr (TAGGED) {
    if (row < end) {
      uint64_t* dst = reinterpret_cast<uint64_t*>(area) + off;
#pragma unroll
      for (int e = 0; e < W; ++e) publish_tagged(dst + e, s[e], tag);
    }
  } else {
    if (row < end) {
      uint64_t* dst = reinterpret_cast<uint64_t*>(p.V + (int64_t)y * p.proj_stride + off);
#pragma unroll
      for (int e = 0; e < W / 2; ++e)
        publish_u64(dst + e, ((uint64_t)__float_as_uint(s[2 * e + 1]) << 32) | __float_as_uint(s[2 * e]));
    }
    wait_memory_ops();
    __syncthreads();
    if (t == 0)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(area) + b, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int R, bool TAGGED>
__device__ inline void lead_reduce_rows(const MfmaParams& p, int y, int b, uint32_t tag) {
  if (p.lead_rows == kThreads * 4 / R)
    lead_sum<R, 4, TAGGED>(p, y, b, tag);
  else
    lead_sum<R, 2, TAGGED>(p, y, b, tag);
}

// ---------------------------------------------------------------- expand
// MT rows per tile.  MT = 64: wave w computes rows 16w..16w+15 over the whole
// chunk.  MT = 16 (short segments, e.g. decode batches with a few rows per
// LoRA): the four waves share the 16 rows and each computes a quarter of the
// chunk's columns, so no wave idles and the smaller LDS footprint lets more
// workgroups stream B_k at once.
// LEAD: the launch carries lead workgroups (p.lead_reduce); a template flag so
// that the kernels without them keep their register count (occupancy).
template <class T, int R, bool EXT, int MT, bool LEAD>
__global__ __launch_bounds__(kThreads) void sgmv_mfma_expand_kernel(MfmaParams p) {
  constexpr int K2 = 2 * R;            // virtual K: [V_hi | V_lo] against [B_k; B_k]
  constexpr int KSTEPS = K2 / 32;
  constexpr int WR = MT / 16;          // 16-row groups of the tile
  constexpr int WC = kWaves / WR;      // waves that share a row group, each on its own columns
  static_assert(WR * WC == kWaves, "tile rows are 16, 32 or 64");
  constexpr int NTC = kCW / 16;        // 16-wide column tiles per chunk
  constexpr int NTW = NTC / WC;        // column tiles per wave
  constexpr int CV = kCW / 8;          // 128-bit column vectors per chunk row
  constexpr int CVW = CV / WC;         // ... of one wave's columns
  // LDS stride (halves) of transposed B_k, per column: 40 dwords at r = 64 and
  // 24 at r = 16, which the 16 columns of one 128-bit MFMA operand read cover
  // without bank conflicts (r + 8 halves costs a second pass).  At r = 32 the
  // conflict-free 24 dwords would leave room for only two 64-row workgroups
  // per CU instead of three; it keeps r + 8.
  constexpr int BST = R + (R == 64 ? 16 : R == 32 ? 8 : 32);
  // Within a column, B_k's ranks sit in groups of 8 (one 128-bit MFMA operand
  // read); group g of column c is stored at group g ^ swz(c), constant over a
  // 16-column MFMA tile (the operand reads stay conflict-free).  At r = 64 the
  // xor takes the even groups, so that with the pair map below the transposed
  // stores of a half-wave (8 rank pairs of 4 tiles) meet every bank once.
  constexpr int GMASK = R / 8 - 1;
  auto swz = [](int c) { return (R == 64 ? 2 * (c >> 4) : c >> 4) & GMASK; };
  // (rank pair, 8-column group) item pr of a chunk -> first rank j and first
  // chunk column cl.  At r = 64 a half-wave takes rank pairs 0..7 of every
  // other column group (4 tiles) and a wave 8 whole column groups, so its
  // loads still read 128 contiguous bytes of each B_k row.
  auto item_of = [](int pr, int& j, int& cl) {
    if constexpr (R == 64) {
      const int rest = pr >> 6;
      j = 2 * (((pr >> 2) & 7) + 8 * (rest >> 1));
      cl = 8 * ((((pr & 3) << 1) | ((pr >> 5) & 1)) + 8 * (rest & 1));
    } else {
      j = (pr / (kCW / 8)) * 2;
      cl = (pr % (kCW / 8)) * 8;
    }
  };
  constexpr int VST = K2 + 8;          // LDS stride (halves) of [V_hi | V_lo], per row
  constexpr int OST = kCW / WC + 4;    // LDS stride (floats) of a wave's result tile
  constexpr int NBP = (R / 2 * CV + kThreads - 1) / kThreads;  // (j, j+1) B_k vector pairs per thread
  constexpr int NYV = 16 * CVW / 64;   // Y vectors per lane (16 rows of the wave's columns)
  __shared__ __attribute__((aligned(16))) uint16_t lds_bt[kCW * BST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[MT * VST];
  __shared__ __attribute__((aligned(16))) float lds_o[kWaves * 16 * OST];
  // fp16 holds V's hi and lo halves only below 65504: a tile row whose V is
  // larger is scaled down by a power of two before the split and its product
  // scaled back in fp32 (both exact).  bf16 has fp32's range: no scaling.
  constexpr bool kRowScale = T::kMaxFinite < 1e5f;
  __shared__ float lds_rs[MT];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int q = lane >> 4;
  const int ml = lane & 15;
  const int wr = wave / WC;            // row group of the wave
  const int colw = (wave % WC) * (kCW / WC);  // first chunk column of the wave
  const Projection pj = p.proj[blockIdx.y];
  // Malformed launch test; it also batches the argument loads (as in the shrink).
  const bool bad_size = (p.n_rows | p.h_out | p.num_segs | p.num_loras | p.num_units_x | p.direct_units_x |
                         (p.chunks_per_wg - 1) | (int32_t)(p.proj_stride >> 32) | (p.ksplit - 1) |
                         (int32_t)(p.partial_stride >> 32)) < 0;
  const bool bad_ptr = (p.seg_indptr == nullptr) | (p.lora_idx == nullptr) |
                       (p.V == nullptr) | (pj.B_ptrs == nullptr) |
                       (pj.Y == nullptr);
  if (bad_size | bad_ptr) return;
  // 16-row tiles read V as tagged words (a tile's V is small); larger tiles,
  // each reading 4 KiB of V per 16 rows from every column group, wait for one
  // flag per row block and read V itself (half the device-coherent bytes).
  constexpr bool kTaggedV = MT == 16;
  const int lead = LEAD ? p.lead_blocks * p.lead_proj : 0;
  if (LEAD && (p.partials == nullptr) | (p.lead_area == nullptr) | (p.errors == nullptr) |
      ((p.lead_blocks | (p.lead_proj - 1) | (p.lead_rows - 1)) < 0))
    return;
  const uint32_t tag = LEAD ? launch_tag() : 0u;
  if (LEAD && (int)blockIdx.x < lead) {
    if (blockIdx.y == 0) lead_reduce_rows<R, kTaggedV>(p, blockIdx.x / p.lead_blocks, blockIdx.x % p.lead_blocks, tag);
    return;
  }
  const int nchunks = (p.h_out + kCW - 1) / kCW;
  const int ngroups = (nchunks + p.chunks_per_wg - 1) / p.chunks_per_wg;
  // Linear order: column group major, so the row units that read one slice of
  // B_k share an XCD.
  const int idx = xcd_linear_index(lead);
  if (idx >= p.num_units_x * ngroups) return;
  const int grp = idx / p.num_units_x;
  const int unit = idx - grp * p.num_units_x;
  const Unit un = resolve_unit<MT>(p.seg_indptr, p.lora_idx, p.num_segs, p.num_loras, p.n_rows,
                                   p.direct_units_x, unit);
  if (un.L <= 0) return;
  const int L = un.L, r0 = un.r0;
  const int ch0 = grp * p.chunks_per_wg;
  const int ch1 = nchunks < ch0 + p.chunks_per_wg ? nchunks : ch0 + p.chunks_per_wg;
  const uint16_t* Bk = reinterpret_cast<const uint16_t*>(pj.B_ptrs[un.k]);
  // Rank of the LoRA: B_k has rk rows; V's ranks >= rk are zero.  The LoRA's
  // scale multiplies V (fp32) before it is split.
  int rk = R;
  float sk = 1.f;
  if constexpr (EXT) {
    if (pj.ranks) rk = lora_rank<R>(pj.ranks[un.k]);
    if (pj.scales) sk = pj.scales[un.k];
    if (rk == 0) return;  // Y keeps its value
  }
  uint16_t* Ybase = pj.Y;
  const float* Vp = p.V + (int64_t)blockIdx.y * p.proj_stride;
  // Row of Y behind each tile row this lane loads and stores, looked up once
  // (tile rows past the segment take the first row and are never stored).
  int yrow[NYV];
#pragma unroll
  for (int u = 0; u < NYV; ++u) {
    const int rr = wr * 16 + (lane + 64 * u) / CVW;
    const int srow = r0 + (rr < L ? rr : 0);
    yrow[u] = EXT && p.row_idx ? p.row_idx[srow] : srow;
  }

  // Loads of one chunk (all lanes issue the same loads; addresses of lanes
  // without work are clamped to a valid element).
  auto issue = [&](int ch, u32x4 (&bv)[NBP][2], u32x4 (&yv)[NYV]) {
    const int c0 = ch * kCW;
#pragma unroll
    for (int m = 0; m < NBP; ++m) {
      const int pv = t + kThreads * m;
      int j, cl;
      item_of(pv, j, cl);
      const int c = c0 + cl;
      const bool ok = pv < R / 2 * CV && ch < ch1 && c < p.h_out && (!EXT || j < rk);
      bv[m][0] = load_stream(Bk + (ok ? (int64_t)j * p.h_out + c : 0));
      bv[m][1] = load_stream(Bk + (ok ? (int64_t)(j + 1) * p.h_out + c : 0));
    }
#pragma unroll
    for (int u = 0; u < NYV; ++u) {
      const int v = lane + 64 * u;
      const int rr = wr * 16 + v / CVW;
      const int c = c0 + colw + (v % CVW) * 8;
      const bool ok = rr < L && ch < ch1 && c < p.h_out;
      yv[u] = load_stream(Ybase + (int64_t)yrow[u] * p.h_out + (ok ? c : 0));
    }
  };
  // V of the tile rows (all fetched at once, ahead of the first chunk's loads
  // so that waiting for V does not wait for them), split hi/lo, then this
  // wave's MFMA A fragments.
  constexpr int NVF = MT * R / 4;                       // float4 of V in the tile
  constexpr int NV4 = (NVF + kThreads - 1) / kThreads;  // ... per thread
  f32x4 vv[NV4];
  u32x4 bvA[NBP][2], yvA[NYV], bvB[NBP][2], yvB[NYV];
  if (LEAD) {
    // V of these rows is summed by lead workgroups of this launch: the first
    // chunk's loads go out, then the wait (bounded; a limit of 0, the host's
    // test hook, waits for a tag no word carries).
    issue(ch0, bvA, yvA);
    __shared__ uint32_t lds_gave_up;
    if (t == 0) lds_gave_up = 0;
    __syncthreads();
    const uint32_t want = p.wait_ticks != 0 ? tag : ~tag;
    const char* area = static_cast<const char*>(p.lead_area) + (int64_t)blockIdx.y * p.proj_stride * 4;
    const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + p.wait_ticks;
    uint64_t now = 0;  // read beside each round of polls, checked at the next
    bool done;
    if constexpr (kTaggedV) {
      // Every thread polls the tagged words of its V values.
      const uint64_t* vt = reinterpret_cast<const uint64_t*>(area);
      uint64_t w[NV4][4];
#pragma unroll
      for (int m = 0; m < NV4; ++m) {
        const int o = (t + kThreads * m) * 4;
        const int rr = o / R;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[m][e] = fetch_tagged(vt + (int64_t)(r0 + (rr < L ? rr : 0)) * R + o % R + e);
      }
      for (;;) {
        done = true;
#pragma unroll
        for (int m = 0; m < NV4; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((uint32_t)(w[m][e] >> 32) != want) done = false;
        if (done || now > deadline) break;
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int m = 0; m < NV4; ++m) {
          const int o = (t + kThreads * m) * 4;
          const int rr = o / R;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((uint32_t)(w[m][e] >> 32) != want)
              w[m][e] = fetch_tagged(vt + (int64_t)(r0 + (rr < L ? rr : 0)) * R + o % R + e);
        }
        now = __builtin_amdgcn_s_memrealtime();
      }
#pragma unroll
      for (int m = 0; m < NV4; ++m)
        vv[m] = f32x4{__uint_as_float((uint32_t)w[m][0]), __uint_as_float((uint32_t)w[m][1]),
                      __uint_as_float((uint32_t)w[m][2]), __uint_as_float((uint32_t)w[m][3])};
    } else {
      // One lane per row block of the tile polls its flag.
      done = true;
      if (t < 64) {
        const int b0 = r0 / p.lead_rows, nb = (r0 + L - 1) / p.lead_rows - b0 + 1;
        const uint32_t* fl = reinterpret_cast<const uint32_t*>(area) + b0;
        if (lane < nb) {
          uint32_t f = __hip_atomic_load(fl + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          while (f != want && now <= deadline) {
            __builtin_amdgcn_s_sleep(1);
            f = __hip_atomic_load(fl + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            now = __builtin_amdgcn_s_memrealtime();
          }
          done = f == want;
        }
      }
    }
    if (!done) lds_gave_up = 1;
    __syncthreads();
    if (lds_gave_up) {
      if (t == 0) __hip_atomic_fetch_or(p.errors, kDecodeErrWaitTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;  // Y untouched
    }
    if constexpr (!kTaggedV) {
#pragma unroll
      for (int m = 0; m < NV4; ++m) {
        const int o = (t + kThreads * m) * 4;
        const int rr = o / R;
        const uint64_t* src =
            reinterpret_cast<const uint64_t*>(Vp + (int64_t)(r0 + (rr < L ? rr : 0)) * R + o % R);
        const uint64_t lo = fetch_published_u64(src), hi = fetch_published_u64(src + 1);
        vv[m] = f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                      __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < NV4; ++m) {
      const int o = (t + kThreads * m) * 4;
      const int rr = o / R;
      vv[m] = *reinterpret_cast<const f32x4*>(Vp + (int64_t)(r0 + (rr < L ? rr : 0)) * R + o % R);
    }
    issue(ch0, bvA, yvA);
  }
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    const int o = (t + kThreads * m) * 4;
    if (o < NVF * 4) {
      const int rr = o / R, j = o % R;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = rr < L ? vv[m][e] * sk : 0.f;
      if constexpr (kRowScale) {
        // The R / 4 lanes of one row (consecutive lanes) agree on its largest
        // magnitude; rows under 2^15 keep the factor 1 (the same bits as
        // without scaling).
        float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
        for (int d = 1; d < R / 4; d <<= 1) mx = fmaxf(mx, shfl_xor(mx, d));
        const int k = isfinite(mx) && mx >= 32768.f ? ilogbf(mx) - 14 : 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ldexpf(v[e], -k);
        if (j == 0) lds_rs[rr] = ldexpf(1.f, k);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t hi = T::round(v[e]);
        const uint16_t lo = T::round(v[e] - T::one(hi));
        lds_v[rr * VST + j + e] = hi;
        lds_v[rr * VST + R + j + e] = lo;
      }
    }
  }
  __syncthreads();
  u32x4 af[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) af[s] = load_vec(&lds_v[(wr * 16 + ml) * VST + s * 32 + q * 8]);
  float* out = lds_o + wave * 16 * OST;

  auto compute = [&](int ch, const u32x4 (&bv)[NBP][2], const u32x4 (&yv)[NYV]) {
    const int c0 = ch * kCW;
    __syncthreads();  // the previous chunk is done with lds_bt and lds_o
#pragma unroll
    for (int m = 0; m < NBP; ++m) {
      const int pr = t + kThreads * m;
      if (pr < R / 2 * CV) {
        int j, cl;
        item_of(pr, j, cl);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const bool live = !EXT || j < rk;  // rk is even, so j < rk covers row j + 1 too
        const int js = (((j >> 3) ^ swz(cl)) << 3) | (j & 7);  // columns cl..cl+7 share swz(cl)
        store_pair_transposed(&lds_bt[cl * BST + js], BST, live ? bv[m][0] : z, live ? bv[m][1] : z);
      }
    }
    __syncthreads();
    // A wave whose 16 rows are all past the segment has nothing to compute or
    // store; each wave's result tile is its own, so only the wave itself
    // waits for it (LDS operations of one wave complete in order).
    if (wr * 16 >= L) return;
#pragma unroll
    for (int n = 0; n < NTW; ++n) {
      const int cn = colw + n * 16;    // first chunk column of the tile
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int kb = (s * 32 + q * 8) % R;  // rank of the B_k copy this k-group reads
        acc = mfma<T>(af[s], load_vec(&lds_bt[(cn + ml) * BST + (((kb >> 3) ^ swz(cn)) << 3)]), acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(q * 4 + i) * OST + n * 16 + ml] = acc[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < NYV; ++u) {
      const int v = lane + 64 * u;
      const int rl = v / CVW;
      const int cl = (v % CVW) * 8;
      const int rr = wr * 16 + rl;
      const int c = c0 + colw + cl;
      if (rr < L && ch < ch1 && c < p.h_out) {
        float yf[8];
        unpack8<T>(yv[u], yf);
        if constexpr (kRowScale) {
          const float rs = lds_rs[rr];
#pragma unroll
          for (int e = 0; e < 8; ++e) yf[e] += out[rl * OST + cl + e] * rs;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) yf[e] += out[rl * OST + cl + e];
        }
        // 16-row tiles (short segments, many units per LoRA re-reading its
        // B_k slice) store Y non-temporally, which leaves B_k in L2 (13B
        // forward 5.91 -> 5.81 ms); larger tiles were 2-4% slower that way.
        if constexpr (MT == 16)
          store_stream(Ybase + (int64_t)yrow[u] * p.h_out + c, pack8<T>(yf));
        else
          store_vec(Ybase + (int64_t)yrow[u] * p.h_out + c, pack8<T>(yf));
      }
    }
  };
  // Ping-pong over chunk pairs: chunk ch+1 is in flight while chunk ch is
  // computed.  The body has no branch, so the loads of one buffer are waited
  // for only where that buffer is consumed (a chunk past ch1 loads clamped
  // addresses); an odd last chunk is computed once after the loop.
  int ch = ch0;
  for (; ch + 1 < ch1; ch += 2) {
    issue(ch + 1, bvB, yvB);
    compute(ch, bvA, yvA);
    issue(ch + 2, bvA, yvA);
    compute(ch + 1, bvB, yvB);
  }
  // An odd last chunk, already in flight in buffer A.
  if (ch < ch1) compute(ch, bvA, yvA);
}

unsigned xcd_grid(unsigned items) { return kXcds * ((items + kXcds - 1) / kXcds); }

template <class T, int R>
hipError_t launch_t(int stage, const MfmaParams& p, int np, hipStream_t s) {
  unsigned grid = 0;
  bool ext = p.row_idx != nullptr;
  for (int i = 0; i < np; ++i) ext = ext || p.proj[i].ranks || p.proj[i].scales;
  if (stage == 0) {
    grid = xcd_grid((unsigned)p.num_units64 * (unsigned)p.ksplit);
    if (grid && np > 0) {
      using K = void (*)(MfmaParams);
      // [x through LDS][ext]
      static constexpr K kernels[2][2] = {
          {sgmv_mfma_shrink_kernel<T, R, false, false>, sgmv_mfma_shrink_kernel<T, R, true, false>},
          {sgmv_mfma_shrink_kernel<T, R, false, true>, sgmv_mfma_shrink_kernel<T, R, true, true>}};
      hipLaunchKernelGGL(kernels[p.x_lds ? 1 : 0][ext], dim3(grid, np), dim3(kThreads), 0, s, p);
    }
  } else if (stage == 1) {
    constexpr unsigned rows = kThreads / (R / 4);
    grid = ((unsigned)p.n_rows + rows - 1) / rows;
    if (grid && np > 0) hipLaunchKernelGGL((sgmv_mfma_reduce_kernel<R>), dim3(grid, np), dim3(kThreads), 0, s, p);
  } else {
    if (p.expand_rows != 16 && p.expand_rows != 32 && p.expand_rows != kMT) return hipErrorInvalidValue;
    const int nchunks = (p.h_out + kCW - 1) / kCW;
    grid = xcd_grid((unsigned)p.num_units_x * (unsigned)((nchunks + p.chunks_per_wg - 1) / p.chunks_per_wg));
    if (p.lead_reduce) {
      if (p.lead_blocks % kXcds != 0 || p.lead_proj != np ||
          (p.lead_rows != kThreads * 4 / R && p.lead_rows != kThreads * 2 / R) ||
          (int64_t)p.lead_blocks * p.lead_rows < (int64_t)p.n_rows)
        return hipErrorInvalidValue;
      if (grid) grid += (unsigned)(p.lead_blocks * np);
    }
    if (grid && np > 0) {
      using K = void (*)(MfmaParams);
      // [lead workgroups][tile rows 64, 32, 16][ext]
      static constexpr K kernels[2][3][2] = {
          {{sgmv_mfma_expand_kernel<T, R, false, kMT, false>, sgmv_mfma_expand_kernel<T, R, true, kMT, false>},
           {sgmv_mfma_expand_kernel<T, R, false, 32, false>, sgmv_mfma_expand_kernel<T, R, true, 32, false>},
           {sgmv_mfma_expand_kernel<T, R, false, 16, false>, sgmv_mfma_expand_kernel<T, R, true, 16, false>}},
          {{sgmv_mfma_expand_kernel<T, R, false, kMT, true>, sgmv_mfma_expand_kernel<T, R, true, kMT, true>},
           {sgmv_mfma_expand_kernel<T, R, false, 32, true>, sgmv_mfma_expand_kernel<T, R, true, 32, true>},
           {sgmv_mfma_expand_kernel<T, R, false, 16, true>, sgmv_mfma_expand_kernel<T, R, true, 16, true>}}};
      const int which = p.expand_rows == kMT ? 0 : p.expand_rows == 32 ? 1 : 2;
      hipLaunchKernelGGL(kernels[p.lead_reduce ? 1 : 0][which][ext], dim3(grid, np), dim3(kThreads), 0, s, p);
    }
  }
  return grid && np > 0 ? hipGetLastError() : hipSuccess;
}

template <class T>
hipError_t launch_rank(int rank, int stage, const MfmaParams& p, int np, hipStream_t s) {
  switch (rank) {
    case 16: return launch_t<T, 16>(stage, p, np, s);
    case 32: return launch_t<T, 32>(stage, p, np, s);
    case 64: return launch_t<T, 64>(stage, p, np, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_stage(int dtype, int rank, int stage, const MfmaParams& p, int np, hipStream_t s) {
  return dtype == 1 ? launch_rank<BF16>(rank, stage, p, np, s) : launch_rank<F16>(rank, stage, p, np, s);
}

}  // namespace


hipError_t launch_mfma_shrink(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream) {
  hipError_t e = launch_stage(dtype, rank, 0, p, num_proj, stream);
  // Nothing to reduce when the expand launch sums the planes (lead
  // workgroups) or when V is the single plane itself.
  if (e != hipSuccess || p.lead_reduce || p.V == p.partials) return e;
  return launch_stage(dtype, rank, 1, p, num_proj, stream);
}

hipError_t launch_mfma_expand(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream) {
  return launch_stage(dtype, rank, 2, p, num_proj, stream);
}

}  // namespace sgmv
