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
// Three launches:
//  1. shrink: a workgroup (4 waves, 16 rows each) takes up to 64 rows of one
//     segment and one chunk of H1, streamed in stages of 128 H1 rows that are
//     pipelined two deep: the X fragments (registers, straight from HBM) and
//     A_k rows of the next stage are in flight while the current one is
//     multiplied.  Each stage of A_k is staged in LDS, transposed to [r][h] so
//     that a lane reads the 8 consecutive h of one rank with one 128-bit LDS
//     read.  Each H1 chunk writes its own fp32 partial plane of V; workgroups
//     that read the same chunk of A_k run on one XCD.
//  2. reduce: V = sum of the partial planes, in chunk order (reproducible);
//     the LoRA's scale, if any, is applied to V by the expand.
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
__device__ inline int xcd_linear_index() {
  const int per_xcd = gridDim.x / kXcds;
  return (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
}


// ---------------------------------------------------------------- shrink
// H1 rows per pipeline stage: while one stage's X fragments and A_k rows are
// multiplied, the next stage's loads are in flight.
constexpr int kKStage = 128;

// EXT: the extended arguments may be set (row map, per-LoRA ranks and scales;
// see the decode kernel).  Without EXT the kernel carries none of it.
template <class T, int R, bool EXT>
__global__ __launch_bounds__(kThreads) void sgmv_mfma_shrink_kernel(MfmaParams p) {
  constexpr int NT = R / 16;                // 16-wide rank tiles
  constexpr int JG = R / 8;                 // 128-bit vectors per row of A_k
  constexpr int PAIRS = kKStage / 2 * JG;   // (h, h+1) vector pairs of A_k per stage
  constexpr int NPAIR = (PAIRS + kThreads - 1) / kThreads;
  constexpr int MS = kKStage / 32;          // MFMA k-steps per stage
  constexpr int AST = kKStage + 8;          // LDS row stride (halves) of transposed A_k
  // Within a rank row, the stage's h sit in groups of 8 (one 128-bit MFMA
  // operand read); group g of rank row r is stored at group g ^ swz(r), which
  // spreads a wave's transposed stores over the LDS banks at ranks 32 and 64
  // (rank 16 is conflict-free as is) while the operand reads stay
  // conflict-free.
  auto swz = [](int r) { return (r >> 4) << (R == 64 ? 1 : 2); };
  static_assert(kMfmaKChunk % (2 * kKStage) == 0, "H1 chunks hold whole stage pairs");
  __shared__ __attribute__((aligned(16))) uint16_t lds_at[R * AST];

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
  // Row this lane feeds into the MFMA A operand (rows past the segment re-read
  // its last row and are never stored).
  const int row = wave * 16 + ml;
  const int srow = r0 + (row < L ? row : L - 1);
  const uint16_t* xrow = p.X + (EXT && p.row_idx ? (int64_t)p.row_idx[srow] : (int64_t)srow) * p.h_in;

  // All loads of one stage, at clamped (valid) addresses; values past k1 are
  // zeroed where they are consumed.
  auto issue = [&](int kk, u32x4 (&x)[MS], u32x4 (&a)[NPAIR][2]) {
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) {
      const int pr = t + kThreads * m;
      const int h = kk + (pr / JG) * 2, jg = pr % JG;
      const bool ok = pr < PAIRS && (!EXT || jg * 8 < rk);
      a[m][0] = load_stream(Ak + (ok && h < k1 ? (int64_t)h * a_stride + jg * 8 : 0));
      a[m][1] = load_stream(Ak + (ok && h + 1 < k1 ? (int64_t)(h + 1) * a_stride + jg * 8 : 0));
    }
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      const int h = kk + s * 32 + q * 8;
      x[s] = load_stream(xrow + (h < k1 ? h : 0));
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage the A_k rows transposed ([r][h]) so that a lane reads the 8
  // consecutive h of one rank with one 128-bit LDS read, then multiply.
  auto compute = [&](int kk, const u32x4 (&x)[MS], const u32x4 (&a)[NPAIR][2]) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    __syncthreads();  // the previous stage is done with lds_at
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) {
      const int pr = t + kThreads * m;
      if (pr < PAIRS) {
        const int h = (pr / JG) * 2, jg = pr % JG;
        const bool live = !EXT || jg * 8 < rk;
        const int hs = (((h >> 3) ^ swz(jg * 8)) << 3) | (h & 7);  // rows jg*8..+7 share swz
        store_pair_transposed(&lds_at[(jg * 8) * AST + hs], AST, live && kk + h < k1 ? a[m][0] : z,
                              live && kk + h + 1 < k1 ? a[m][1] : z);
      }
    }
    __syncthreads();
    if (wave * 16 >= L) return;  // this wave's rows are all past the segment
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      const u32x4 xa = kk + s * 32 + q * 8 < k1 ? x[s] : z;  // ragged tail of H1
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = mfma<T>(xa, load_vec(&lds_at[(n * 16 + ml) * AST + (((4 * s + q) ^ swz(n * 16)) << 3)]), acc[n]);
    }
  };

  // Ping-pong over stage pairs: each buffer is waited for only where it is
  // consumed.  A stage past k1 loads clamped addresses and contributes zeros;
  // no loads are issued past the last stage pair (the stores below would
  // wait for them).
  u32x4 xA[MS], aA[NPAIR][2], xB[MS], aB[NPAIR][2];
  issue(k0, xA, aA);
  for (int kk = k0; kk < k1; kk += 2 * kKStage) {
    issue(kk + kKStage, xB, aB);
    compute(kk, xA, aA);
    if (kk + 2 * kKStage < k1) issue(kk + 2 * kKStage, xA, aA);
    compute(kk + kKStage, xB, aB);
  }

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

// ---------------------------------------------------------------- expand
// MT rows per tile.  MT = 64: wave w computes rows 16w..16w+15 over the whole
// chunk.  MT = 16 (short segments, e.g. decode batches with a few rows per
// LoRA): the four waves share the 16 rows and each computes a quarter of the
// chunk's columns, so no wave idles and the smaller LDS footprint lets more
// workgroups stream B_k at once.
template <class T, int R, bool EXT, int MT>
__global__ __launch_bounds__(kThreads) void sgmv_mfma_expand_kernel(MfmaParams p) {
  constexpr int K2 = 2 * R;            // virtual K: [V_hi | V_lo] against [B_k; B_k]
  constexpr int KSTEPS = K2 / 32;
  constexpr int WR = MT / 16;          // 16-row groups of the tile
  constexpr int WC = kWaves / WR;      // waves that share a row group, each on its own columns
  static_assert(WR * WC == kWaves, "tile rows are 16 or 64");
  constexpr int NTC = kCW / 16;        // 16-wide column tiles per chunk
  constexpr int NTW = NTC / WC;        // column tiles per wave
  constexpr int CV = kCW / 8;          // 128-bit column vectors per chunk row
  constexpr int CVW = CV / WC;         // ... of one wave's columns
  constexpr int BST = R + 8;           // LDS stride (halves) of transposed B_k, per column
  // Within a column, B_k's ranks sit in groups of 8 (one 128-bit MFMA operand
  // read); group g of column c is stored at group g ^ swz(c).  The transposed
  // stores of a wave then spread over the LDS banks (without the swizzle the
  // 16 lanes that write one rank pair of 16 column groups hit 2 banks), and
  // the operand reads stay conflict-free.
  constexpr int GMASK = R / 8 - 1;
  auto swz = [](int c) { return (c >> 4) & GMASK; };
  constexpr int VST = K2 + 8;          // LDS stride (halves) of [V_hi | V_lo], per row
  constexpr int OST = kCW / WC + 4;    // LDS stride (floats) of a wave's result tile
  constexpr int NBP = (R / 2 * CV + kThreads - 1) / kThreads;  // (j, j+1) B_k vector pairs per thread
  constexpr int NYV = 16 * CVW / 64;   // Y vectors per lane (16 rows of the wave's columns)
  __shared__ __attribute__((aligned(16))) uint16_t lds_bt[kCW * BST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[MT * VST];
  __shared__ __attribute__((aligned(16))) float lds_o[kWaves * 16 * OST];

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
                         (p.chunks_per_wg - 1) | (int32_t)(p.proj_stride >> 32)) < 0;
  const bool bad_ptr = (p.seg_indptr == nullptr) | (p.lora_idx == nullptr) | (p.V == nullptr) |
                       (pj.B_ptrs == nullptr) | (pj.Y == nullptr);
  if (bad_size | bad_ptr) return;
  const int nchunks = (p.h_out + kCW - 1) / kCW;
  const int ngroups = (nchunks + p.chunks_per_wg - 1) / p.chunks_per_wg;
  // Linear order: column group major, so the row units that read one slice of
  // B_k share an XCD.
  const int idx = xcd_linear_index();
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
      const int j = (pv / CV) * 2, c = c0 + (pv % CV) * 8;
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
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    const int o = (t + kThreads * m) * 4;
    const int rr = o / R;
    vv[m] = *reinterpret_cast<const f32x4*>(Vp + (int64_t)(r0 + (rr < L ? rr : 0)) * R + o % R);
  }
  u32x4 bvA[NBP][2], yvA[NYV], bvB[NBP][2], yvB[NYV];
  issue(ch0, bvA, yvA);
#pragma unroll
  for (int m = 0; m < NV4; ++m) {
    const int o = (t + kThreads * m) * 4;
    if (o < NVF * 4) {
      const int rr = o / R, j = o % R;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = rr < L ? vv[m][e] * sk : 0.f;
        const uint16_t hi = T::round(v);
        const uint16_t lo = T::round(v - T::one(hi));
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
        const int j = (pr / CV) * 2, cl = (pr % CV) * 8;
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
#pragma unroll
        for (int e = 0; e < 8; ++e) yf[e] += out[rl * OST + cl + e];
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
      if (ext)
        hipLaunchKernelGGL((sgmv_mfma_shrink_kernel<T, R, true>), dim3(grid, np), dim3(kThreads), 0, s, p);
      else
        hipLaunchKernelGGL((sgmv_mfma_shrink_kernel<T, R, false>), dim3(grid, np), dim3(kThreads), 0, s, p);
    }
  } else if (stage == 1) {
    constexpr unsigned rows = kThreads / (R / 4);
    grid = ((unsigned)p.n_rows + rows - 1) / rows;
    if (grid && np > 0) hipLaunchKernelGGL((sgmv_mfma_reduce_kernel<R>), dim3(grid, np), dim3(kThreads), 0, s, p);
  } else {
    if (p.expand_rows != 16 && p.expand_rows != kMT) return hipErrorInvalidValue;
    const int nchunks = (p.h_out + kCW - 1) / kCW;
    grid = xcd_grid((unsigned)p.num_units_x * (unsigned)((nchunks + p.chunks_per_wg - 1) / p.chunks_per_wg));
    if (grid && np > 0) {
      using K = void (*)(MfmaParams);
      // [short tiles][ext]
      static constexpr K kernels[2][2] = {
          {sgmv_mfma_expand_kernel<T, R, false, kMT>, sgmv_mfma_expand_kernel<T, R, true, kMT>},
          {sgmv_mfma_expand_kernel<T, R, false, 16>, sgmv_mfma_expand_kernel<T, R, true, 16>}};
      hipLaunchKernelGGL(kernels[p.expand_rows == 16][ext], dim3(grid, np), dim3(kThreads), 0, s, p);
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

bool mfma_supported(int rank) { return rank == 16 || rank == 32 || rank == 64; }

hipError_t launch_mfma_shrink(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream) {
  hipError_t e = launch_stage(dtype, rank, 0, p, num_proj, stream);
  if (e != hipSuccess) return e;
  return launch_stage(dtype, rank, 1, p, num_proj, stream);
}

hipError_t launch_mfma_expand(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream) {
  return launch_stage(dtype, rank, 2, p, num_proj, stream);
}

}  // namespace sgmv
