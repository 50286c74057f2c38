// sgmv_base.hip - base projection with the LoRA term added before its one
// rounding (gfx950), for decode-sized batches.
//
// The LoRA paragraph of the Punica README (page "Punica：多 LoRA 模型统一服务框架")
// gives a row vector x the output x@W + x@A@B; the multi-LoRA paragraph runs
// X@W once for the whole batch and adds every row's own LoRA term.  For at
// most 128 rows this file computes
//     Y[i, :] = X[i, :] @ W + V[i, :] @ B_k      (k: LoRA of row i's segment)
// with V = X @ A_k, the sum kept in fp32 and rounded once.  Rows no segment covers get X @ W.
//
// Two launches:
//  1. partials: workgroup (g, s) multiplies X[:, K_g] by W[K_g, strip s] (SC
//     columns) on the matrix cores and writes its tile of fp32 partial plane
//     g.  W (the bulk of the bytes) streams from HBM exactly once; X (n x h_in,
//     a few hundred KiB) is re-read from L2 by every strip.  Each stage of W
//     rows is staged in LDS transposed to [column][k], so that a lane reads 8
//     consecutive k of one column with one 128-bit read; the X stage is kept
//     row-major ([row][k]), which is already the MFMA operand layout.  Further
//     workgroups of the same launch compute the LoRA shrink, one fp32 partial
//     plane of V per K chunk (nothing in the launch waits for anything).
//  2. epilogue: one wave per (row, 512 columns) sums the partial planes of Y
//     and of V in plane order, adds V[i] @ B_k over its columns and stores Y.
#include "sgmv_device.h"
#include "sgmv_mfma_ops.h"
#include "sgmv_plan.h"

namespace sgmv {
namespace {

constexpr int kXcds = 8;

// ---------------------------------------------------------------- LoRA shrink
// Segment of row i (64 segments at a time; -1: none covers it).
__device__ inline int segment_of_row(const BaseParams& p, int i) {
  const int lane = threadIdx.x & 63;
  int seg = -1;
  if (p.num_segs > 0 && p.seg_indptr != nullptr && p.lora_idx != nullptr) {
    for (int s0 = 0; s0 < p.num_segs; s0 += 64) {
      const int s = s0 + lane;
      bool hit = false;
      if (s < p.num_segs) hit = p.seg_indptr[s] <= i && i < p.seg_indptr[s + 1];
      const unsigned long long m = __ballot(hit);
      if (m) {
        seg = s0 + __builtin_ctzll(m);
        break;
      }
    }
  }
  return __builtin_amdgcn_readfirstlane(seg);
}

// Workgroup (i, g) of the shrink role: partial V plane g of row i,
//   vpart[g][i][j] = sum_{h in K_g} X[i, h] * A_k[h, j],
// in fp32 with vector FMA (each row may use its own LoRA, so this is not a
// shared-operand product).  Thread t owns 8 ranks (group t % JG) of the rows
// h = t / JG + HPT m; one round of loads covers HPT * kUnroll = 512 rows.  The
// threads of one rank group are summed by a butterfly within each wave, then
// the four waves in wave order through LDS (a fixed order).
template <class T, int R>
__device__ inline void shrink_role(const BaseParams& p, int item, float* lds) {
  constexpr int JG = R / 8;               // 128-bit vectors per row of A_k
  constexpr int HPT = kThreads / JG;      // rows of A_k per load of the workgroup
  constexpr int kUnroll = 512 / HPT;      // loads per thread per round
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int i = item / p.ksplit;
  const int g = item - i * p.ksplit;
  if (i >= p.n_rows) return;  // padding of the shrink grid to a multiple of 8
  const int seg = segment_of_row(p, i);
  const int k = seg >= 0 ? p.lora_idx[seg] : -1;
  const bool lora = k >= 0 && k < p.num_loras && p.A_ptrs != nullptr && p.B_ptrs != nullptr;
  // Workgroup (i, 0) records row i's B_k (0: no LoRA term) for the epilogue.
  if (g == 0 && t == 0 && p.row_b != nullptr) p.row_b[i] = lora ? p.B_ptrs[k] : 0ull;
  if (!lora) return;
  const uint16_t* Ak = reinterpret_cast<const uint16_t*>(p.A_ptrs[k]);
  const uint16_t* xrow = p.X + (int64_t)i * p.h_in;
  const int k0 = g * p.kc;
  const int k1 = p.h_in < k0 + p.kc ? p.h_in : k0 + p.kc;
  const int jg = t % JG, h0 = t / JG;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int hb = k0 + h0; hb < k1; hb += HPT * kUnroll) {
    u32x4 a[kUnroll];
    uint16_t xb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int h = hb + u * HPT;
      const bool ok = h < k1;
      a[u] = load_stream(Ak + (ok ? (int64_t)h * R + jg * 8 : 0));
      xb[u] = load_stream_u16(xrow + (ok ? h : 0));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float x = hb + u * HPT < k1 ? T::one(xb[u]) : 0.f;
      float af[8];
      unpack8<T>(a[u], af);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(x, af[e], acc[e]);
    }
  }
  // Butterfly over the lanes of one rank group (lanes jg + JG m of the wave).
#pragma unroll
  for (int mask = JG; mask < 64; mask <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += shfl_xor(acc[e], mask);
  if (lane < JG)
#pragma unroll
    for (int e = 0; e < 8; ++e) lds[(wave * JG + lane) * 8 + e] = acc[e];
  __syncthreads();
  if (t < R) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += lds[w * R + t];
    p.vpartials[((int64_t)g * p.n_rows + i) * R + t] = v;
  }
}

// ---------------------------------------------------------------- partials
// Workgroup (g, s): rows of X and W [K_g] x strip s of SC columns, on the
// matrix cores; writes its tile of fp32 partial plane g.
template <class T, int R, int SC, int NRT>
__global__ __launch_bounds__(kThreads) void sgmv_base_partial_kernel(BaseParams p) {
  constexpr int KS = kBaseStageRows;    // W rows per stage
  constexpr int WST = KS + 8;           // LDS stride (halves) of transposed W, per column
  constexpr int XST = KS + 8;           // LDS stride (halves) of the X stage, per row
  constexpr int CV = SC / 8;            // 128-bit vectors per W row of the strip
  constexpr int NWP = KS / 2 * CV / kThreads;        // (k, k+1) W vector pairs per thread
  constexpr int XV = KS / 8;            // 128-bit vectors per X row of a stage
  constexpr int NXV = (NRT * 16 * XV + kThreads - 1) / kThreads;  // X vectors per thread
  constexpr int KSTEPS = KS / 32;       // MFMA k-steps per stage
  constexpr int NTW = SC / 16 / kWaves; // 16-column tiles per wave
  static_assert(NWP * kThreads == KS / 2 * CV, "W stage splits evenly over the threads");
  static_assert(NTW * 16 * kWaves == SC, "strip splits evenly over the waves");
  // Within a column, the stage's k sit in groups of 8 (one 128-bit operand
  // read); group g of column c is stored at group g ^ swz(c), which spreads a
  // wave's transposed stores over the LDS banks.
  auto swz = [](int c) { return (c >> 4) & (KS / 8 - 1); };
  __shared__ __attribute__((aligned(16))) uint16_t lds_wt[SC * WST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[NRT * 16 * XST];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int q = lane >> 4;
  const int ml = lane & 15;
  // A malformed launch returns at once (the host rejects all of these).
  const bool bad = ((p.n_rows - 1) | p.h_in | p.h_out | (p.kc - 1) | (p.strips - 1) | (p.ksplit - 1) |
                    (NRT * 16 - p.n_rows) | (int32_t)(p.plane_stride >> 32)) < 0;
  const bool bad_ptr = (p.X == nullptr) | (p.W == nullptr) | (p.partials == nullptr);
  if (bad | bad_ptr) return;
  // The first shrink_grid workgroups compute the LoRA shrink (dispatched
  // first, they finish while W streams).
  if ((int)blockIdx.x < p.shrink_grid) {
    if (p.vpartials != nullptr) shrink_role<T, R>(p, (int)blockIdx.x, reinterpret_cast<float*>(lds_wt));
    return;
  }
  // Linear order of the base product: K split major; each XCD (workgroup b
  // runs on XCD b % 8; shrink_grid is a multiple of 8) takes a contiguous run
  // of it, so the strips that read one chunk of X share an L2.
  const int b = (int)blockIdx.x - p.shrink_grid;
  const int per_xcd = p.base_grid / kXcds;
  const int idx = (b % kXcds) * per_xcd + b / kXcds;
  if (idx >= p.strips * p.ksplit) return;
  const int g = idx / p.strips;
  const int c0 = (idx - g * p.strips) * SC;
  const int n = p.n_rows;
  const int k0 = g * p.kc;
  const int k1 = p.h_in < k0 + p.kc ? p.h_in : k0 + p.kc;
  const uint16_t* W = p.W;
  const uint16_t* X = p.X;

  // All loads of one stage, at clamped (valid) addresses; what lies past the
  // matrix is zeroed where it is staged.
  auto issue = [&](int kk, u32x4 (&w)[NWP][2], u32x4 (&x)[NXV]) {
#pragma unroll
    for (int m = 0; m < NWP; ++m) {
      const int pv = t + kThreads * m;
      const int k = kk + (pv / CV) * 2, c = c0 + (pv % CV) * 8;
      const bool ok = c < p.h_out;
      w[m][0] = load_stream(W + (ok && k < k1 ? (int64_t)k * p.h_out + c : 0));
      w[m][1] = load_stream(W + (ok && k + 1 < k1 ? (int64_t)(k + 1) * p.h_out + c : 0));
    }
#pragma unroll
    for (int m = 0; m < NXV; ++m) {
      const int xv = t + kThreads * m;
      const int r = xv / XV, k = kk + (xv % XV) * 8;
      x[m] = load_vec(X + (r < n && k < k1 ? (int64_t)r * p.h_in + k : 0));
    }
  };

  f32x4 acc[NRT][NTW];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kk, const u32x4 (&w)[NWP][2], const u32x4 (&x)[NXV]) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    __syncthreads();  // the previous stage is done with the LDS tiles
#pragma unroll
    for (int m = 0; m < NWP; ++m) {
      const int pv = t + kThreads * m;
      const int kr = (pv / CV) * 2, cl = (pv % CV) * 8;
      const bool ok = c0 + cl < p.h_out;
      const int ks = (((kr >> 3) ^ swz(cl)) << 3) | (kr & 7);  // columns cl..cl+7 share swz(cl)
      store_pair_transposed(&lds_wt[cl * WST + ks], WST, ok && kk + kr < k1 ? w[m][0] : z,
                            ok && kk + kr + 1 < k1 ? w[m][1] : z);
    }
#pragma unroll
    for (int m = 0; m < NXV; ++m) {
      const int xv = t + kThreads * m;
      const int r = xv / XV, kx = (xv % XV) * 8;
      if (r < NRT * 16) store_vec(&lds_x[r * XST + kx], r < n && kk + kx < k1 ? x[m] : z);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      u32x4 bf[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int cn = (wave * NTW + j) * 16;  // first column of the tile
        bf[j] = load_vec(&lds_wt[(cn + ml) * WST + (((4 * s + q) ^ swz(cn)) << 3)]);
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const u32x4 af = load_vec(&lds_x[(rt * 16 + ml) * XST + s * 32 + q * 8]);
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[rt][j] = mfma<T>(af, bf[j], acc[rt][j]);
      }
    }
  };

  // Ping-pong over stage pairs; a stage past k1 loads clamped addresses and
  // contributes zeros.  The loop body issues its loads unconditionally (a
  // load under a branch makes the compiler wait for every load in flight,
  // the next stage's included, before the current stage is used); the last
  // stage pair, which issues nothing beyond itself, is peeled.
  u32x4 wA[NWP][2], xA[NXV], wB[NWP][2], xB[NXV];
  issue(k0, wA, xA);
  int kk = k0;
  for (; kk + 2 * KS < k1; kk += 2 * KS) {
    issue(kk + KS, wB, xB);
    compute(kk, wA, xA);
    issue(kk + 2 * KS, wA, xA);
    compute(kk + KS, wB, xB);
  }
  issue(kk + KS, wB, xB);
  compute(kk, wA, xA);
  compute(kk + KS, wB, xB);

  // D[4q+i][ml] of tile (rt, j): row rt*16 + 4q + i, column c0 + (wave*NTW + j)*16 + ml.
  float* dst = p.partials + (int64_t)g * p.plane_stride;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + q * 4 + i;
        const int c = c0 + (wave * NTW + j) * 16 + ml;
        if (r < n && c < p.h_out) dst[(int64_t)r * p.h_out + c] = acc[rt][j][i];
      }
}

// ---------------------------------------------------------------- packed W
// The packed layout of W [h_in, h_out] holds, for 16-column block nb and
// 32-row k-step ks, one 1 KiB block at element (nb * kst + ks) * 512, with
// kst = ceil(h_in / 128) * 4 k-steps per column block.  Inside the block, the
// 8 elements at lane L = 16 q + m are W[32 ks + 8 q + e][16 nb + m], e = 0..7:
// the B operand of one 16x16x32 MFMA, so a wave reads it with one fully
// coalesced 128-bit load per lane.  Column blocks run to an even count;
// entries past the matrix are zero.
__global__ __launch_bounds__(64) void sgmv_base_pack_kernel(const uint16_t* __restrict__ W, int h_in,
                                                            int h_out, int kst, uint16_t* __restrict__ Wp) {
  const int ks = blockIdx.x, nb = blockIdx.y, lane = threadIdx.x;
  const int q = lane >> 4, m = lane & 15;
  const int c = nb * 16 + m;
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = ks * 32 + q * 8 + e;
    v[e] = c < h_out && k < h_in ? W[(int64_t)k * h_out + c] : (uint16_t)0;
  }
  u32x4 o;
#pragma unroll
  for (int w = 0; w < 4; ++w) o[w] = (uint32_t)v[2 * w] | ((uint32_t)v[2 * w + 1] << 16);
  store_vec(Wp + ((int64_t)nb * kst + ks) * 512 + lane * 8, o);
}

// Workgroup (g, s) as in sgmv_base_partial_kernel, from the packed W: wave w
// owns column blocks 8 s + 2 w and 8 s + 2 w + 1 over K chunk g and feeds the
// matrix cores straight from its W loads.  A ring of S register sets of D
// k-steps: S - 1 sets are in flight while one is multiplied.  X operands:
//  - up to two row tiles: each wave loads them from L2 with its W (no LDS,
//    no barrier);
//  - four or eight row tiles (XL): the workgroup's X chunk ([64 or 128
//    rows][kc], at most 64 or 128 KiB) is staged in LDS once, behind one barrier, its 16-byte groups at
//    group ^ (row & 7) within a row so that the 16 rows of one operand read
//    fall on different banks.  Four operand loads per k-step from L2 would
//    outnumber the two of W.
template <class T, int R, int NRT>
__global__ __launch_bounds__(kThreads) void sgmv_base_packed_kernel(BaseParams p) {
  constexpr int D = 4;  // k-steps per register set (kst and the chunk are multiples of 4)
  constexpr int S = 2;  // register sets (three measured slower)
  constexpr bool XL = NRT > 2;
  constexpr int NX = XL ? 0 : NRT;  // X operands per k-step held in the ring
  constexpr int XE = base_packed_x_elems(NRT * 16);
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[XL ? XE : kWaves * 128];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int q = lane >> 4;
  const int ml = lane & 15;
  const int kst = p.packed_ksteps;
  const bool bad = ((p.n_rows - 1) | p.h_in | p.h_out | (p.kc - 1) | (p.strips - 1) | (p.ksplit - 1) |
                    (kst - 1) | (NRT * 16 - p.n_rows) | (XL ? XE - NRT * 16 * p.kc : 0) |
                    (int32_t)(p.plane_stride >> 32)) < 0;
  const bool bad_ptr = (p.X == nullptr) | (p.W == nullptr) | (p.partials == nullptr);
  if (bad | bad_ptr) return;
  if ((int)blockIdx.x < p.shrink_grid) {
    if (p.vpartials != nullptr) shrink_role<T, R>(p, (int)blockIdx.x, reinterpret_cast<float*>(lds_x));
    return;
  }
  const int b = (int)blockIdx.x - p.shrink_grid;
  const int per_xcd = p.base_grid / kXcds;
  const int idx = (b % kXcds) * per_xcd + b / kXcds;
  if (idx >= p.strips * p.ksplit) return;  // the whole workgroup
  const int g = idx / p.strips;
  const int nb0 = __builtin_amdgcn_readfirstlane((idx - g * p.strips) * 8 + wave * 2);
  const bool active = nb0 * 16 < p.h_out;  // whole waves; inactive ones still stage X
  const int ks0 = g * (p.kc / 32);
  const int ks1 = kst < ks0 + p.kc / 32 ? kst : ks0 + p.kc / 32;
  const int nk = (ks1 - ks0) * 32;  // k of this chunk (a multiple of 128)
  const int n = p.n_rows;
  const uint16_t* Wb = p.W + (int64_t)nb0 * kst * 512;
  const uint32_t wlane = (uint32_t)lane * 8, wnext = (uint32_t)kst * 512;

  uint32_t xoff[NRT];
  bool xrow[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = rt * 16 + ml;
    xrow[rt] = r < n;
    xoff[rt] = (uint32_t)((r < n ? r : 0) * p.h_in + q * 8);
  }
  auto issue = [&](int ks, u32x4 (&w)[D][2], u32x4 (&x)[D][NX > 0 ? NX : 1]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const uint32_t o = (uint32_t)(ks + d) * 512 + wlane;
      w[d][0] = load_stream(Wb + o);
      w[d][1] = load_stream(Wb + o + wnext);
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int rt = 0; rt < NX; ++rt) {
        const bool ok = xrow[rt] && (ks + d) * 32 + q * 8 < p.h_in;
        x[d][rt] = load_vec(p.X + (ok ? xoff[rt] + (uint32_t)(ks + d) * 32 : 0u));
        if (!ok) x[d][rt] = u32x4{0u, 0u, 0u, 0u};
      }
  };
  u32x4 w[S][D][2], x[S][D][NX > 0 ? NX : 1];
  if (active) {
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      if (ks0 + i * D < ks1) issue(ks0 + i * D, w[i], x[i]);
  }

  // Stage X[0 .. NRT*16)[k0 .. k0 + nk) (zero past n rows or h_in), 8 vectors
  // of 16 bytes per thread per round.
  if constexpr (XL) {
    const int k0 = ks0 * 32;
    const int gpr = nk / 8;  // 16-byte groups per row
    const int total = NRT * 16 * gpr;
    for (int v0 = 0; v0 < total; v0 += kThreads * 8) {
      u32x4 xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = v0 + u * kThreads + t;
        const int r = v / gpr, gi = v - r * gpr;
        const bool ok = v < total && r < n && k0 + gi * 8 < p.h_in;
        xv[u] = load_vec(p.X + (ok ? (int64_t)r * p.h_in + k0 + gi * 8 : 0));
        if (!ok) xv[u] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = v0 + u * kThreads + t;
        const int r = v / gpr, gi = v - r * gpr;
        if (v < total) store_vec(&lds_x[r * nk + ((gi ^ (r & 7)) << 3)], xv[u]);
      }
    }
  }
  if constexpr (XL) __syncthreads();
  if (!active) return;  // no barrier follows

  f32x4 acc[NRT][2];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int ks, const u32x4 (&wv)[D][2], const u32x4 (&xv)[D][NX > 0 ? NX : 1]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int gi = (ks - ks0 + d) * 4 + q;  // 16-byte group of this lane's 8 k
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int r = rt * 16 + ml;
        u32x4 af;
        if constexpr (XL)
          af = load_vec(&lds_x[r * nk + ((gi ^ (r & 7)) << 3)]);
        else
          af = xv[d][rt < NX ? rt : 0];
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[rt][j] = mfma<T>(af, wv[d][j], acc[rt][j]);
      }
    }
  };

  for (int ks = ks0; ks < ks1; ks += S * D) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      // Set (i + S - 1) % S was multiplied in the previous turn: refill it
      // with the step S - 1 sets ahead, then multiply set i.
      const int cur = ks + i * D, nxt = cur + (S - 1) * D;
      if (nxt < ks1) issue(nxt, w[(i + S - 1) % S], x[(i + S - 1) % S]);
      if (cur < ks1) mma(cur, w[i], x[i]);
    }
  }

  // D[4q+i][ml] of tile (rt, j): row rt*16 + 4q + i, column 16 (nb0 + j) + ml.
  float* dst = p.partials + (int64_t)g * p.plane_stride;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + q * 4 + i;
        const int c = (nb0 + j) * 16 + ml;
        if (r < n && c < p.h_out) dst[(int64_t)r * p.h_out + c] = acc[rt][j][i];
      }
}

// ---------------------------------------------------------------- epilogue
// One wave per (row i, 512 columns): lane l owns columns c .. c+7,
// c = 512 * blockIdx.x + 8 * l.  Y[i, c..] = sum of the partial planes (plane
// order) + V[i] @ B_k (ranks in ascending order), rounded once.
template <class T, int R>
__global__ __launch_bounds__(64) void sgmv_base_epilogue_kernel(BaseParams p) {
  constexpr int kBatch = 8;   // plane loads in flight per lane
  const int lane = threadIdx.x;
  const int i = blockIdx.y;
  const bool bad = (p.n_rows | p.h_out | p.num_segs | p.num_loras | (p.ksplit - 1) |
                    (int32_t)(p.plane_stride >> 32)) < 0;
  const bool bad_ptr = (p.partials == nullptr) | (p.Y == nullptr && p.Yf == nullptr);
  if (bad | bad_ptr || i >= p.n_rows) return;
  const int c = blockIdx.x * 512 + lane * 8;
  const bool col_ok = c < p.h_out;
  const int cc = col_ok ? c : 0;

  // Everything this wave needs that depends only on the row is fetched in one
  // round: row i's B_k (recorded by the shrink), the partial planes of V
  // (lane j < R: rank j) and the partial planes of Y (up to kBatch planes).
  const bool lora_planes = p.vpartials != nullptr && p.row_b != nullptr;
  const uint64_t bptr = lora_planes ? p.row_b[i] : 0ull;
  float pv[kBatch];
  const float* vp = lora_planes ? p.vpartials + (int64_t)i * R + (lane < R ? lane : 0) : nullptr;
  if (lora_planes) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int g = u < p.ksplit ? u : p.ksplit - 1;
      pv[u] = vp[(int64_t)g * p.n_rows * R];
    }
  }
  const float* row = p.partials + (int64_t)i * p.h_out + cc;
  f32x4 a[kBatch], b[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int g = u < p.ksplit ? u : p.ksplit - 1;
    a[u] = *reinterpret_cast<const f32x4*>(row + (int64_t)g * p.plane_stride);
    b[u] = *reinterpret_cast<const f32x4*>(row + (int64_t)g * p.plane_stride + 4);
  }
  const bool lora = bptr != 0ull;

  constexpr int JB = R < 16 ? R : 16;  // B_k rows per batch of loads
  const uint16_t* Bk = reinterpret_cast<const uint16_t*>(bptr);
  u32x4 bv[JB];
  if (lora) {
#pragma unroll
    for (int j = 0; j < JB; ++j) bv[j] = load_stream(Bk + (int64_t)j * p.h_out + cc);
  }
  // V[i] = sum of its partial planes in plane order (lane j < R owns rank j),
  // shared through LDS.
  __shared__ float lds_v[R];
  if (lora && lane < R) {
    float v = 0.f;
    for (int g0 = 0; g0 < p.ksplit; g0 += kBatch) {
      if (g0 > 0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int g = g0 + u < p.ksplit ? g0 + u : p.ksplit - 1;
          pv[u] = vp[(int64_t)g * p.n_rows * R];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v = g0 + u < p.ksplit ? v + pv[u] : v;
    }
    lds_v[lane] = v;
  }
  __syncthreads();

  // Base: sum of the partial planes in plane order.
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int g0 = 0; g0 < p.ksplit; g0 += kBatch) {
    if (g0 > 0) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int g = g0 + u < p.ksplit ? g0 + u : p.ksplit - 1;
        a[u] = *reinterpret_cast<const f32x4*>(row + (int64_t)g * p.plane_stride);
        b[u] = *reinterpret_cast<const f32x4*>(row + (int64_t)g * p.plane_stride + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool live = g0 + u < p.ksplit;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = live ? y[e] + a[u][e] : y[e];
        y[4 + e] = live ? y[4 + e] + b[u][e] : y[4 + e];
      }
    }
  }
  if (lora) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j0 = 0; j0 < R; j0 += JB) {
      if (j0 > 0) {
#pragma unroll
        for (int j = 0; j < JB; ++j) bv[j] = load_stream(Bk + (int64_t)(j0 + j) * p.h_out + cc);
      }
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        float bf[8];
        unpack8<T>(bv[j], bf);
        const float vj = lds_v[j0 + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = __builtin_fmaf(vj, bf[e], s[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] += s[e];
  }
  if (!col_ok) return;
  if (p.Yf != nullptr) {
    // A shard's partial output: fp32, unrounded (summed across shards, then
    // rounded once, by the caller).
    float* yf = p.Yf + (int64_t)i * p.h_out + c;
    *reinterpret_cast<f32x4*>(yf) = f32x4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4*>(yf + 4) = f32x4{y[4], y[5], y[6], y[7]};
  } else {
    store_vec(p.Y + (int64_t)i * p.h_out + c, pack8<T>(y));
  }
}

// Grid: shrink_grid shrink workgroups (n_rows * ksplit rounded up to a
// multiple of 8; none without a LoRA term), then the base product's
// workgroups (a multiple of 8, for the XCD mapping).
template <class T, int R, int SC>
hipError_t launch_partial(const BaseParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.shrink_grid + (unsigned)p.base_grid);
  if (p.n_rows <= 16)
    hipLaunchKernelGGL((sgmv_base_partial_kernel<T, R, SC, 1>), grid, dim3(kThreads), 0, s, p);
  else if (p.n_rows <= 32)
    hipLaunchKernelGGL((sgmv_base_partial_kernel<T, R, SC, 2>), grid, dim3(kThreads), 0, s, p);
  else if (p.n_rows <= 64)
    hipLaunchKernelGGL((sgmv_base_partial_kernel<T, R, SC, 4>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((sgmv_base_partial_kernel<T, R, SC, 8>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <class T, int R>
hipError_t launch_packed(const BaseParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.shrink_grid + (unsigned)p.base_grid);
  if (p.n_rows <= 16)
    hipLaunchKernelGGL((sgmv_base_packed_kernel<T, R, 1>), grid, dim3(kThreads), 0, s, p);
  else if (p.n_rows <= 32)
    hipLaunchKernelGGL((sgmv_base_packed_kernel<T, R, 2>), grid, dim3(kThreads), 0, s, p);
  else if (p.n_rows <= 64)
    hipLaunchKernelGGL((sgmv_base_packed_kernel<T, R, 4>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((sgmv_base_packed_kernel<T, R, 8>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <class T, int R>
hipError_t launch_r(const BaseParams& p, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  if (p.packed_ksteps > 0) {
    if (p.strip_cols == 128) e = launch_packed<T, R>(p, s);
  } else {
    switch (p.strip_cols) {
      case 64: e = launch_partial<T, R, 64>(p, s); break;
      case 128: e = launch_partial<T, R, 128>(p, s); break;
      case 256: e = launch_partial<T, R, 256>(p, s); break;
    }
  }
  if (e != hipSuccess) return e;
  const dim3 egrid((unsigned)((p.h_out + 511) / 512), (unsigned)p.n_rows);
  hipLaunchKernelGGL((sgmv_base_epilogue_kernel<T, R>), egrid, dim3(64), 0, s, p);
  return hipGetLastError();
}

template <class T>
hipError_t launch_t(int rank, const BaseParams& p, hipStream_t s) {
  switch (rank) {
    case 8: return launch_r<T, 8>(p, s);
    case 16: return launch_r<T, 16>(p, s);
    case 32: return launch_r<T, 32>(p, s);
    case 64: return launch_r<T, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_base_pack(const uint16_t* W, int h_in, int h_out, uint16_t* Wp, hipStream_t stream) {
  if (h_in <= 0 || h_out <= 0) return hipErrorInvalidValue;
  const int kst = (h_in + 127) / 128 * 4;
  const int nbp = ((h_out + 15) / 16 + 1) / 2 * 2;
  hipLaunchKernelGGL(sgmv_base_pack_kernel, dim3((unsigned)kst, (unsigned)nbp), dim3(64), 0, stream, W, h_in,
                     h_out, kst, Wp);
  return hipGetLastError();
}

hipError_t launch_base(int dtype, int rank, const BaseParams& p, hipStream_t stream) {
  if (p.n_rows <= 0 || p.strips <= 0) return hipSuccess;
  if (p.n_rows > kBaseMaxRows) return hipErrorInvalidValue;
  return dtype == 1 ? launch_t<BF16>(rank, p, stream) : launch_t<F16>(rank, p, stream);
}

}  // namespace sgmv
