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
// Shrink: a workgroup (4 waves) takes a 64-row tile of one segment and a
// chunk of H1.  A_k is staged through LDS transposed ([r][h], so a lane reads
// its 8 consecutive h of one rank with one 128-bit LDS read); X fragments go
// straight from HBM into registers.  With several H1 chunks, each writes its
// own fp32 partial [n_rows, r]; the expand sums them in a fixed order.
//
// Expand: a workgroup takes a 64-row tile and 128 output columns.  V is split
// into V_hi + V_lo (both in the input format), which the MFMA consumes as a
// K dimension of 2r against [B_k; B_k], keeping ~2x the input format's
// significand bits of V.  B_k is staged transposed in LDS ([c][j]); the
// result tile goes through LDS so that Y is read and written with 128-bit
// accesses (Y is prefetched before the MFMA work).
#include "sgmv_device.h"
#include "sgmv_plan.h"
#include "sgmv_units.h"

namespace sgmv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMT = kMfmaRowsPerTile;  // 64 rows per tile: 16 per wave
constexpr int kKSub = 256;             // A_k rows staged per sub-chunk (shrink)
constexpr int kCW = kMfmaColsPerTile;  // 128 output columns per expand workgroup

template <class T>
__device__ inline f32x4 mfma(const u32x4& a, const u32x4& b, f32x4 c);
template <>
__device__ inline f32x4 mfma<F16>(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}
template <>
__device__ inline f32x4 mfma<BF16>(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

template <class T>
__device__ inline float widen(uint16_t b) {
  return T::one(b);
}

// ---------------------------------------------------------------- shrink
template <class T, int R>
__global__ __launch_bounds__(kThreads) void sgmv_mfma_shrink_kernel(MfmaParams p) {
  constexpr int NT = R / 16;                   // 16-wide rank tiles
  constexpr int JG = R / 8;                    // 128-bit vectors per row of A_k
  constexpr int NAV = kKSub * JG / kThreads;   // A_k vectors per thread per sub-chunk
  constexpr int KSTEPS = kKSub / 32;           // MFMA k-steps per sub-chunk
  constexpr int AST = kKSub + 8;               // LDS row stride (halves) of transposed A_k
  __shared__ __attribute__((aligned(16))) uint16_t lds_at[R * AST];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int q = lane >> 4;   // k-group of the lane (8 k each)
  const int ml = lane & 15;  // row (A operand) / rank column (B operand) of the lane
  const int KS = p.ksplit;
  const int unit = blockIdx.x / KS;
  const int g = blockIdx.x - unit * KS;
  const Unit un = resolve_unit<kMT>(p.seg_indptr, p.lora_idx, p.num_segs, p.num_loras, p.n_rows,
                                    p.direct_units, unit);
  if (un.L <= 0) return;
  const int L = un.L, r0 = un.r0;
  const uint16_t* Ak = reinterpret_cast<const uint16_t*>(p.A_ptrs[un.k]);
  const int k0 = g * p.kc;
  const int k1 = p.h_in < k0 + p.kc ? p.h_in : k0 + p.kc;

  const int row = wave * 16 + ml;  // this lane's row of the tile (A operand)
  const uint16_t* xrow = p.X + (int64_t)(r0 + (row < L ? row : L - 1)) * p.h_in;

  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kk = k0; kk < k1; kk += kKSub) {
    const int nk = k1 - kk < kKSub ? k1 - kk : kKSub;  // multiple of 8
    // Loads of this sub-chunk: A_k rows [kk, kk+nk) and this lane's X fragments.
    u32x4 av[NAV];
#pragma unroll
    for (int m = 0; m < NAV; ++m) {
      const int v = t + kThreads * m;
      const int h = v / JG;
      av[m] = load_stream(Ak + (h < nk ? (int64_t)(kk + h) * R + (v % JG) * 8 : 0));
    }
    u32x4 xf[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int h = kk + s * 32 + q * 8;
      xf[s] = load_stream(xrow + (h < k1 ? h : 0));
    }
    __syncthreads();  // the previous sub-chunk is done with lds_at
#pragma unroll
    for (int m = 0; m < NAV; ++m) {
      const int v = t + kThreads * m;
      const int h = v / JG, jg = v % JG;
      const bool ok = h < nk;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t word = ok ? av[m][w] : 0u;
        lds_at[(jg * 8 + 2 * w) * AST + h] = (uint16_t)(word & 0xffffu);
        lds_at[(jg * 8 + 2 * w + 1) * AST + h] = (uint16_t)(word >> 16);
      }
    }
    __syncthreads();
    const int steps = (nk + 31) / 32;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (s < steps) {
        u32x4 a = xf[s];
        if (kk + s * 32 + q * 8 >= k1) a = u32x4{0u, 0u, 0u, 0u};  // ragged tail of H1
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const u32x4 b = load_vec(&lds_at[(n * 16 + ml) * AST + s * 32 + q * 8]);
          acc[n] = mfma<T>(a, b, acc[n]);
        }
      }
    }
  }

  // D[4q+i][ml] of rank tile n: row wave*16 + 4q + i, rank n*16 + ml.
  float* dst = p.V + (int64_t)g * p.partial_stride;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = wave * 16 + q * 4 + i;
      if (rr < L) dst[(int64_t)(r0 + rr) * R + n * 16 + ml] = acc[n][i];
    }
}

// ---------------------------------------------------------------- expand
template <class T, int R>
__global__ __launch_bounds__(kThreads) void sgmv_mfma_expand_kernel(MfmaParams p) {
  constexpr int K2 = 2 * R;           // virtual K: [V_hi | V_lo] against [B_k; B_k]
  constexpr int KSTEPS = K2 / 32;
  constexpr int NTC = kCW / 16;       // 16-wide column tiles per wave
  constexpr int BST = R + 8;          // LDS stride (halves) of transposed B_k, per column
  constexpr int VST = K2 + 8;         // LDS stride (halves) of [V_hi | V_lo], per row
  constexpr int OST = kCW + 4;        // LDS stride (floats) of the result tile
  constexpr int NBV = R * (kCW / 8) / kThreads;  // B_k vectors per thread
  constexpr int NYV = 16 * (kCW / 8) / 64;       // Y vectors per lane (16 rows of the wave)
  static_assert(NBV >= 1 && NYV >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t lds_bt[kCW * BST];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kMT * VST];
  __shared__ __attribute__((aligned(16))) float lds_o[kWaves * 16 * OST];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int q = lane >> 4;
  const int ml = lane & 15;
  const int nchunks = (p.h_out + kCW - 1) / kCW;
  const int unit = blockIdx.x / nchunks;
  const int cc = blockIdx.x - unit * nchunks;
  const Unit un = resolve_unit<kMT>(p.seg_indptr, p.lora_idx, p.num_segs, p.num_loras, p.n_rows,
                                    p.direct_units, unit);
  if (un.L <= 0) return;
  const int L = un.L, r0 = un.r0;
  const int c0 = cc * kCW;
  const uint16_t* Bk = reinterpret_cast<const uint16_t*>(p.B_ptrs[un.k]);

  // Y of this wave's 16 rows: vector u -> (row, 8-column group), fetched first.
  u32x4 yv[NYV];
#pragma unroll
  for (int u = 0; u < NYV; ++u) {
    const int v = lane + 64 * u;
    const int rr = wave * 16 + v / (kCW / 8);
    const int c = c0 + (v % (kCW / 8)) * 8;
    const bool ok = rr < L && c < p.h_out;
    yv[u] = load_stream(p.Y + (int64_t)r0 * p.h_out + (ok ? (int64_t)rr * p.h_out + c : 0));
  }
  u32x4 bv[NBV];
#pragma unroll
  for (int m = 0; m < NBV; ++m) {
    const int v = t + kThreads * m;
    const int j = v / (kCW / 8);
    const int c = c0 + (v % (kCW / 8)) * 8;
    bv[m] = load_stream(Bk + (c < p.h_out ? (int64_t)j * p.h_out + c : 0));
  }
  // V of the tile rows (sum of the shrink's split partials, fixed order), split hi/lo.
  for (int o = t; o < kMT * R; o += kThreads) {
    const int rr = o / R, j = o % R;
    float v = 0.f;
    if (rr < L)
      for (int s = 0; s < p.ksplit; ++s) v += p.V[(int64_t)s * p.partial_stride + (int64_t)(r0 + rr) * R + j];
    const uint16_t hi = T::round(v);
    const uint16_t lo = T::round(v - widen<T>(hi));
    lds_v[rr * VST + j] = hi;
    lds_v[rr * VST + R + j] = lo;
  }
#pragma unroll
  for (int m = 0; m < NBV; ++m) {
    const int v = t + kThreads * m;
    const int j = v / (kCW / 8);
    const int cl = (v % (kCW / 8)) * 8;
    const bool ok = c0 + cl < p.h_out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t word = ok ? bv[m][w] : 0u;
      lds_bt[(cl + 2 * w) * BST + j] = (uint16_t)(word & 0xffffu);
      lds_bt[(cl + 2 * w + 1) * BST + j] = (uint16_t)(word >> 16);
    }
  }
  __syncthreads();

  u32x4 af[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) af[s] = load_vec(&lds_v[(wave * 16 + ml) * VST + s * 32 + q * 8]);
  float* out = lds_o + wave * 16 * OST;
#pragma unroll
  for (int n = 0; n < NTC; ++n) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int kb = (s * 32 + q * 8) % R;  // rank of the B_k copy this k-group reads
      const u32x4 b = load_vec(&lds_bt[(n * 16 + ml) * BST + kb]);
      acc = mfma<T>(af[s], b, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(q * 4 + i) * OST + n * 16 + ml] = acc[i];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NYV; ++u) {
    const int v = lane + 64 * u;
    const int rl = v / (kCW / 8);
    const int cl = (v % (kCW / 8)) * 8;
    const int rr = wave * 16 + rl;
    if (rr < L && c0 + cl < p.h_out) {
      float yf[8];
      unpack8<T>(yv[u], yf);
#pragma unroll
      for (int e = 0; e < 8; ++e) yf[e] += out[rl * OST + cl + e];
      store_vec(p.Y + (int64_t)(r0 + rr) * p.h_out + c0 + cl, pack8<T>(yf));
    }
  }
}

template <class T, int R>
hipError_t launch_t(int stage, const MfmaParams& p, hipStream_t s) {
  if (stage == 0) {
    const unsigned grid = (unsigned)p.num_units * (unsigned)p.ksplit;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((sgmv_mfma_shrink_kernel<T, R>), dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    const unsigned grid = (unsigned)p.num_units * (unsigned)((p.h_out + kCW - 1) / kCW);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((sgmv_mfma_expand_kernel<T, R>), dim3(grid), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

template <class T>
hipError_t launch_rank(int rank, int stage, const MfmaParams& p, hipStream_t s) {
  switch (rank) {
    case 16: return launch_t<T, 16>(stage, p, s);
    case 32: return launch_t<T, 32>(stage, p, s);
    case 64: return launch_t<T, 64>(stage, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool mfma_supported(int rank) { return rank == 16 || rank == 32 || rank == 64; }

hipError_t launch_mfma_shrink(int dtype, int rank, const MfmaParams& p, hipStream_t stream) {
  return dtype == 1 ? launch_rank<BF16>(rank, 0, p, stream) : launch_rank<F16>(rank, 0, p, stream);
}

hipError_t launch_mfma_expand(int dtype, int rank, const MfmaParams& p, hipStream_t stream) {
  return dtype == 1 ? launch_rank<BF16>(rank, 1, p, stream) : launch_rank<F16>(rank, 1, p, stream);
}

}  // namespace sgmv
