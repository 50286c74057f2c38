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
// split partials), kModeExpand reads V, kModeFused does both in one launch:
// each workgroup publishes its shrink partial, waits until all splits of its
// unit have published, sums them, then expands its column chunk.  The fused
// grid is sized by the host to be co-resident, so the wait always ends.
#include "sgmv_device.h"
#include "sgmv_plan.h"

namespace sgmv {
namespace {

constexpr int kNA = 2;  // 128-bit A loads per thread per shrink pass
constexpr int kNB = 2;  // 128-bit B loads per thread per expand pass

template <int R>
constexpr int log2_groups() {
  return R == 8 ? 0 : R == 16 ? 1 : R == 32 ? 2 : 3;
}

struct Unit {
  int r0;  // first row
  int L;   // rows (0: nothing to do)
  int k;   // LoRA id
};

// Map unit u to its segment, first row and row count.  With direct units the
// unit is the segment; otherwise every wave scans ceil(len_s / RB) over the
// segments (64 at a time) and finds the segment whose unit range holds u.
template <int RB>
__device__ inline Unit resolve_unit(const VecParams& p, int u) {
  Unit out{0, 0, 0};
  int s = -1, rb = 0;
  if (p.direct_units) {
    if (u < p.num_segs) s = u;
  } else {
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int c0 = 0; c0 < p.num_segs; c0 += 64) {
      const int sl = c0 + lane;
      int units = 0;
      if (sl < p.num_segs) {
        int len = p.seg_indptr[sl + 1] - p.seg_indptr[sl];
        len = len > 0 ? len : 0;
        units = (len + RB - 1) / RB;
      }
      int incl = units;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int up = __shfl_up(incl, d, 64);
        if (lane >= d) incl += up;
      }
      const int excl = incl - units;
      const bool hit = sl < p.num_segs && u >= base + excl && u < base + incl;
      const unsigned long long m = __ballot(hit);
      if (m) {
        const int l = __builtin_ctzll(m);
        s = c0 + l;
        rb = u - base - __shfl(excl, l, 64);
        break;
      }
      base += __shfl(incl, 63, 64);
    }
  }
  s = __builtin_amdgcn_readfirstlane(s);
  rb = __builtin_amdgcn_readfirstlane(rb);
  if (s < 0) return out;
  const int lo = p.seg_indptr[s];
  const int hi = p.seg_indptr[s + 1];
  const int k = p.lora_idx[s];
  const int r0 = lo + rb * RB;
  int r1 = hi < r0 + RB ? hi : r0 + RB;
  r1 = r1 < p.n_rows ? r1 : p.n_rows;
  if (r0 < 0 || r1 <= r0 || k < 0 || k >= p.num_loras) return out;
  out.r0 = r0;
  out.L = r1 - r0;
  out.k = k;
  return out;
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

template <class T, int R, int RB, int MODE>
__global__ __launch_bounds__(kThreads) void sgmv_vec_kernel(VecParams p) {
  constexpr int JG = R / 8;                 // 128-bit vectors per row of A_k
  constexpr int B0 = log2_groups<R>();
  constexpr int HP = vec_rows_per_pass(R);  // A_k rows per shrink pass
  constexpr int CP = vec_cols_per_pass(R);  // B_k columns per expand pass
  constexpr bool kShrink = MODE != kModeExpand;
  constexpr bool kExpand = MODE != kModeShrink;
  constexpr int NXV = (RB * HP / 8 + kThreads - 1) / kThreads;  // X vectors / thread / pass
  constexpr int NYV = (RB * CP / 8 + kThreads - 1) / kThreads;  // Y vectors / thread / pass

  __shared__ __attribute__((aligned(16))) uint16_t lds_x[kShrink ? RB * HP : 8];
  __shared__ float lds_red[kShrink ? kWaves * RB * R : 1];
  __shared__ float lds_v[RB * R];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[kExpand ? R * CP : 8];
  __shared__ __attribute__((aligned(16))) float lds_out[kExpand ? kThreads * 8 : 4];
  __shared__ int lds_flag;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int G = p.splits;
  const int unit = blockIdx.x / G;
  const int g = blockIdx.x - unit * G;
  const Unit un = resolve_unit<RB>(p, unit);
  if (un.L <= 0) return;  // uniform over the workgroup
  const int L = un.L;
  const int r0 = un.r0;

  // ---- expand operands: B_k columns [c0, c1), Y rows [r0, r0+L) ----
  const uint16_t* Bk = nullptr;
  int c0 = 0, c1 = 0;
  u32x4 bv[kNB];
  u32x4 yv[NYV];
  auto load_expand_pass = [&](int cp0) {
    const int cvr = (c1 - cp0 < CP ? c1 - cp0 : CP) / 8;
#pragma unroll
    for (int q = 0; q < kNB; ++q) {
      const int v = t + kThreads * q;
      if (v < R * cvr) {
        const int j = v / cvr, cv = v - j * cvr;
        bv[q] = load_stream(Bk + (int64_t)j * p.h_out + cp0 + cv * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < NYV; ++q) {
      const int y = t + kThreads * q;
      if (y < L * cvr) {
        const int i = y / cvr, cv = y - i * cvr;
        yv[q] = load_stream(p.Y + (int64_t)(r0 + i) * p.h_out + cp0 + cv * 8);
      }
    }
  };
  if constexpr (kExpand) {
    Bk = reinterpret_cast<const uint16_t*>(p.B_ptrs[un.k]);
    c0 = g * p.cw;
    c1 = p.h_out < c0 + p.cw ? p.h_out : c0 + p.cw;
    // In the fused kernel the first expand pass is fetched before the shrink
    // so that its latency overlaps the shrink and the hand-off.
    if constexpr (MODE == kModeFused)
      if (c0 < c1) load_expand_pass(c0);
  }

  if constexpr (kShrink) {
    const uint16_t* Ak = reinterpret_cast<const uint16_t*>(p.A_ptrs[un.k]);
    const int h0 = g * p.kc;
    const int h1 = p.h_in < h0 + p.kc ? p.h_in : h0 + p.kc;
    float acc[RB][8];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;

    for (int hp0 = h0; hp0 < h1; hp0 += HP) {
      const int hpn = h1 - hp0 < HP ? h1 - hp0 : HP;  // multiple of 8
      const int xvr = hpn / 8;                        // X vectors per row in this pass
      u32x4 xv[NXV];
#pragma unroll
      for (int q = 0; q < NXV; ++q) {
        const int x = t + kThreads * q;
        if (x < L * xvr) {
          const int i = x / xvr, c = x - i * xvr;
          xv[q] = load_stream(p.X + (int64_t)(r0 + i) * p.h_in + hp0 + c * 8);
        }
      }
      u32x4 av[kNA];
#pragma unroll
      for (int q = 0; q < kNA; ++q) {
        const int v = t + kThreads * q;
        if (v < hpn * JG) av[q] = load_stream(Ak + (int64_t)hp0 * R + v * 8);
      }
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
        if (v < hpn * JG) {
          const int hl = v / JG;  // row of A_k inside the pass; this thread's 8 ranks are (t % JG)*8..
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

    float* part = p.partials + ((int64_t)unit * G + g) * (RB * R);
    if (MODE == kModeShrink && G == 1) {
      for (int o = t; o < L * R; o += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += lds_red[w * RB * R + o];
        p.V[(int64_t)(r0 + o / R) * R + (o % R)] = s;
      }
      return;
    }
    for (int o = t; o < L * R; o += kThreads) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += lds_red[w * RB * R + o];
      part[o] = s;
    }
    __threadfence();
    __syncthreads();
    uint32_t* arrive = p.counters + unit;
    if constexpr (MODE == kModeShrink) {
      if (t == 0) lds_flag = counter_add_release(arrive, 1u) == (uint32_t)(G - 1);
      __syncthreads();
      if (!lds_flag) return;
      fence_acquire_agent();
      const float* base = p.partials + (int64_t)unit * G * (RB * R);
      for (int o = t; o < L * R; o += kThreads) {
        float s = 0.f;
        for (int gg = 0; gg < G; ++gg) s += base[gg * (RB * R) + o];
        p.V[(int64_t)(r0 + o / R) * R + (o % R)] = s;
      }
      if (t == 0) counter_store_relaxed(arrive, 0u);
      return;
    } else {
      if (t == 0) {
        counter_add_release(arrive, 1u);
        while (counter_load_acquire(arrive) < (uint32_t)G) __builtin_amdgcn_s_sleep(1);
      }
      __syncthreads();
      fence_acquire_agent();
      const float* base = p.partials + (int64_t)unit * G * (RB * R);
      for (int o = t; o < L * R; o += kThreads) {
        float s = 0.f;
        for (int gg = 0; gg < G; ++gg) s += base[gg * (RB * R) + o];
        lds_v[o] = s;
      }
      __syncthreads();
      if (t == 0) {
        uint32_t* depart = p.counters + p.num_units + unit;
        if (counter_add_release(depart, 1u) == (uint32_t)(G - 1)) {
          counter_store_relaxed(arrive, 0u);
          counter_store_relaxed(depart, 0u);
        }
      }
    }
  }

  if constexpr (kExpand) {
    if constexpr (MODE == kModeExpand) {
      for (int o = t; o < L * R; o += kThreads) lds_v[o] = p.V[(int64_t)(r0 + o / R) * R + (o % R)];
    }
    for (int cp0 = c0; cp0 < c1; cp0 += CP) {
      const int cvr = (c1 - cp0 < CP ? c1 - cp0 : CP) / 8;
      if (MODE != kModeFused || cp0 != c0) load_expand_pass(cp0);
      __syncthreads();  // lds_v ready / previous pass done with lds_b, lds_out
#pragma unroll
      for (int q = 0; q < kNB; ++q) {
        const int v = t + kThreads * q;
        if (v < R * cvr) {
          const int j = v / cvr, cv = v - j * cvr;
          store_vec(&lds_b[j * CP + cv * 8], bv[q]);
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
          store_vec(p.Y + (int64_t)(r0 + i) * p.h_out + cp0 + cv * 8, pack8<T>(yf));
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
            store_vec(p.Y + (int64_t)(r0 + i) * p.h_out + cp0 + cv * 8, pack8<T>(yf));
          }
        }
      }
    }
  }
}

template <class T, int R, int RB, int MODE>
hipError_t launch_one(const VecParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)p.num_units * (unsigned)p.splits;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((sgmv_vec_kernel<T, R, RB, MODE>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <class T, int R, int RB>
hipError_t launch_mode(int mode, const VecParams& p, hipStream_t s) {
  switch (mode) {
    case kModeShrink: return launch_one<T, R, RB, kModeShrink>(p, s);
    case kModeExpand: return launch_one<T, R, RB, kModeExpand>(p, s);
    case kModeFused: return launch_one<T, R, RB, kModeFused>(p, s);
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

template <class T, int R, int RB>
int capacity_for() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&sgmv_vec_kernel<T, R, RB, kModeFused>), kThreads,
          0) != hipSuccess)
    return 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return per_cu * cus;
}

template <class T, int R>
int capacity_rb(int rb) {
  switch (rb) {
    case 1: return capacity_for<T, R, 1>();
    case 4: return capacity_for<T, R, 4>();
    case 16: return capacity_for<T, R, 16>();
  }
  return 0;
}

template <class T>
int capacity_rank(int rank, int rb) {
  switch (rank) {
    case 8: return capacity_rb<T, 8>(rb);
    case 16: return capacity_rb<T, 16>(rb);
    case 32: return capacity_rb<T, 32>(rb);
    case 64: return capacity_rb<T, 64>(rb);
  }
  return 0;
}

}  // namespace

hipError_t launch_vec(int dtype, int rank, int rb, int mode, const VecParams& p, hipStream_t stream) {
  return dtype == 1 ? launch_rank<BF16>(rank, rb, mode, p, stream)
                    : launch_rank<F16>(rank, rb, mode, p, stream);
}

int fused_resident_capacity(int dtype, int rank, int rb) {
  return dtype == 1 ? capacity_rank<BF16>(rank, rb) : capacity_rank<F16>(rank, rb);
}

}  // namespace sgmv
