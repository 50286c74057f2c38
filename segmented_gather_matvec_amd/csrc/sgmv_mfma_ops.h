// sgmv_mfma_ops.h - matrix-core helpers shared by the MFMA kernels (gfx950).
//
// v_mfma_f32_16x16x32_{f16,bf16}: lane l holds A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] (e < 8) and D[4(l/16)+i][l%16] (i < 4).  Both operands
// need 8 consecutive k per lane, so a row-major [k][n] operand is staged in
// LDS transposed ([n][k]) with store_pair_transposed.
#pragma once

#include "sgmv_device.h"

namespace sgmv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 128-bit store with the non-temporal hint (streamed output that should not
// displace reused data from the caches).
typedef __attribute__((address_space(1))) u32x4* global_u32x4_wptr;
__device__ inline void store_stream(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, (global_u32x4_wptr)p);
}

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

// Two 8-element rows (u, v) of a row-major tile, written transposed into LDS
// as 32-bit pairs: dst[e*stride] = {u[e], v[e]} for e < 8 (dst in 16-bit
// units, even offset).
__device__ inline void store_pair_transposed(uint16_t* dst, int stride, const u32x4& u, const u32x4& v) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (u[w] & 0xffffu) | (v[w] << 16);
    const uint32_t hi = (u[w] >> 16) | (v[w] & 0xffff0000u);
    *reinterpret_cast<uint32_t*>(dst + (2 * w) * stride) = lo;
    *reinterpret_cast<uint32_t*>(dst + (2 * w + 1) * stride) = hi;
  }
}

// The same pair, with the pair's rows 0..3 at dst_lo + k * stride and rows
// 4..7 at dst_hi + (k - 4) * stride.
__device__ inline void store_pair_transposed_split(uint16_t* dst_lo, uint16_t* dst_hi, int stride, const u32x4& u,
                                                   const u32x4& v) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint16_t* d = w < 2 ? dst_lo + (2 * w) * stride : dst_hi + (2 * w - 4) * stride;
    const uint32_t lo = (u[w] & 0xffffu) | (v[w] << 16);
    const uint32_t hi = (u[w] >> 16) | (v[w] & 0xffff0000u);
    *reinterpret_cast<uint32_t*>(d) = lo;
    *reinterpret_cast<uint32_t*>(d + stride) = hi;
  }
}

}  // namespace sgmv
