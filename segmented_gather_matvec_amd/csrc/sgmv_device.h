// sgmv_device.h - device-side helpers shared by the libsgmv kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// The packet id of the current kernel dispatch (LLVM intrinsic; it makes the
// runtime pass the id in user SGPRs).
extern "C" __device__ unsigned long long sgmv_llvm_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

namespace sgmv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // every kernel runs 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;

// Element formats.  Values travel as raw 16-bit patterns and are widened to
// fp32 for arithmetic.
struct F16 {
  static constexpr float kMaxFinite = 65504.f;
  __device__ static inline float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  __device__ static inline float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  __device__ static inline float one(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
  // round to nearest even (v_cvt_f16_f32 under the default rounding mode)
  __device__ static inline uint16_t round(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
};

struct BF16 {
  static constexpr float kMaxFinite = 3.3895314e38f;
  __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static inline float one(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
  // round to nearest even (v_cvt_pk_bf16_f32)
  __device__ static inline uint16_t round(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
};

// Eight 16-bit values of a 128-bit vector, widened to fp32.
template <class T>
__device__ inline void unpack8(const u32x4& v, float (&f)[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = T::lo(v[w]);
    f[2 * w + 1] = T::hi(v[w]);
  }
}

template <class T>
__device__ inline u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    v[w] = (uint32_t)T::round(f[2 * w]) | ((uint32_t)T::round(f[2 * w + 1]) << 16);
  return v;
}

// 128-bit loads of data that is read exactly once per call (LoRA weights,
// X, Y): the non-temporal hint keeps them from displacing reusable lines.
// (Pointers read from the LoRA tables are generic; the cast lets the compiler
// use global instead of flat loads.)
typedef const __attribute__((address_space(1))) u32x4* global_u32x4_ptr;
typedef const __attribute__((address_space(1))) uint16_t* global_u16_ptr;
__device__ inline u32x4 load_stream(const void* p) {
  return __builtin_nontemporal_load((global_u32x4_ptr)p);
}
__device__ inline uint16_t load_stream_u16(const uint16_t* p) {
  return __builtin_nontemporal_load((global_u16_ptr)p);
}
__device__ inline u32x4 load_vec(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void store_vec(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ inline float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Cross-workgroup hand-off (device scope) without whole-cache maintenance.
// Agent-scope release/acquire fences lower to a write-back / invalidate of the
// entire L2 of the XCD on gfx950, which costs far more than the few hundred
// bytes handed over here.  Instead, every datum that crosses workgroups is
// itself a relaxed device-scope atomic access (sc1: written through to, and
// read from, the device-coherent level), and ordering comes from waiting for
// the stores to complete before the counter update that announces them.
__device__ inline void publish_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float fetch_published_f32(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A tag that differs on every launch, replays of a captured graph included:
// the dispatch packet id mixed with the queue address.  Always odd, so a
// zero-filled word never matches.
__device__ inline uint32_t launch_tag() {
  const uint64_t did = sgmv_llvm_dispatch_id();
  const uint64_t q = reinterpret_cast<uint64_t>(__builtin_amdgcn_queue_ptr());
  const uint32_t qh = (uint32_t)(q >> 12) * 0x9E3779B1u;
  return (((uint32_t)did ^ qh) << 1) | 1u;
}
__device__ inline uint64_t fetch_published_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void publish_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A value and its validity in one device-coherent 64-bit word {fp32, tag}:
// no counter, fence or flag is needed to hand it to another workgroup.
__device__ inline void publish_tagged(uint64_t* slot, float v, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(v);
  __hip_atomic_store(slot, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t fetch_tagged(const uint64_t* slot) {
  return __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this thread issued has completed.
__device__ inline void wait_memory_ops() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ inline uint32_t counter_add(uint32_t* c, uint32_t v) {
  return __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t counter_load(const uint32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void counter_store(uint32_t* c, uint32_t v) {
  __hip_atomic_store(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sgmv
