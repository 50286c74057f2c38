// sgmv_api.cpp - host side of libsgmv: argument checks, the segment builder,
// problem planning (kernel family, row blocks, splits) and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/sgmv.h"
#include "sgmv_host.h"
#include "sgmv_plan.h"

namespace {

using namespace sgmv_host;
using sgmv::VecParams;

constexpr int kMaxDevices = 64;

static_assert(sgmv::kDecodeErrWaitTimeout == SGMV_DEVICE_ERR_WAIT_TIMEOUT, "error bits of the ABI");
static_assert(sgmv::kInlineSegs == SGMV_HOST_META_MAX_SEGS, "segments carried in the kernel arguments");

// Longest wait of a decode-route workgroup for its unit's other partials
// (sgmv_set_wait_limit).  A legitimate wait lasts microseconds; the bound is
// there for a launch that does not have the device to itself.
std::atomic<int64_t> g_wait_limit_us{1000000};

// The limit in ticks of the current device's real-time counter (0 only for a
// limit of 0).
uint32_t wait_ticks() {
  static std::mutex mu;
  static int khz[kMaxDevices];
  const int64_t us = g_wait_limit_us.load(std::memory_order_relaxed);
  if (us == 0) return 0;
  int dev = 0, rate = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    std::lock_guard<std::mutex> lock(mu);
    if (khz[dev] == 0 &&
        (hipDeviceGetAttribute(&khz[dev], hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz[dev] <= 0))
      khz[dev] = 100000;  // the 100 MHz counter of CDNA devices
    rate = khz[dev];
  } else {
    rate = 100000;
  }
  const double ticks = (double)us * rate / 1000.0;
  return ticks >= 4294967295.0 ? 0xffffffffu : std::max<uint32_t>(1u, (uint32_t)ticks);
}

// Variant of the decode kernel a call launches: bit 0 at most 64 LoRAs (the
// pointer tables fetched one entry per lane), bit 1 a row map, bit 2 rank or
// scale tables.  Their register use, hence their occupancy, differs.
int decode_variant(const sgmv_problem_t& p, bool map, bool het) {
  return (p.num_loras <= 64 ? 1 : 0) | (map ? 2 : 0) | (het ? 4 : 0);
}

int decode_capacity(int dtype, int rank, int rb, int variant) {
  static std::mutex mu;
  static int cache[kMaxDevices][2][4][3][sgmv::kDecodeInlineVariant + 1];
  static bool init[kMaxDevices][2][4][3][sgmv::kDecodeInlineVariant + 1];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (variant < 0 || variant > sgmv::kDecodeInlineVariant) return 0;
  const int ri = rank == 8 ? 0 : rank == 16 ? 1 : rank == 32 ? 2 : 3;
  const int bi = rb == 1 ? 0 : rb == 4 ? 1 : 2;
  std::lock_guard<std::mutex> lock(mu);
  if (!init[dev][dtype][ri][bi][variant]) {
    cache[dev][dtype][ri][bi][variant] = sgmv::decode_resident_capacity(dtype, rank, rb, variant);
    init[dev][dtype][ri][bi][variant] = true;
  }
  return cache[dev][dtype][ri][bi][variant];
}

// The first candidate whose grid is co-resident on the current device (the
// kernel's workgroups wait for each other; the capacity is the launched
// variant's, see decode_variant).  When none is, the smallest row block runs
// in passes: launches of the largest co-resident grid, each over the next
// round_units units, up to kMaxDecodeRounds; else unsupported.
// (kMaxDecodeRounds: Distinct batches, H = 4096, r = 16, took 512 rows in 4
// passes in 40.2 us against 43.2 us on the two-launch route.)
DecodePlan plan_decode(const sgmv_problem_t& p, int variant) {
  DecodePlan c[3];
  const int n = decode_candidates(p, c);
  for (int i = 0; i < n; ++i) {
    const int cap = decode_capacity(p.dtype, p.rank, c[i].rb, variant);
    if (cap > 0 && c[i].grid <= cap && c[i].grid <= kMaxResidentGrid) return c[i];
  }
  // (Batches with long segments go to the matrix-core kernels instead.)
  if (n > 0 && !stage_uses_mfma(p)) {
    DecodePlan d = c[0];
    const int64_t cap = decode_capacity(p.dtype, p.rank, d.rb, variant);
    const int64_t step = d.split_major ? 1 : 8;  // the XCD mapping covers units 8 at a time
    const int64_t ru = std::min(cap, kMaxResidentGrid) / d.splits / step * step;
    if (ru >= step) {
      d.round_units = ru;
      d.grid = ru * d.splits;
      d.rounds = ceil_div(d.num_units, ru);
      if (d.rounds <= kMaxDecodeRounds && d.num_units * d.splits <= kMaxDecodeRounds * kMaxResidentGrid) return d;
    }
  }
  return DecodePlan{};
}

sgmv::MfmaParams mfma_params(const sgmv_problem_t& p, const MfmaPlan& m, const int32_t* seg_indptr,
                             const int32_t* lora_idx) {
  sgmv::MfmaParams q{};
  q.seg_indptr = seg_indptr;
  q.lora_idx = lora_idx;
  q.partial_stride = (int64_t)p.n_rows * p.rank;
  q.n_rows = p.n_rows;
  q.h_in = p.h_in;
  q.h_out = p.h_out;
  q.num_segs = p.num_segs;
  q.num_loras = p.num_loras;
  q.num_units64 = (int32_t)m.units64;
  q.direct_units64 = m.direct64;
  q.ksplit = m.ksplit;
  q.kc = m.kc;
  q.chunks_per_wg = m.chunks_per_wg;
  q.expand_rows = m.expand_rows;
  q.num_units_x = (int32_t)m.units_x;
  q.direct_units_x = m.direct_x;
  q.x_lds = m.x_lds;
  return q;
}


bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }
bool aligned2(const void* p) { return ((uintptr_t)p & 1u) == 0; }

VecParams base_params(const sgmv_problem_t& p, const VecPlan& v, const int32_t* seg_indptr,
                      const int32_t* lora_idx, void* ws) {
  VecParams q{};
  q.seg_indptr = seg_indptr;
  q.lora_idx = lora_idx;
  q.counters = static_cast<uint32_t*>(ws);
  q.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + SGMV_WS_COUNTER_BYTES);
  q.n_rows = p.n_rows;
  q.h_in = p.h_in;
  q.h_out = p.h_out;
  q.num_segs = p.num_segs;
  q.num_loras = p.num_loras;
  q.num_units = (int32_t)v.num_units;
  q.splits = v.splits;
  q.kc = v.kc;
  q.cw = v.cw;
  q.direct_units = v.direct;
  return q;
}

sgmv_status_t hip_status(hipError_t e) { return e == hipSuccess ? SGMV_OK : SGMV_ERR_HIP; }

// sgmv_lora_apply runs the one-launch decode kernel when one of its plans fits
// on the device at once, else the matrix-core or vector kernels.
bool use_decode(const sgmv_problem_t& p, const DecodePlan& d) {
  return p.variant != SGMV_VARIANT_VECTOR && p.variant != SGMV_VARIANT_MFMA && d.supported;
}

sgmv_route_t apply_route(const sgmv_problem_t& p, const DecodePlan& d) {
  if (nothing_to_do(p)) return SGMV_ROUTE_NONE;
  if (use_decode(p, d)) return SGMV_ROUTE_DECODE;
  return stage_uses_mfma(p) ? SGMV_ROUTE_MFMA : SGMV_ROUTE_VECTOR;
}

sgmv::Projection kernel_projection(const sgmv_projection_t& pj) {
  sgmv::Projection k{};
  k.A_ptrs = reinterpret_cast<const uint64_t*>(pj.A_ptrs);
  k.B_ptrs = reinterpret_cast<const uint64_t*>(pj.B_ptrs);
  k.Y = static_cast<uint16_t*>(pj.Y);
  k.ranks = pj.ranks;
  k.scales = pj.scales;
  return k;
}

// Arguments of the decode kernel for plan d; ws is projection 0's workspace
// slice, stride the bytes between slices.
hipError_t decode_params(const sgmv_problem_t& p, const DecodePlan& d, const void* X, const sgmv_projection_t* pj,
                         int np, const int32_t* seg_indptr, const int32_t* lora_idx, const int32_t* row_idx,
                         char* ws, size_t stride, sgmv::DecodeParams* out) {
  sgmv::DecodeParams& q = *out;
  q = sgmv::DecodeParams{};
  const hipError_t e = sgmv::decode_error_word(&q.errors);
  if (e != hipSuccess) return e;
  q.wait_ticks = wait_ticks();
  q.X = static_cast<const uint16_t*>(X);
  for (int i = 0; i < np; ++i) q.proj[i] = kernel_projection(pj[i]);
  q.seg_indptr = seg_indptr;
  q.lora_idx = lora_idx;
  q.row_idx = row_idx;
  q.slots = reinterpret_cast<uint64_t*>(ws + apply_ws_layout(p).decode_off);
  q.slot_stride = (int64_t)(stride / sizeof(uint64_t));
  q.n_rows = p.n_rows;
  q.h_in = p.h_in;
  q.h_out = p.h_out;
  q.num_segs = p.num_segs;
  q.num_loras = p.num_loras;
  q.num_units = (int32_t)d.num_units;
  q.splits = d.splits;
  q.kc = d.kc;
  q.cw = d.cw;
  q.direct_units = d.direct;
  q.split_major = d.split_major;
  q.round_units = (int32_t)d.round_units;
  return hipSuccess;
}

// sgmv_lora_apply for num_proj projections that share X, the shapes and the
// segments.  Projection i uses the workspace slice [i*stride, i*stride + need).
// clear_counters: zero the two-launch route's counters with a fill kernel
// before its shrink (a workspace whose counter area may not be zero).
sgmv_status_t apply(const sgmv_problem_t& p, const void* X, const sgmv_projection_t* pj, int np,
                    const int32_t* seg_indptr, const int32_t* lora_idx, const int32_t* row_idx, char* ws,
                    size_t stride, hipStream_t s, bool clear_counters = false) {
  bool het = false;
  for (int i = 0; i < np; ++i) het = het || pj[i].ranks || pj[i].scales;
  const int variant = decode_variant(p, row_idx != nullptr, het);
  const DecodePlan d = plan_decode(p, variant);
  const sgmv_route_t route = apply_route(p, d);
  if (route == SGMV_ROUTE_DECODE) {
    // The workgroups of one projection wait for each other; all projections
    // run in one launch when all of them fit on the device at once.
    if (np > 1 && d.grid * np > decode_capacity(p.dtype, p.rank, d.rb, variant)) {
      for (int i = 0; i < np; ++i) {
        const sgmv_status_t st = apply(p, X, pj + i, 1, seg_indptr, lora_idx, row_idx, ws + (size_t)i * stride,
                                       stride, s, clear_counters);
        if (st != SGMV_OK) return st;
      }
      return SGMV_OK;
    }
    sgmv::DecodeParams q{};
    if (decode_params(p, d, X, pj, np, seg_indptr, lora_idx, row_idx, ws, stride, &q) != hipSuccess)
      return SGMV_ERR_HIP;
    // One launch per pass of round_units units (a single one when they all
    // fit on the device at once); each launch's workgroups are co-resident.
    for (int64_t pass = 0; pass < d.rounds; ++pass) {
      q.unit_base = (int32_t)(pass * d.round_units);
      const hipError_t e = sgmv::launch_decode(p.dtype, p.rank, d.rb, q, np, s);
      if (e != hipSuccess) return SGMV_ERR_HIP;
    }
    return SGMV_OK;
  }
  if (route == SGMV_ROUTE_MFMA) {
    // Matrix-core route: the shrink writes one fp32 partial plane of V per H1
    // chunk, the reduce sums them (in chunk order) into V, the expand reads V.
    const MfmaPlan m = plan_mfma(p);
    sgmv::MfmaParams q = mfma_params(p, m, seg_indptr, lora_idx);
    q.row_idx = row_idx;
    q.X = static_cast<const uint16_t*>(X);
    for (int i = 0; i < np; ++i) q.proj[i] = kernel_projection(pj[i]);
    q.partials = reinterpret_cast<float*>(ws + SGMV_WS_COUNTER_BYTES);
    q.V = reinterpret_cast<float*>(ws + SGMV_WS_COUNTER_BYTES + m.partial_bytes);
    q.proj_stride = (int64_t)(stride / sizeof(float));
    if (!m.lead) q.V = q.partials;  // a single plane is V itself
    if (m.lead) {
      // Lead workgroups of the expand launch sum the planes; their tagged V
      // words or row-block flags have an area of their own in each
      // projection's slice of the workspace.
      if (sgmv::decode_error_word(&q.errors) != hipSuccess) return SGMV_ERR_HIP;
      q.lead_reduce = 1;
      q.lead_blocks = m.lead_blocks;
      q.lead_rows = m.lead_rows;
      q.lead_proj = np;
      q.wait_ticks = wait_ticks();
      q.lead_area = ws + apply_ws_layout(p).lead_off;
    }
    hipError_t e = sgmv::launch_mfma_shrink(p.dtype, p.rank, q, np, s);
    if (e != hipSuccess) return SGMV_ERR_HIP;
    return hip_status(sgmv::launch_mfma_expand(p.dtype, p.rank, q, np, s));
  }
  // Two launches per projection: shrink into V (held after the shrink's split
  // partials), then expand.
  const VecPlan v = plan_vec(p, kTargetWorkgroups);
  const size_t need = vec_ws_bytes(v, p.rank);
  for (int i = 0; i < np; ++i) {
    char* wsi = ws + (size_t)i * stride;
    VecParams q = base_params(p, v, seg_indptr, lora_idx, wsi);
    q.row_idx = row_idx;
    q.X = static_cast<const uint16_t*>(X);
    q.A_ptrs = reinterpret_cast<const uint64_t*>(pj[i].A_ptrs);
    q.B_ptrs = reinterpret_cast<const uint64_t*>(pj[i].B_ptrs);
    q.Y = static_cast<uint16_t*>(pj[i].Y);
    q.ranks = pj[i].ranks;
    q.scales = pj[i].scales;
    q.V = reinterpret_cast<float*>(wsi + need);
    hipError_t e = hipSuccess;
    if (clear_counters) e = sgmv::launch_clear_u32(q.counters, 2 * v.num_units, s);
    if (e != hipSuccess) return SGMV_ERR_HIP;
    e = sgmv::launch_vec(p.dtype, p.rank, v.rb, sgmv::kModeShrink, q, s);
    if (e != hipSuccess) return SGMV_ERR_HIP;
    e = sgmv::launch_vec(p.dtype, p.rank, v.rb, sgmv::kModeExpand, q, s);
    if (e != hipSuccess) return SGMV_ERR_HIP;
  }
  return SGMV_OK;
}

// Static scratch of sgmv_lora_apply_noalloc: device memory of the library,
// one copy on every GPU it runs on, held until the process ends.  In host code
// the array's name is not a device address; the address of each device's copy
// comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[SGMV_NOALLOC_MAX_WORKSPACE];

hipError_t scratch_address(char** out) {
  static std::mutex mu;
  static char* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    char* ptr = nullptr;
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&ptr), HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

sgmv_status_t sgmv_shrink(const sgmv_problem_t* p, const void* X, const void* const* A_ptrs,
                          float* V, const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                          size_t ws_bytes, void* stream) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (nothing_to_do(*p)) return SGMV_OK;
  if (!X || !A_ptrs || !V || !seg_indptr || !lora_idx) return SGMV_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(V) || !aligned8(A_ptrs)) return SGMV_ERR_UNSUPPORTED;
  if (stage_uses_mfma(*p)) {
    const MfmaPlan m = plan_mfma(*p);
    if (!ws || ws_bytes < SGMV_WS_COUNTER_BYTES + m.partial_bytes) return SGMV_ERR_WORKSPACE;
    if (!aligned16(ws)) return SGMV_ERR_UNSUPPORTED;
    sgmv::MfmaParams q = mfma_params(*p, m, seg_indptr, lora_idx);
    q.X = static_cast<const uint16_t*>(X);
    q.proj[0].A_ptrs = reinterpret_cast<const uint64_t*>(A_ptrs);
    q.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + SGMV_WS_COUNTER_BYTES);
    q.V = V;
    return hip_status(sgmv::launch_mfma_shrink(p->dtype, p->rank, q, 1, static_cast<hipStream_t>(stream)));
  }
  const VecPlan v = plan_vec(*p, kTargetWorkgroups);
  if (!ws || ws_bytes < vec_ws_bytes(v, p->rank)) return SGMV_ERR_WORKSPACE;
  if (!aligned16(ws)) return SGMV_ERR_UNSUPPORTED;
  VecParams q = base_params(*p, v, seg_indptr, lora_idx, ws);
  q.X = static_cast<const uint16_t*>(X);
  q.A_ptrs = reinterpret_cast<const uint64_t*>(A_ptrs);
  q.V = V;
  return hip_status(sgmv::launch_vec(p->dtype, p->rank, v.rb, sgmv::kModeShrink, q,
                                     static_cast<hipStream_t>(stream)));
}

sgmv_status_t sgmv_expand(const sgmv_problem_t* p, const float* V, const void* const* B_ptrs,
                          void* Y, const int32_t* seg_indptr, const int32_t* lora_idx,
                          void* stream) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (nothing_to_do(*p)) return SGMV_OK;
  if (!V || !B_ptrs || !Y || !seg_indptr || !lora_idx) return SGMV_ERR_INVALID_ARG;
  if (!aligned16(V) || !aligned16(Y) || !aligned8(B_ptrs)) return SGMV_ERR_UNSUPPORTED;
  if (stage_uses_mfma(*p)) {
    sgmv::MfmaParams q = mfma_params(*p, plan_mfma(*p), seg_indptr, lora_idx);
    q.V = const_cast<float*>(V);
    q.proj[0].B_ptrs = reinterpret_cast<const uint64_t*>(B_ptrs);
    q.proj[0].Y = static_cast<uint16_t*>(Y);
    return hip_status(sgmv::launch_mfma_expand(p->dtype, p->rank, q, 1, static_cast<hipStream_t>(stream)));
  }
  const VecPlan v = plan_vec(*p, kTargetWorkgroups);
  VecParams q = base_params(*p, v, seg_indptr, lora_idx, nullptr);
  q.counters = nullptr;
  q.partials = nullptr;
  q.V = const_cast<float*>(V);
  q.B_ptrs = reinterpret_cast<const uint64_t*>(B_ptrs);
  q.Y = static_cast<uint16_t*>(Y);
  return hip_status(sgmv::launch_vec(p->dtype, p->rank, v.rb, sgmv::kModeExpand, q,
                                     static_cast<hipStream_t>(stream)));
}

sgmv_status_t sgmv_query_plan(const sgmv_problem_t* p, sgmv_plan_info_t* info) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (!info) return SGMV_ERR_INVALID_ARG;
  *info = sgmv_plan_info_t{};
  const DecodePlan d = plan_decode(*p, decode_variant(*p, false, false));
  info->route = apply_route(*p, d);
  switch (info->route) {
    case SGMV_ROUTE_DECODE:
      info->launches = (int32_t)d.rounds;
      info->rows_per_unit = d.rb;
      info->units = (int32_t)d.num_units;
      info->splits = d.splits;
      info->grid = (int32_t)d.grid;
      break;
    case SGMV_ROUTE_MFMA: {
      const MfmaPlan m = plan_mfma(*p);
      info->launches = 2;  // the planes are summed by the expand launch's lead workgroups
      info->rows_per_unit = sgmv::kMfmaRowsPerTile;
      info->units = (int32_t)m.units64;
      info->splits = m.ksplit;
      info->grid = (int32_t)(m.units64 * m.ksplit);
      break;
    }
    case SGMV_ROUTE_VECTOR: {
      const VecPlan v = plan_vec(*p, kTargetWorkgroups);
      info->launches = 2;
      info->rows_per_unit = v.rb;
      info->units = (int32_t)v.num_units;
      info->splits = v.splits;
      info->grid = (int32_t)(v.num_units * v.splits);
      break;
    }
    default: break;
  }
  return SGMV_OK;
}

sgmv_status_t sgmv_set_wait_limit(int64_t microseconds) {
  if (microseconds < 0) return SGMV_ERR_INVALID_ARG;
  g_wait_limit_us.store(microseconds, std::memory_order_relaxed);
  return SGMV_OK;
}

sgmv_status_t sgmv_take_device_errors(uint32_t* flags) {
  if (!flags) return SGMV_ERR_INVALID_ARG;
  uint32_t* word = nullptr;
  if (sgmv::decode_error_word(&word) != hipSuccess) return SGMV_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return SGMV_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, word, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return SGMV_ERR_HIP;
  if (v != 0) {
    const uint32_t zero = 0;
    if (hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return SGMV_ERR_HIP;
  }
  *flags = v;
  return SGMV_OK;
}

sgmv_status_t sgmv_lora_apply(const sgmv_problem_t* p, const void* X, const void* const* A_ptrs,
                              const void* const* B_ptrs, void* Y, const int32_t* seg_indptr,
                              const int32_t* lora_idx, void* ws, size_t ws_bytes, void* stream) {
  const sgmv_projection_t one{A_ptrs, B_ptrs, Y, nullptr, nullptr};
  return sgmv_lora_apply_batched(p, X, &one, 1, seg_indptr, lora_idx, nullptr, ws, ws_bytes, stream);
}

sgmv_status_t sgmv_lora_apply_noalloc(const sgmv_problem_t* p, const void* X, const void* const* A_ptrs,
                                      const void* const* B_ptrs, void* Y, const int32_t* seg_indptr,
                                      const int32_t* lora_idx, void* stream) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (nothing_to_do(*p)) return SGMV_OK;
  if (!X || !A_ptrs || !B_ptrs || !Y || !seg_indptr || !lora_idx) return SGMV_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Y) || !aligned8(A_ptrs) || !aligned8(B_ptrs)) return SGMV_ERR_UNSUPPORTED;
  const size_t need = apply_ws_layout(*p).total;
  if (need > (size_t)SGMV_NOALLOC_MAX_WORKSPACE) return SGMV_ERR_WORKSPACE;
  char* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return SGMV_ERR_HIP;
  const sgmv_projection_t one{A_ptrs, B_ptrs, Y, nullptr, nullptr};
  // The scratch keeps the last call's contents: the two-launch route clears
  // its counters itself; the decode route's tagged slots and the matrix-core
  // route's planes need no initial value.
  return apply(*p, X, &one, 1, seg_indptr, lora_idx, nullptr, ws, (size_t)round_up((int64_t)need, 256),
               static_cast<hipStream_t>(stream), /*clear_counters=*/true);
}

sgmv_status_t sgmv_lora_apply_batched(const sgmv_problem_t* p, const void* X,
                                      const sgmv_projection_t* projections, int32_t num_projections,
                                      const int32_t* seg_indptr, const int32_t* lora_idx,
                                      const int32_t* row_idx, void* ws, size_t ws_bytes, void* stream) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (!projections || num_projections < 1 || num_projections > SGMV_MAX_PROJECTIONS) return SGMV_ERR_INVALID_ARG;
  if (nothing_to_do(*p)) return SGMV_OK;
  if (!X || !seg_indptr || !lora_idx) return SGMV_ERR_INVALID_ARG;
  if (!aligned16(X)) return SGMV_ERR_UNSUPPORTED;
  for (int32_t i = 0; i < num_projections; ++i) {
    const sgmv_projection_t& pj = projections[i];
    if (!pj.A_ptrs || !pj.B_ptrs || !pj.Y) return SGMV_ERR_INVALID_ARG;
    if (!aligned16(pj.Y) || !aligned8(pj.A_ptrs) || !aligned8(pj.B_ptrs)) return SGMV_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(pj.ranks) | reinterpret_cast<uintptr_t>(pj.scales)) % 4 != 0)
      return SGMV_ERR_UNSUPPORTED;
  }
  if (!ws) return SGMV_ERR_WORKSPACE;
  if (!aligned16(ws)) return SGMV_ERR_UNSUPPORTED;
  const size_t need = apply_ws_layout(*p).total;
  const size_t stride = (size_t)round_up((int64_t)need, 256);
  if (ws_bytes < stride * (size_t)(num_projections - 1) + need) return SGMV_ERR_WORKSPACE;
  return apply(*p, X, projections, num_projections, seg_indptr, lora_idx, row_idx, static_cast<char*>(ws),
               stride, static_cast<hipStream_t>(stream));
}

sgmv_status_t sgmv_lora_apply_host_meta(const sgmv_problem_t* p, const void* X, const void* const* A_ptrs_host,
                                        const void* const* B_ptrs_host, void* Y, const int32_t* seg_indptr_host,
                                        const int32_t* lora_idx_host, void* ws, size_t ws_bytes, void* stream) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (nothing_to_do(*p)) return SGMV_OK;
  if (!X || !A_ptrs_host || !B_ptrs_host || !Y || !seg_indptr_host || !lora_idx_host) return SGMV_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Y)) return SGMV_ERR_UNSUPPORTED;
  st = sgmv_check_segments(p, seg_indptr_host, lora_idx_host);
  if (st != SGMV_OK) return st;
  if (p->num_segs > sgmv::kInlineSegs) return SGMV_ERR_UNSUPPORTED;
  // Each segment's A_k and B_k, gathered here on the host.
  sgmv::InlineMeta m{};
  for (int32_t s = 0; s <= p->num_segs; ++s) m.seg[s] = seg_indptr_host[s];
  for (int32_t s = 0; s < p->num_segs; ++s) {
    m.a[s] = reinterpret_cast<uint64_t>(A_ptrs_host[lora_idx_host[s]]);
    m.b[s] = reinterpret_cast<uint64_t>(B_ptrs_host[lora_idx_host[s]]);
    if (m.a[s] == 0 || m.b[s] == 0) return SGMV_ERR_INVALID_ARG;
    if ((m.a[s] | m.b[s]) % 16 != 0) return SGMV_ERR_UNSUPPORTED;
  }
  if (!ws) return SGMV_ERR_WORKSPACE;
  if (!aligned16(ws)) return SGMV_ERR_UNSUPPORTED;
  if (ws_bytes < apply_ws_layout(*p).total) return SGMV_ERR_WORKSPACE;
  const DecodePlan d = plan_decode(*p, sgmv::kDecodeInlineVariant);
  if (apply_route(*p, d) != SGMV_ROUTE_DECODE) return SGMV_ERR_UNSUPPORTED;
  const sgmv_projection_t one{nullptr, nullptr, Y, nullptr, nullptr};
  sgmv::DecodeParams q{};
  const size_t stride = (size_t)round_up((int64_t)apply_ws_layout(*p).total, 256);
  if (decode_params(*p, d, X, &one, 1, nullptr, nullptr, nullptr, static_cast<char*>(ws), stride, &q) != hipSuccess)
    return SGMV_ERR_HIP;
  for (int64_t pass = 0; pass < d.rounds; ++pass) {
    q.unit_base = (int32_t)(pass * d.round_units);
    if (sgmv::launch_decode_inline(p->dtype, p->rank, d.rb, q, m, static_cast<hipStream_t>(stream)) != hipSuccess)
      return SGMV_ERR_HIP;
  }
  return SGMV_OK;
}

}  // extern "C"

namespace {

// Yf (non-null): write the fp32 sum unrounded into Yf instead of rounding it into Y.
sgmv_status_t base_apply(const sgmv_problem_t* p, const void* X, const void* W, bool packed,
                         const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                         const int32_t* seg_indptr, const int32_t* lora_idx, void* ws, size_t ws_bytes,
                         void* stream, float* Yf = nullptr) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (p->n_rows > sgmv::kBaseMaxRows) return SGMV_ERR_UNSUPPORTED;
  if (p->n_rows == 0) return SGMV_OK;
  if (!X || !W || (!Y && !Yf)) return SGMV_ERR_INVALID_ARG;
  const bool lora = !nothing_to_do(*p);
  if (lora && (!A_ptrs || !B_ptrs || !seg_indptr || !lora_idx)) return SGMV_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Yf ? static_cast<const void*>(Yf) : Y))
    return SGMV_ERR_UNSUPPORTED;
  if (lora && (!aligned8(A_ptrs) || !aligned8(B_ptrs))) return SGMV_ERR_UNSUPPORTED;
  const BasePlan b = plan_base(*p, packed);
  if (!ws || ws_bytes < b.total) return SGMV_ERR_WORKSPACE;
  if (!aligned16(ws)) return SGMV_ERR_UNSUPPORTED;
  char* w = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  sgmv::BaseParams q{};
  q.n_rows = p->n_rows;
  q.h_in = p->h_in;
  q.h_out = p->h_out;
  q.num_segs = lora ? p->num_segs : 0;
  q.num_loras = p->num_loras;
  q.strip_cols = b.strip_cols;
  q.strips = b.strips;
  q.ksplit = b.ksplit;
  q.kc = b.kc;
  q.base_grid = b.base_grid;
  q.shrink_grid = lora ? (int32_t)round_up((int64_t)p->n_rows * b.ksplit, 8) : 0;
  q.packed_ksteps = packed ? (int32_t)packed_ksteps(p->h_in) : 0;
  q.plane_stride = (int64_t)p->n_rows * p->h_out;
  q.seg_indptr = lora ? seg_indptr : nullptr;
  q.lora_idx = lora ? lora_idx : nullptr;
  q.X = static_cast<const uint16_t*>(X);
  q.W = static_cast<const uint16_t*>(W);
  q.A_ptrs = lora ? reinterpret_cast<const uint64_t*>(A_ptrs) : nullptr;
  q.B_ptrs = lora ? reinterpret_cast<const uint64_t*>(B_ptrs) : nullptr;
  q.vpartials = lora ? reinterpret_cast<float*>(w + b.v_off) : nullptr;
  q.row_b = lora ? reinterpret_cast<uint64_t*>(w + b.b_off) : nullptr;
  q.partials = reinterpret_cast<float*>(w + b.p_off);
  q.Y = Yf ? nullptr : static_cast<uint16_t*>(Y);
  q.Yf = Yf;
  return hip_status(sgmv::launch_base(p->dtype, p->rank, q, s));
}

}  // namespace

extern "C" {

sgmv_status_t sgmv_base_lora_apply(const sgmv_problem_t* p, const void* X, const void* W,
                                   const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                                   const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                                   size_t ws_bytes, void* stream) {
  return base_apply(p, X, W, false, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, ws_bytes, stream);
}

sgmv_status_t sgmv_base_pack_weight(const void* W, int32_t h_in, int32_t h_out, void* Wp, size_t wp_bytes,
                                    void* stream) {
  if (!W || !Wp || h_in <= 0 || h_out <= 0) return SGMV_ERR_INVALID_ARG;
  if (wp_bytes < (size_t)packed_bytes(h_in, h_out)) return SGMV_ERR_WORKSPACE;
  if (!aligned2(W) || !aligned16(Wp)) return SGMV_ERR_UNSUPPORTED;
  return hip_status(sgmv::launch_base_pack(static_cast<const uint16_t*>(W), h_in, h_out,
                                           static_cast<uint16_t*>(Wp), static_cast<hipStream_t>(stream)));
}

sgmv_status_t sgmv_base_lora_apply_partial(const sgmv_problem_t* p, const void* X, const void* W,
                                           int32_t w_packed, const void* const* A_ptrs,
                                           const void* const* B_ptrs, float* Yp, const int32_t* seg_indptr,
                                           const int32_t* lora_idx, void* ws, size_t ws_bytes, void* stream) {
  if (w_packed != 0 && w_packed != 1) return SGMV_ERR_INVALID_ARG;
  if (!Yp) return SGMV_ERR_INVALID_ARG;
  return base_apply(p, X, W, w_packed == 1, A_ptrs, B_ptrs, nullptr, seg_indptr, lora_idx, ws, ws_bytes, stream,
                    Yp);
}

sgmv_status_t sgmv_base_lora_apply_packed(const sgmv_problem_t* p, const void* X, const void* Wp,
                                          const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                                          const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                                          size_t ws_bytes, void* stream) {
  return base_apply(p, X, Wp, true, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, ws_bytes, stream);
}

}  // extern "C"
