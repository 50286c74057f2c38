// sgmv_api.cpp - host side of libsgmv: argument checks, the segment builder,
// problem planning (kernel family, row blocks, splits) and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/sgmv.h"
#include "sgmv_plan.h"

namespace {

using sgmv::VecParams;

constexpr int kMaxDevices = 64;
constexpr int64_t kCounterSlots = (int64_t)(SGMV_WS_COUNTER_BYTES / sizeof(uint32_t));
// Aim for this many workgroups per launch of the vector kernels: two per CU of
// a 256-CU MI355X keeps enough 128-bit loads in flight to cover HBM latency.
constexpr int kTargetWorkgroups = 512;
constexpr int kMaxSplits = 1024;

bool rank_supported(int r) { return r == 8 || r == 16 || r == 32 || r == 64; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }

// Plan of one vector-kernel launch.
struct VecPlan {
  int rb = 1;
  int direct = 1;
  int64_t num_units = 0;
  int splits = 1;
  int kc = 8;
  int cw = 8;
  size_t partial_bytes() const {
    return (size_t)num_units * (size_t)splits * (size_t)rb * sizeof(float);  // times rank
  }
};

int pick_rb(int max_seg_len) { return max_seg_len <= 1 ? 1 : (max_seg_len <= 4 ? 4 : 16); }

VecPlan plan_vec(const sgmv_problem_t& p, int64_t target_wgs) {
  VecPlan v;
  v.rb = pick_rb(p.max_seg_len);
  if (p.max_seg_len <= v.rb) {
    v.direct = 1;
    v.num_units = p.num_segs;
  } else {
    v.direct = 0;
    const int64_t per_seg = ceil_div(p.max_seg_len, v.rb);
    v.num_units = std::min<int64_t>((int64_t)p.num_segs * per_seg, ceil_div(p.n_rows, v.rb) + p.num_segs);
  }
  const int64_t max_split = std::min<int64_t>(
      {ceil_div(p.h_in, 8), ceil_div(p.h_out, 8), (int64_t)kMaxSplits});
  int64_t g = p.splits > 0 ? p.splits : ceil_div(target_wgs, std::max<int64_t>(v.num_units, 1));
  g = std::max<int64_t>(1, std::min(g, max_split));
  v.splits = (int)g;
  v.kc = (int)round_up(ceil_div(p.h_in, g), 8);
  v.cw = (int)round_up(ceil_div(p.h_out, g), 8);
  return v;
}

size_t vec_ws_bytes(const VecPlan& v, int rank) {
  return SGMV_WS_COUNTER_BYTES + v.partial_bytes() * (size_t)rank;
}

// fp32 intermediate V [n_rows, rank] of the two-launch route of sgmv_lora_apply.
size_t v_area_bytes(const sgmv_problem_t& p) {
  return (size_t)round_up((int64_t)p.n_rows * p.rank * (int64_t)sizeof(float), 256);
}

// Plan of one decode-kernel launch (sgmv_lora_apply on short segments).
struct DecodePlan {
  bool supported = false;  // shapes the decode kernel takes
  int rb = 1;
  int direct = 1;
  int64_t num_units = 0;
  int splits = 1;
  int kc = 8;
  int cw = 8;
  int64_t grid = 0;         // workgroups of the launch: round_units * splits
  int64_t round_units = 0;  // units covered by one pass of the grid
  int64_t rounds = 1;       // passes: more than one when the units do not all fit at once
  size_t slot_bytes = 0;
  int split_major = 0;
};

DecodePlan plan_decode_rb(const sgmv_problem_t& p, int rb, int split_major) {
  DecodePlan d;
  d.rb = rb;
  d.split_major = split_major;
  if (!sgmv::decode_supported(p.rank, d.rb)) return d;
  if (p.max_seg_len <= d.rb) {
    d.direct = 1;
    d.num_units = p.num_segs;
  } else {
    d.direct = 0;
    const int64_t per_seg = ceil_div(p.max_seg_len, d.rb);
    d.num_units = std::min<int64_t>((int64_t)p.num_segs * per_seg, ceil_div(p.n_rows, d.rb) + p.num_segs);
  }
  const int64_t gmin = std::max(ceil_div(p.h_in, sgmv::decode_max_kc(p.rank)),
                                ceil_div(p.h_out, sgmv::decode_max_cw()));
  const int64_t gmax = std::min<int64_t>({ceil_div(p.h_in, 8), ceil_div(p.h_out, 8), (int64_t)kMaxSplits});
  if (gmin > gmax) return d;
  // The fewest splits whose chunks fit one workgroup: every extra split adds a
  // partial to each unit's exchange, and measured over batches of 1 to 64 rows
  // the exchange fan-in costs more than the bandwidth of the extra workgroups
  // gains (one row: 8.8 us at 128 splits, 4.0 us at 8).
  const int parts = 1;  // one published partial per workgroup
  int64_t g = p.splits > 0 ? p.splits : gmin;
  g = std::max(gmin, std::min(g, gmax));
  d.splits = (int)g;
  d.kc = (int)round_up(ceil_div(p.h_in, g), 8);
  d.cw = (int)round_up(ceil_div(p.h_out, g), 8);
  d.round_units = split_major ? d.num_units : 8 * ceil_div(d.num_units, 8);
  d.grid = d.round_units * g;
  d.slot_bytes = (size_t)d.num_units * (size_t)g * parts * d.rb * p.rank * sizeof(uint64_t);
  d.supported = d.grid > 0 && d.grid <= (int64_t)INT32_MAX;
  return d;
}

// Variant of the decode kernel a call launches: bit 0 at most 64 LoRAs (the
// pointer tables fetched one entry per lane), bit 1 a row map, bit 2 rank or
// scale tables.  Their register use, hence their occupancy, differs.
int decode_variant(const sgmv_problem_t& p, bool map, bool het) {
  return (p.num_loras <= 64 ? 1 : 0) | (map ? 2 : 0) | (het ? 4 : 0);
}

int decode_capacity(int dtype, int rank, int rb, int variant) {
  static std::mutex mu;
  static int cache[kMaxDevices][2][4][3][8];
  static bool init[kMaxDevices][2][4][3][8];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (variant < 0 || variant > 7) return 0;
  const int ri = rank == 8 ? 0 : rank == 16 ? 1 : rank == 32 ? 2 : 3;
  const int bi = rb == 1 ? 0 : rb == 4 ? 1 : 2;
  std::lock_guard<std::mutex> lock(mu);
  if (!init[dev][dtype][ri][bi][variant]) {
    cache[dev][dtype][ri][bi][variant] = sgmv::decode_resident_capacity(
        dtype, rank, rb, (variant & 1) != 0, (variant & 2) != 0, (variant & 4) != 0);
    init[dev][dtype][ri][bi][variant] = true;
  }
  return cache[dev][dtype][ri][bi][variant];
}

// Passes (launches) of the decode kernel over the units beyond which the
// two-launch route is taken instead (Distinct batches, H = 4096, r = 16: 256
// rows in 2 passes 20.0 us against 27.4 us; 512 rows in 4 passes 40.2 against
// 43.2 us).
constexpr int64_t kMaxDecodeRounds = 4;

// Candidate decode plans, smallest row block first. Blocks of one row keep
// the most workgroups busy; when segments hold several rows (rows that share
// a LoRA), the split-major mapping puts equal splits of neighbouring units on
// one XCD, so a segment's rows re-read their A_k / B_k slice from that XCD's
// L2 rather than from HBM. Segments of one row keep a unit on one XCD.
int decode_candidates(const sgmv_problem_t& p, DecodePlan out[3]) {
  const int split_major = p.max_seg_len > 1 ? 1 : 0;
  int n = 0;
  for (int rb : {1, 4, 16}) {
    const DecodePlan d = plan_decode_rb(p, rb, split_major);
    if (d.supported) out[n++] = d;
    if (p.max_seg_len <= rb) break;  // a larger block only adds empty rows
  }
  return n;
}

// The matrix-core kernels take over segments longer than the decode kernel's
// row blocks (at ranks 16..64); AUTO picks them when the decode kernel cannot
// run the call.
bool stage_uses_mfma(const sgmv_problem_t& p) {
  if (!sgmv::mfma_supported(p.rank)) return false;
  if (p.variant == SGMV_VARIANT_MFMA) return true;
  return p.variant == SGMV_VARIANT_AUTO && p.max_seg_len > 16;
}

// The first candidate whose grid is co-resident on the current device (the
// kernel's workgroups wait for each other; the capacity is the launched
// variant's, see decode_variant).  When none is, the smallest row block runs
// in passes: launches of the largest co-resident grid, each over the next
// round_units units, up to kMaxDecodeRounds; else unsupported.
DecodePlan plan_decode(const sgmv_problem_t& p, int variant) {
  DecodePlan c[3];
  const int n = decode_candidates(p, c);
  for (int i = 0; i < n; ++i) {
    const int cap = decode_capacity(p.dtype, p.rank, c[i].rb, variant);
    if (cap > 0 && c[i].grid <= cap) return c[i];
  }
  // (Batches with long segments go to the matrix-core kernels instead.)
  if (n > 0 && !stage_uses_mfma(p)) {
    DecodePlan d = c[0];
    const int64_t cap = decode_capacity(p.dtype, p.rank, d.rb, variant);
    const int64_t step = d.split_major ? 1 : 8;  // the XCD mapping covers units 8 at a time
    const int64_t ru = cap / d.splits / step * step;
    if (ru >= step) {
      d.round_units = ru;
      d.grid = ru * d.splits;
      d.rounds = ceil_div(d.num_units, ru);
      if (d.rounds <= kMaxDecodeRounds) return d;
    }
  }
  return DecodePlan{};
}

size_t decode_ws_bytes(const sgmv_problem_t& p) {
  DecodePlan c[3];
  const int n = decode_candidates(p, c);
  size_t b = 0;
  for (int i = 0; i < n; ++i) b = std::max(b, c[i].slot_bytes);
  return b;
}

// Plan of the matrix-core kernels (long segments).
struct MfmaPlan {
  int64_t units64 = 0;
  int direct64 = 1;
  int ksplit = 1;
  int kc = 0;
  int chunks_per_wg = 1;
  int expand_rows = sgmv::kMfmaRowsPerTile;  // rows of one expand tile (16 for short tiles)
  int64_t units_x = 0;                        // expand units of <= expand_rows rows
  int direct_x = 1;
  size_t partial_bytes = 0;  // split partials of V, fp32 [ksplit][n_rows][rank]
};

// Aim for about four shrink workgroups (row tile x H1 chunk) per CU.
// Expand: when row tiles are mostly full, a chunk is bandwidth-bound and
// about four workgroups per CU (dispatched as slots free up) hide latency
// best.  When they are mostly short (decode-like rows of many LoRAs), the
// expand takes 16-row tiles and three 128-column chunks per workgroup: a sweep
// of 1 to 10 chunks on 256 rows in 34 segments (r = 64, H = 5120 and 13824)
// found 3 best, about 1.5% ahead of a grid sized to be resident at once.
constexpr int kMfmaShrinkTarget = 1024;
constexpr int kMfmaExpandTarget = 1024;
constexpr int kMfmaShortTileRows = 32;   // mean rows per 64-row tile below which tiles count as short
constexpr int kMfmaShortExpandRows = 16; // expand tile rows for short tiles
constexpr int kMfmaShortChunksPerWg = 3;

int64_t units_for(const sgmv_problem_t& p, int rows, int* direct) {
  if (p.max_seg_len <= rows) {
    *direct = 1;
    return p.num_segs;
  }
  *direct = 0;
  return std::min<int64_t>((int64_t)p.num_segs * ceil_div(p.max_seg_len, rows), ceil_div(p.n_rows, rows) + p.num_segs);
}

MfmaPlan plan_mfma(const sgmv_problem_t& p) {
  MfmaPlan m;
  m.units64 = units_for(p, sgmv::kMfmaRowsPerTile, &m.direct64);
  // The H1 split multiplies the workgroups, but every split writes (and the
  // reduce reads) one fp32 plane of V: keep that traffic within a quarter of
  // what the shrink must read anyway (X, plus A_k once per segment).
  const int64_t units = std::max<int64_t>(m.units64, 1);
  const double must_read = 2.0 * (double)p.n_rows * p.h_in + 2.0 * (double)p.num_segs * p.h_in * p.rank;
  const double per_split = 8.0 * (double)p.n_rows * p.rank;
  const int64_t ks_traffic = std::max<int64_t>(1, (int64_t)(0.25 * must_read / std::max(per_split, 1.0)));
  const int64_t ks = std::max<int64_t>(1, std::min<int64_t>({ceil_div(kMfmaShrinkTarget, units), ks_traffic,
                                                             ceil_div(p.h_in, sgmv::kMfmaKChunk)}));
  m.kc = (int)round_up(ceil_div(p.h_in, ks), sgmv::kMfmaKChunk);
  m.ksplit = (int)ceil_div(p.h_in, m.kc);
  const int64_t nchunks = ceil_div(p.h_out, sgmv::kMfmaColsPerTile);
  m.units_x = m.units64;
  m.direct_x = m.direct64;
  if ((int64_t)p.n_rows < kMfmaShortTileRows * units) {
    // Short tiles: 16-row expand tiles (all four waves compute), a few chunks
    // per workgroup.
    m.expand_rows = kMfmaShortExpandRows;
    m.units_x = units_for(p, kMfmaShortExpandRows, &m.direct_x);
    m.chunks_per_wg = (int)std::min<int64_t>(nchunks, kMfmaShortChunksPerWg);
  } else {
    const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(nchunks, kMfmaExpandTarget / units));
    m.chunks_per_wg = (int)ceil_div(nchunks, groups);
  }
  m.partial_bytes = (size_t)m.ksplit * (size_t)p.n_rows * p.rank * sizeof(float);
  return m;
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
  return q;
}


bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }
bool aligned2(const void* p) { return ((uintptr_t)p & 1u) == 0; }

bool nothing_to_do(const sgmv_problem_t& p) {
  return p.num_segs == 0 || p.n_rows == 0 || p.max_seg_len == 0;
}

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

size_t apply_ws_bytes(const sgmv_problem_t& p) {
  const VecPlan v = plan_vec(p, kTargetWorkgroups);
  const size_t two_launch = vec_ws_bytes(v, p.rank) + v_area_bytes(p);
  const size_t one_launch = SGMV_WS_COUNTER_BYTES + decode_ws_bytes(p);
  const size_t matrix = sgmv::mfma_supported(p.rank)
                            ? SGMV_WS_COUNTER_BYTES + plan_mfma(p).partial_bytes + v_area_bytes(p)
                            : 0;
  return std::max({two_launch, one_launch, matrix});
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

// sgmv_lora_apply for num_proj projections that share X, the shapes and the
// segments.  Projection i uses the workspace slice [i*stride, i*stride + need).
sgmv_status_t apply(const sgmv_problem_t& p, const void* X, const sgmv_projection_t* pj, int np,
                    const int32_t* seg_indptr, const int32_t* lora_idx, const int32_t* row_idx, char* ws,
                    size_t stride, hipStream_t s) {
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
        const sgmv_status_t st =
            apply(p, X, pj + i, 1, seg_indptr, lora_idx, row_idx, ws + (size_t)i * stride, stride, s);
        if (st != SGMV_OK) return st;
      }
      return SGMV_OK;
    }
    sgmv::DecodeParams q{};
    q.X = static_cast<const uint16_t*>(X);
    for (int i = 0; i < np; ++i) q.proj[i] = kernel_projection(pj[i]);
    q.seg_indptr = seg_indptr;
    q.lora_idx = lora_idx;
    q.row_idx = row_idx;
    q.slots = reinterpret_cast<uint64_t*>(ws + SGMV_WS_COUNTER_BYTES);
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
    hipError_t e = sgmv::launch_vec(p.dtype, p.rank, v.rb, sgmv::kModeShrink, q, s);
    if (e != hipSuccess) return SGMV_ERR_HIP;
    e = sgmv::launch_vec(p.dtype, p.rank, v.rb, sgmv::kModeExpand, q, s);
    if (e != hipSuccess) return SGMV_ERR_HIP;
  }
  return SGMV_OK;
}

}  // namespace

// Base projection with the LoRA term: W strips of kBaseStripCols columns,
// split over K into fp32 partial planes so that about kBaseTarget workgroups
// stream W at once.  A sweep of strips (64, 128, 256 columns) against targets
// (128 to 1024) on 32-row batches (H = 4096 and 11008 -> 4096) found 128 x 256
// best: more splits write (and the epilogue reads) more partial planes.
constexpr int kBaseStripCols = 128;
constexpr int kBaseTarget = 256;

struct BasePlan {
  int strip_cols = kBaseStripCols;
  int strips = 0;
  int ksplit = 1;
  int kc = 0;
  int base_grid = 0;
  size_t b_off = 0, v_off = 0, p_off = 0, total = 0;  // workspace layout
};

BasePlan plan_base(const sgmv_problem_t& p, bool packed) {
  BasePlan b;
  b.strips = (int)ceil_div(p.h_out, b.strip_cols);
  const int64_t max_split = ceil_div(p.h_in, sgmv::kBaseStageRows);
  const int64_t ks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(kBaseTarget, b.strips), max_split));
  b.kc = (int)round_up(ceil_div(p.h_in, ks), sgmv::kBaseStageRows);
  if (packed && p.n_rows > 32) {
    // The packed-W kernel stages the X chunk of its four row tiles (64 x kc) in LDS.
    const int64_t cap = sgmv::kBasePackedXElems / 64 / sgmv::kBaseStageRows * sgmv::kBaseStageRows;
    b.kc = (int)std::min<int64_t>(b.kc, cap);
  }
  b.ksplit = (int)ceil_div(p.h_in, b.kc);
  b.base_grid = (int)round_up((int64_t)b.strips * b.ksplit, 8);
  // [B_k of each row][partial planes of V][partial planes of Y]
  b.b_off = 0;
  b.v_off = (size_t)round_up((int64_t)p.n_rows * (int64_t)sizeof(uint64_t), 256);
  b.p_off = b.v_off + (size_t)round_up((int64_t)b.ksplit * p.n_rows * p.rank * (int64_t)sizeof(float), 256);
  b.total = b.p_off + (size_t)b.ksplit * (size_t)p.n_rows * (size_t)p.h_out * sizeof(float);
  return b;
}

extern "C" {

const char* sgmv_status_str(sgmv_status_t status) {
  switch (status) {
    case SGMV_OK: return "SGMV_OK";
    case SGMV_ERR_INVALID_ARG: return "SGMV_ERR_INVALID_ARG: invalid argument";
    case SGMV_ERR_UNSUPPORTED: return "SGMV_ERR_UNSUPPORTED: shape, rank, dtype or alignment not supported";
    case SGMV_ERR_WORKSPACE: return "SGMV_ERR_WORKSPACE: workspace missing or too small";
    case SGMV_ERR_HIP: return "SGMV_ERR_HIP: HIP runtime or launch failure";
  }
  return "SGMV_ERR_UNKNOWN";
}

sgmv_status_t sgmv_build_segments(const int32_t* req_lora, int32_t n, int32_t num_loras,
                                  int32_t* perm, int32_t* seg_indptr, int32_t* lora_idx,
                                  int32_t* num_segs, int32_t* max_seg_len) {
  if (n < 0 || num_loras < 1 || !seg_indptr || !num_segs || !max_seg_len) return SGMV_ERR_INVALID_ARG;
  if (n > 0 && (!req_lora || !perm || !lora_idx)) return SGMV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (req_lora[i] < 0 || req_lora[i] >= num_loras) return SGMV_ERR_INVALID_ARG;
  seg_indptr[0] = 0;
  int32_t S = 0, longest = 0;
  if ((int64_t)num_loras <= 4 * (int64_t)n + 1024) {
    // Counting sort: O(n + num_loras), stable.
    std::vector<int32_t> start((size_t)num_loras + 1, 0);
    for (int32_t i = 0; i < n; ++i) ++start[(size_t)req_lora[i] + 1];
    for (int32_t k = 0; k < num_loras; ++k) {
      const int32_t c = start[(size_t)k + 1];
      if (c > 0) {
        lora_idx[S] = k;
        seg_indptr[S + 1] = seg_indptr[S] + c;
        longest = std::max(longest, c);
        ++S;
      }
      start[(size_t)k + 1] += start[(size_t)k];
    }
    for (int32_t i = 0; i < n; ++i) perm[start[(size_t)req_lora[i]]++] = i;
  } else {
    // Sparse ids: stable comparison sort, O(n log n).
    std::vector<std::pair<int32_t, int32_t>> key((size_t)n);
    for (int32_t i = 0; i < n; ++i) key[(size_t)i] = {req_lora[i], i};
    std::sort(key.begin(), key.end());
    for (int32_t j = 0; j < n; ++j) {
      perm[j] = key[(size_t)j].second;
      if (j == 0 || key[(size_t)j].first != key[(size_t)j - 1].first) {
        if (j > 0) seg_indptr[S] = j;
        lora_idx[S++] = key[(size_t)j].first;
      }
    }
    if (n > 0) seg_indptr[S] = n;
    for (int32_t s = 0; s < S; ++s) longest = std::max(longest, seg_indptr[s + 1] - seg_indptr[s]);
  }
  *num_segs = S;
  *max_seg_len = longest;
  return SGMV_OK;
}

sgmv_status_t sgmv_check_problem(const sgmv_problem_t* p) {
  if (!p) return SGMV_ERR_INVALID_ARG;
  if (p->n_rows < 0 || p->h_in <= 0 || p->h_out <= 0 || p->num_segs < 0 || p->num_loras < 0 ||
      p->max_seg_len < 0 || p->max_seg_len > p->n_rows || p->splits < 0)
    return SGMV_ERR_INVALID_ARG;
  if (p->num_segs > 0 && p->num_loras < 1) return SGMV_ERR_INVALID_ARG;
  if (p->variant < SGMV_VARIANT_AUTO || p->variant > SGMV_VARIANT_MFMA) return SGMV_ERR_INVALID_ARG;
  if (p->dtype != SGMV_F16 && p->dtype != SGMV_BF16) return SGMV_ERR_UNSUPPORTED;
  if (!rank_supported(p->rank)) return SGMV_ERR_UNSUPPORTED;
  if (p->h_in % 8 != 0 || p->h_out % 8 != 0) return SGMV_ERR_UNSUPPORTED;
  if (p->variant == SGMV_VARIANT_MFMA && !sgmv::mfma_supported(p->rank)) return SGMV_ERR_UNSUPPORTED;
  const VecPlan v = plan_vec(*p, kTargetWorkgroups);
  if (2 * v.num_units > kCounterSlots) return SGMV_ERR_UNSUPPORTED;
  return SGMV_OK;
}

sgmv_status_t sgmv_check_segments(const sgmv_problem_t* p, const int32_t* seg_indptr_host,
                                  const int32_t* lora_idx_host) {
  if (!p) return SGMV_ERR_INVALID_ARG;
  if (p->num_segs < 0) return SGMV_ERR_INVALID_ARG;
  if (!seg_indptr_host || (p->num_segs > 0 && !lora_idx_host)) return SGMV_ERR_INVALID_ARG;
  if (seg_indptr_host[0] != 0) return SGMV_ERR_INVALID_ARG;
  for (int32_t s = 0; s < p->num_segs; ++s) {
    const int32_t len = seg_indptr_host[s + 1] - seg_indptr_host[s];
    if (len < 0 || len > p->max_seg_len) return SGMV_ERR_INVALID_ARG;
    if (lora_idx_host[s] < 0 || lora_idx_host[s] >= p->num_loras) return SGMV_ERR_INVALID_ARG;
  }
  if (seg_indptr_host[p->num_segs] > p->n_rows) return SGMV_ERR_INVALID_ARG;
  return SGMV_OK;
}

sgmv_status_t sgmv_workspace_bytes(const sgmv_problem_t* p, size_t* bytes) {
  if (!bytes) return SGMV_ERR_INVALID_ARG;
  const sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  *bytes = apply_ws_bytes(*p);
  return SGMV_OK;
}

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
      info->launches = 3;
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

sgmv_status_t sgmv_lora_apply(const sgmv_problem_t* p, const void* X, const void* const* A_ptrs,
                              const void* const* B_ptrs, void* Y, const int32_t* seg_indptr,
                              const int32_t* lora_idx, void* ws, size_t ws_bytes, void* stream) {
  const sgmv_projection_t one{A_ptrs, B_ptrs, Y, nullptr, nullptr};
  return sgmv_lora_apply_batched(p, X, &one, 1, seg_indptr, lora_idx, nullptr, ws, ws_bytes, stream);
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
  const size_t need = apply_ws_bytes(*p);
  const size_t stride = (size_t)round_up((int64_t)need, 256);
  if (ws_bytes < stride * (size_t)(num_projections - 1) + need) return SGMV_ERR_WORKSPACE;
  return apply(*p, X, projections, num_projections, seg_indptr, lora_idx, row_idx, static_cast<char*>(ws),
               stride, static_cast<hipStream_t>(stream));
}

sgmv_status_t sgmv_base_workspace_bytes(const sgmv_problem_t* p, size_t* bytes) {
  if (!bytes) return SGMV_ERR_INVALID_ARG;
  const sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (p->n_rows > sgmv::kBaseMaxRows) return SGMV_ERR_UNSUPPORTED;
  *bytes = std::max(plan_base(*p, false).total, plan_base(*p, true).total);
  return SGMV_OK;
}

}  // extern "C"

namespace {

// Bytes of the packed layout of W [h_in, h_out]: 16-column blocks (an even
// count) of ceil(h_in / 128) * 4 k-steps of 1 KiB each.
int64_t packed_ksteps(int64_t h_in) { return ceil_div(h_in, 128) * 4; }
int64_t packed_bytes(int64_t h_in, int64_t h_out) {
  return round_up(ceil_div(h_out, 16), 2) * packed_ksteps(h_in) * 1024;
}

sgmv_status_t base_apply(const sgmv_problem_t* p, const void* X, const void* W, bool packed,
                         const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                         const int32_t* seg_indptr, const int32_t* lora_idx, void* ws, size_t ws_bytes,
                         void* stream) {
  sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (p->n_rows > sgmv::kBaseMaxRows) return SGMV_ERR_UNSUPPORTED;
  if (p->n_rows == 0) return SGMV_OK;
  if (!X || !W || !Y) return SGMV_ERR_INVALID_ARG;
  const bool lora = !nothing_to_do(*p);
  if (lora && (!A_ptrs || !B_ptrs || !seg_indptr || !lora_idx)) return SGMV_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y)) return SGMV_ERR_UNSUPPORTED;
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
  q.Y = static_cast<uint16_t*>(Y);
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

sgmv_status_t sgmv_base_packed_weight_bytes(int32_t h_in, int32_t h_out, size_t* bytes) {
  if (!bytes || h_in <= 0 || h_out <= 0) return SGMV_ERR_INVALID_ARG;
  *bytes = (size_t)packed_bytes(h_in, h_out);
  return SGMV_OK;
}

sgmv_status_t sgmv_base_pack_weight(const void* W, int32_t h_in, int32_t h_out, void* Wp, size_t wp_bytes,
                                    void* stream) {
  if (!W || !Wp || h_in <= 0 || h_out <= 0) return SGMV_ERR_INVALID_ARG;
  if (wp_bytes < (size_t)packed_bytes(h_in, h_out)) return SGMV_ERR_WORKSPACE;
  if (!aligned2(W) || !aligned16(Wp)) return SGMV_ERR_UNSUPPORTED;
  return hip_status(sgmv::launch_base_pack(static_cast<const uint16_t*>(W), h_in, h_out,
                                           static_cast<uint16_t*>(Wp), static_cast<hipStream_t>(stream)));
}

sgmv_status_t sgmv_base_lora_apply_packed(const sgmv_problem_t* p, const void* X, const void* Wp,
                                          const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                                          const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                                          size_t ws_bytes, void* stream) {
  return base_apply(p, X, Wp, true, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, ws_bytes, stream);
}

}  // extern "C"
