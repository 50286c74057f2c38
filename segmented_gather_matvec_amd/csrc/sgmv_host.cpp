// sgmv_host.cpp - host-only part of libsgmv: the segment builder, the problem
// and metadata checks, and the shape plans and workspace sizes of every
// kernel family.  No HIP calls: everything here runs without a device (and is
// what the host sanitizer build exercises).
#include "sgmv_host.h"

#include <algorithm>
#include <utility>
#include <vector>

namespace sgmv_host {

namespace {

int pick_rb(int max_seg_len) { return max_seg_len <= 1 ? 1 : (max_seg_len <= 4 ? 4 : 16); }

// Units of at most `rows` rows of one segment: one per segment when every
// segment fits one block (direct), else an upper bound from max_seg_len.
int64_t units_for(const sgmv_problem_t& p, int rows, int* direct) {
  if (p.max_seg_len <= rows) {
    *direct = 1;
    return p.num_segs;
  }
  *direct = 0;
  return std::min<int64_t>((int64_t)p.num_segs * ceil_div(p.max_seg_len, rows), ceil_div(p.n_rows, rows) + p.num_segs);
}

}  // namespace

VecPlan plan_vec(const sgmv_problem_t& p, int64_t target_wgs) {
  VecPlan v;
  v.rb = pick_rb(p.max_seg_len);
  int direct = 1;
  v.num_units = units_for(p, v.rb, &direct);
  v.direct = direct;
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

size_t v_area_bytes(const sgmv_problem_t& p) {
  return (size_t)round_up((int64_t)p.n_rows * p.rank * (int64_t)sizeof(float), 256);
}

DecodePlan plan_decode_rb(const sgmv_problem_t& p, int rb, int split_major) {
  DecodePlan d;
  d.rb = rb;
  d.split_major = split_major;
  if (!sgmv::decode_supported(p.rank, d.rb)) return d;
  int direct = 1;
  d.num_units = units_for(p, d.rb, &direct);
  d.direct = direct;
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

// Blocks of one row keep the most workgroups busy; when segments hold several
// rows (rows that share a LoRA), the split-major mapping puts equal splits of
// neighbouring units on one XCD, so a segment's rows re-read their A_k / B_k
// slice from that XCD's L2 rather than from HBM.  Segments of one row keep a
// unit on one XCD.
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

size_t decode_slot_bytes(const sgmv_problem_t& p) {
  DecodePlan c[3];
  const int n = decode_candidates(p, c);
  // With long segments the decode route is taken only when one launch holds
  // every unit; otherwise the smallest row block may run in passes.
  const int64_t limit = stage_uses_mfma(p) ? kMaxResidentGrid : kMaxDecodeRounds * kMaxResidentGrid;
  size_t b = 0;
  for (int i = 0; i < n; ++i)
    if (c[i].grid <= limit || (i == 0 && !stage_uses_mfma(p) && c[i].num_units * c[i].splits <= limit))
      b = std::max(b, c[i].slot_bytes);
  return b;
}

bool stage_uses_mfma(const sgmv_problem_t& p) {
  if (!sgmv::mfma_supported(p.rank)) return false;
  if (p.variant == SGMV_VARIANT_MFMA) return true;
  return p.variant == SGMV_VARIANT_AUTO && p.max_seg_len > 16;
}

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
constexpr int kMfmaLowRankExpandRows = 32;  // expand tile rows for full tiles at rank <= 16
constexpr int kMfmaShortChunksPerWg = 3;

MfmaPlan plan_mfma(const sgmv_problem_t& p) {
  MfmaPlan m;
  int direct = 1;
  m.units64 = units_for(p, sgmv::kMfmaRowsPerTile, &direct);
  m.direct64 = direct;
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
    m.units_x = units_for(p, kMfmaShortExpandRows, &direct);
    m.direct_x = direct;
    m.chunks_per_wg = (int)std::min<int64_t>(nchunks, kMfmaShortChunksPerWg);
  } else {
    // Full tiles: the shrink stages X through LDS, whole row pieces per load
    // (mixed r = 64 batches, shrink: 11008 -> 4096 50.2 -> 43.3 us, 4096 ->
    // 11008 21.9 -> 18.1 us).  Short tiles keep X in registers: the LDS stage
    // adds latency to every stage of their few-stage workgroups (13B shapes,
    // 13824 -> 5120 shrink: 17.0 -> 18.4 us through LDS).
    m.x_lds = 1;
    // Full tiles: each tile re-reads its B_k slice, r x 2 bytes per output per
    // tile row.  At rank <= 16 that is cheap, and 32-row tiles (twice the
    // workgroups) won: 78.9 -> 72.7 us on the mixed r = 16 4096 -> 11008 batch,
    // equal at 11008 -> 4096; at rank 64 they lost 4-10%.
    if (p.rank <= 16) {
      m.expand_rows = kMfmaLowRankExpandRows;
      m.units_x = units_for(p, kMfmaLowRankExpandRows, &direct);
      m.direct_x = direct;
    }
    const int64_t ux = std::max<int64_t>(m.units_x, 1);
    const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(nchunks, kMfmaExpandTarget / ux));
    m.chunks_per_wg = (int)ceil_div(nchunks, groups);
  }
  m.partial_bytes = (size_t)m.ksplit * (size_t)p.n_rows * p.rank * sizeof(float);
  // The first workgroups of the expand launch sum the planes (1024 / rank rows
  // each, 512 / rank beyond 16 planes); the reduce launch remains for the
  // standalone shrink.  This beat each expand workgroup summing the planes of
  // its own rows (which re-reads them once per column group) at every split:
  // mixed r = 64, 4096 -> 11008 (4 planes) 85.3 -> 83.0 us per call, r = 16
  // 11008 -> 4096 (9 planes) 53.9 -> 53.4 us, the other shapes equal.
  m.lead = m.ksplit > 1 ? 1 : 0;
  m.lead_rows = m.ksplit > 16 ? 512 / p.rank : 1024 / p.rank;
  m.lead_blocks = (int)round_up(ceil_div(p.n_rows, m.lead_rows), 8);
  m.vt_bytes = m.lead ? (size_t)round_up((int64_t)p.n_rows * p.rank * (int64_t)sizeof(uint64_t), 256) : 0;
  return m;
}

WsLayout apply_ws_layout(const sgmv_problem_t& p) {
  const VecPlan v = plan_vec(p, kTargetWorkgroups);
  const size_t two_launch = vec_ws_bytes(v, p.rank) + v_area_bytes(p);
  const size_t matrix =
      sgmv::mfma_supported(p.rank) ? SGMV_WS_COUNTER_BYTES + plan_mfma(p).partial_bytes + v_area_bytes(p) : 0;
  WsLayout w;
  w.decode_off = (size_t)round_up((int64_t)std::max(two_launch, matrix), 256);
  // Tagged words only in areas of their own: a stale word there is a tag of
  // an earlier launch, never another route's fp32 data posing as one.
  w.lead_off = (size_t)round_up((int64_t)(w.decode_off + decode_slot_bytes(p)), 256);
  w.total = w.lead_off + (sgmv::mfma_supported(p.rank) ? plan_mfma(p).vt_bytes : 0);
  return w;
}

// Base projection: W strips of kBaseStripCols columns, split over K into fp32
// partial planes so that about kBaseTarget workgroups stream W at once.  A
// sweep of strips (64, 128, 256 columns) against targets (128 to 1024) on
// 32-row batches (H = 4096 and 11008 -> 4096) found 128 x 256 best: more
// splits write (and the epilogue reads) more partial planes.  Narrow outputs
// (a column shard of a tensor-parallel layer, 4096 -> 512) would take 32
// splits for 256 workgroups; capped at 8 the row-major and packed calls took
// 11.6 / 11.9 us instead of 16.5 / 17.0 us (the epilogue sums fewer planes;
// caps of 4 and 16 were slower for one layout or the other).  Both layouts
// share the cap, so they keep splitting K alike.  Full-width outputs already
// stay below it.
constexpr int kBaseStripCols = 128;
constexpr int kBaseTarget = 256;
constexpr int kBaseMaxSplit = 8;

static_assert(sgmv::kBaseMaxRows == SGMV_BASE_MAX_ROWS, "one row limit for the base projection");

BasePlan plan_base(const sgmv_problem_t& p, bool packed) {
  BasePlan b;
  b.strip_cols = kBaseStripCols;
  b.strips = (int)ceil_div(p.h_out, b.strip_cols);
  const int64_t max_split = ceil_div(p.h_in, sgmv::kBaseStageRows);
  const int64_t ks = std::max<int64_t>(1, std::min<int64_t>({ceil_div(kBaseTarget, b.strips), max_split,
                                                             (int64_t)kBaseMaxSplit}));
  b.kc = (int)round_up(ceil_div(p.h_in, ks), sgmv::kBaseStageRows);
  if (packed && p.n_rows > 32) {
    // The packed-W kernel stages the X chunk of its four or eight row tiles
    // (64 or 128 rows x kc) in LDS.
    const int64_t rows = p.n_rows > 64 ? 128 : 64;
    const int64_t cap = sgmv::base_packed_x_elems((int)rows) / rows / sgmv::kBaseStageRows * sgmv::kBaseStageRows;
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

int64_t packed_ksteps(int64_t h_in) { return ceil_div(h_in, 128) * 4; }
int64_t packed_bytes(int64_t h_in, int64_t h_out) {
  return round_up(ceil_div(h_out, 16), 2) * packed_ksteps(h_in) * 1024;
}

}  // namespace sgmv_host

using namespace sgmv_host;

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
  if (p->h_in > SGMV_MAX_HIDDEN || p->h_out > SGMV_MAX_HIDDEN) return SGMV_ERR_UNSUPPORTED;
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
    const int64_t len = (int64_t)seg_indptr_host[s + 1] - seg_indptr_host[s];
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
  *bytes = apply_ws_layout(*p).total;
  return SGMV_OK;
}

sgmv_status_t sgmv_base_workspace_bytes(const sgmv_problem_t* p, size_t* bytes) {
  if (!bytes) return SGMV_ERR_INVALID_ARG;
  const sgmv_status_t st = sgmv_check_problem(p);
  if (st != SGMV_OK) return st;
  if (p->n_rows > sgmv::kBaseMaxRows) return SGMV_ERR_UNSUPPORTED;
  *bytes = std::max(plan_base(*p, false).total, plan_base(*p, true).total);
  return SGMV_OK;
}

sgmv_status_t sgmv_base_packed_weight_bytes(int32_t h_in, int32_t h_out, size_t* bytes) {
  if (!bytes || h_in <= 0 || h_out <= 0) return SGMV_ERR_INVALID_ARG;
  if (h_in > SGMV_MAX_HIDDEN || h_out > SGMV_MAX_HIDDEN) return SGMV_ERR_UNSUPPORTED;
  *bytes = (size_t)packed_bytes(h_in, h_out);
  return SGMV_OK;
}

}  // extern "C"
