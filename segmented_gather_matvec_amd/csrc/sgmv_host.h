// sgmv_host.h - host-only planning and argument checks of libsgmv.
//
// Plain C++ with no HIP dependency: the kernel families' plans (row blocks,
// splits, tiles), the workspace layout and the problem checks are pure
// functions of the host-side shape summary, so they build and run (and are
// tested under the host sanitizers) without a device.  The device-dependent
// parts of planning (the decode kernel's co-resident capacity) live beside
// the launches.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/sgmv.h"
#include "sgmv_shapes.h"

namespace sgmv_host {

constexpr int64_t kCounterSlots = (int64_t)(SGMV_WS_COUNTER_BYTES / sizeof(uint32_t));
// Aim for this many workgroups per launch of the vector kernels: two per CU of
// a 256-CU MI355X keeps enough 128-bit loads in flight to cover HBM latency.
constexpr int kTargetWorkgroups = 512;
constexpr int kMaxSplits = 1024;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }
inline bool rank_supported(int r) { return r == 8 || r == 16 || r == 32 || r == 64; }
inline bool nothing_to_do(const sgmv_problem_t& p) {
  return p.num_segs == 0 || p.n_rows == 0 || p.max_seg_len == 0;
}

// Plan of one vector-kernel launch (split-K shrink or expand).
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
VecPlan plan_vec(const sgmv_problem_t& p, int64_t target_wgs);
// Counter area plus the shrink's split partials.
size_t vec_ws_bytes(const VecPlan& v, int rank);
// fp32 intermediate V [n_rows, rank] of the two-launch and matrix-core routes.
size_t v_area_bytes(const sgmv_problem_t& p);

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
DecodePlan plan_decode_rb(const sgmv_problem_t& p, int rb, int split_major);
// Candidate decode plans, smallest row block first; returns how many.
int decode_candidates(const sgmv_problem_t& p, DecodePlan out[3]);
// Passes (launches) of the decode kernel over the units beyond which the
// two-launch route is taken instead.
constexpr int64_t kMaxDecodeRounds = 4;
// Upper bound on the workgroups any supported device holds at once (8 per CU
// on 1024 CUs; an MI355X holds at most 2048): a decode plan whose launch
// exceeds it is never taken.
constexpr int64_t kMaxResidentGrid = 8192;
// Slot bytes of the largest candidate the decode route can take (on any
// device): the workspace is sized for it.
size_t decode_slot_bytes(const sgmv_problem_t& p);

// The matrix-core kernels take a stage when AUTO sees a segment longer than
// the decode kernel's row blocks (ranks 16..64), or when forced.
bool stage_uses_mfma(const sgmv_problem_t& p);

// Plan of the matrix-core kernels (long segments).
struct MfmaPlan {
  int64_t units64 = 0;
  int direct64 = 1;
  int ksplit = 1;
  int kc = 0;
  int chunks_per_wg = 1;
  int expand_rows = sgmv::kMfmaRowsPerTile;  // rows of one expand tile (16 for short tiles, 32 at rank <= 16)
  int64_t units_x = 0;                        // expand units of <= expand_rows rows
  int direct_x = 1;
  size_t partial_bytes = 0;  // split partials of V, fp32 [ksplit][n_rows][rank]
  int lead = 0;              // 1: lead workgroups of the expand launch sum the planes (ksplit > 1)
  int lead_blocks = 0;       // ... that many per projection (a multiple of 8)
  int lead_rows = 0;         // ... of that many rows each
  size_t vt_bytes = 0;       // their tagged V words or flags, after V in the workspace
  int x_lds = 0;             // 1: the shrink stages X through LDS (full row tiles)
};
MfmaPlan plan_mfma(const sgmv_problem_t& p);

// Workspace of one projection of sgmv_lora_apply(_batched):
//   [0, SGMV_WS_COUNTER_BYTES)   arrival counters of the two-launch shrink
//   [SGMV_WS_COUNTER_BYTES, decode_off)
//                                the vector shrink's split partials then V, or
//                                the matrix-core partial planes then V
//   [decode_off, lead_off)       the decode kernel's tagged slots, which no other
//                                route writes
//   [lead_off, total)            the matrix-core expand's lead area (tagged V
//                                words or row-block flags), which no other route
//                                writes either
struct WsLayout {
  size_t decode_off = 0;
  size_t lead_off = 0;  // the matrix-core expand's lead area (tagged V words or row-block flags)
  size_t total = 0;
};
WsLayout apply_ws_layout(const sgmv_problem_t& p);

// Base projection with the LoRA term: W strips split over K into fp32 partial
// planes, and the workspace layout [B_k of each row][V planes][Y planes].
struct BasePlan {
  int strip_cols = 0;
  int strips = 0;
  int ksplit = 1;
  int kc = 0;
  int base_grid = 0;
  size_t b_off = 0, v_off = 0, p_off = 0, total = 0;
};
BasePlan plan_base(const sgmv_problem_t& p, bool packed);
// Packed layout of W [h_in, h_out]: 16-column blocks (an even count) of
// ceil(h_in / 128) * 4 k-steps of 1 KiB each.
int64_t packed_ksteps(int64_t h_in);
int64_t packed_bytes(int64_t h_in, int64_t h_out);

}  // namespace sgmv_host
