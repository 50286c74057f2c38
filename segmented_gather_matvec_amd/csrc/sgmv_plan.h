// sgmv_plan.h - host-side interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgmv_shapes.h"

namespace sgmv {

// Vector (split-K) kernels: one template, two modes.
enum VecMode : int {
  kModeShrink = 0,  // V = X @ A_k (partials reduced by the last-arriving workgroup)
  kModeExpand = 1   // Y += V @ B_k
};

// A "unit" is one row block (<= RB rows) of one segment; each unit is worked by
// `splits` workgroups, split g covering input rows [g*kc, (g+1)*kc) of A_k in
// the shrink and output columns [g*cw, (g+1)*cw) of B_k in the expand.
struct VecParams {
  const uint16_t* X;
  const uint64_t* A_ptrs;
  const uint64_t* B_ptrs;
  uint16_t* Y;
  float* V;
  const int32_t* seg_indptr;
  const int32_t* lora_idx;
  const int32_t* row_idx;  // null, or row of X / Y of each sorted row
  const int32_t* ranks;    // null, or rank of each LoRA (A_k [h_in, r_k], B_k [r_k, h_out])
  const float* scales;     // null, or scale of each LoRA's term (applied to V by the shrink)
  float* partials;     // [num_units][splits][RB][rank] fp32
  uint32_t* counters;  // [2 * num_units]: arrivals, departures
  int32_t n_rows, h_in, h_out, num_segs, num_loras;
  int32_t num_units;     // units in the grid (an upper bound when not direct)
  int32_t splits;        // workgroups per unit
  int32_t kc;            // shrink input-row chunk per split, multiple of 8
  int32_t cw;            // expand column chunk per split, multiple of 8
  int32_t direct_units;  // 1: unit u is segment u (every segment fits one row block)
};

// Launch one vector kernel; returns the HIP error of the launch.
hipError_t launch_vec(int dtype, int rank, int rb, int mode, const VecParams& p, hipStream_t stream);
// Zero n 32-bit words with a fill kernel on `stream` (graph-capturable).
hipError_t launch_clear_u32(uint32_t* p, int64_t n, hipStream_t stream);

// One projection of a batched call (its own LoRA tables and output); the
// projection of a workgroup is blockIdx.y.
struct Projection {
  const uint64_t* A_ptrs;
  const uint64_t* B_ptrs;
  uint16_t* Y;
  const int32_t* ranks;  // null: every LoRA has the compiled rank
  const float* scales;   // null: scale 1
};


struct DecodeParams {
  // Scalars first and the pointers after them, so that the kernel fetches its
  // arguments in a few wide loads before its first metadata load.
  int32_t num_units, splits, kc, cw, direct_units;
  // 1: workgroup b runs split b % splits of unit b / splits, so the splits of a
  // unit go round-robin over the XCDs and equal splits of neighbouring units
  // (which read the same A_k / B_k slice when they share a LoRA) meet on one
  // XCD. 0: the splits of a unit share an XCD (grid padded to 8 units).
  int32_t split_major;
  int32_t n_rows, h_in, h_out, num_segs, num_loras;
  // This launch covers units unit_base .. unit_base + round_units - 1 (grid =
  // round_units * splits; round_units a multiple of 8 unless split_major).  One
  // launch covers all units when they fit on the device at once; otherwise the
  // host launches passes of round_units units.
  int32_t unit_base, round_units;
  // Longest wait for the unit's other partials, in ticks of the real-time
  // counter (0: give up at once, a test hook).
  uint32_t wait_ticks;
  const int32_t* seg_indptr;
  const int32_t* lora_idx;
  const int32_t* row_idx;  // null, or row of X / Y of each sorted row
  uint64_t* slots;      // projection 0: [num_units][splits][parts][RB*rank] tagged partials
  int64_t slot_stride;  // words between the slot areas of consecutive projections
  const uint16_t* X;
  uint32_t* errors;     // device error word: kDecodeErrWaitTimeout is set by a wait that gave up
  Projection proj[kMaxProjections];
};

// Error bit of the device error word: a workgroup gave up waiting for the
// partial sums of its unit (equal to SGMV_DEVICE_ERR_WAIT_TIMEOUT).
constexpr uint32_t kDecodeErrWaitTimeout = 1u;
// Address of the device error word on the current device (looked up once per
// device with hipGetSymbolAddress).
hipError_t decode_error_word(uint32_t** word);
// Launches num_proj projections (blockIdx.y).
hipError_t launch_decode(int dtype, int rank, int rb, const DecodeParams& p, int num_proj, hipStream_t stream);

// Segment metadata passed in the decode kernel's arguments (calls whose segment
// bounds and LoRA pointer tables are on the host): the bounds of at most
// kInlineSegs segments and the A_k / B_k of each segment.
constexpr int kInlineSegs = 64;
struct InlineMeta {
  int32_t seg[kInlineSegs + 1];
  uint64_t a[kInlineSegs];
  uint64_t b[kInlineSegs];
};
// One projection, no row map, no rank or scale tables; p's table pointers are
// not used.
hipError_t launch_decode_inline(int dtype, int rank, int rb, const DecodeParams& p, const InlineMeta& m,
                                hipStream_t stream);

// Workgroups of the decode kernel variant that fit on the device at once (0 if
// unknown).  variant: bit 0 at most 64 LoRAs, bit 1 a row map, bit 2 rank or
// scale tables; or kDecodeInlineVariant, the kernel with the metadata in its
// arguments.
constexpr int kDecodeInlineVariant = 8;
int decode_resident_capacity(int dtype, int rank, int rb, int variant);

// Matrix-core kernels for long segments: shrink (+ reduce of the H1 split),
// then expand.

struct MfmaParams {
  int32_t n_rows, h_in, h_out, num_segs, num_loras;
  int32_t num_units64, direct_units64;  // units of <= 64 rows of one segment
  int32_t ksplit, kc, chunks_per_wg;
  // Expand tiles of expand_rows (16, 32 or 64) rows of one segment: num_units_x of them.
  int32_t expand_rows, num_units_x, direct_units_x;
  // 1: the shrink stages X through LDS, loaded a whole row piece per
  // instruction (full row tiles); 0: X straight into the operand registers.
  int32_t x_lds;
  // 1 (ksplit > 1): no reduce launch; lead workgroups of the expand
  // launch sum the partial planes of their row blocks (lead_rows rows each,
  // lead_blocks blocks per projection, in plane order: the reduce's bits).
  // With 16-row expand tiles they publish V as tagged words {fp32, launch tag}
  // in the lead area, and the other workgroups poll the words of their rows
  // until every tag is the launch's; with larger tiles (each reading more of
  // V) they write V and then flags[block] = the launch tag in the lead area,
  // and the others wait for the flags of their rows, then read V.  Every wait
  // lasts at most wait_ticks of the real-time counter (0: give up at once).
  // Every grid row starts with lead_blocks * lead_proj workgroups: those of
  // row 0 do the lead work of all lead_proj projections, so that it is
  // dispatched ahead of every waiting workgroup; those of the other rows exit
  // at once.
  int32_t lead_reduce, lead_blocks, lead_rows, lead_proj;
  uint32_t wait_ticks;
  // Projection 0's lead area: [n_rows][rank] tagged words, or [lead_blocks]
  // flags; projection y's at lead_area + y * proj_stride * 4 bytes.
  void* lead_area;
  uint32_t* errors;        // device error word (a wait that gave up sets bit 0)
  const int32_t* seg_indptr;
  const int32_t* lora_idx;
  const int32_t* row_idx;  // null, or row of X / Y of each sorted row
  int64_t partial_stride;  // floats between partial planes (n_rows * rank)
  int64_t proj_stride;     // floats between the V / partial areas of consecutive projections
  const uint16_t* X;
  float* V;                // projection 0; reduce: output; expand: input (fp32 [n_rows, rank])
  float* partials;         // projection 0; shrink: H1-chunk s writes partials + s*partial_stride
  Projection proj[kMaxProjections];
};

// Shrink into the partial planes, then (unless the expand launch sums them, or
// V is the single plane itself) reduce them into V: one or two launches.
hipError_t launch_mfma_shrink(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream);
hipError_t launch_mfma_expand(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream);

// Base projection with the LoRA term (batches of at most kBaseMaxRows rows):
// split-K partial planes of X @ W on the matrix cores (strips of strip_cols
// columns) and of V = X @ A_k in one launch, then an epilogue that sums them,
// adds V @ B_k and rounds once.

struct BaseParams {
  int32_t n_rows, h_in, h_out, num_segs, num_loras;
  int32_t strip_cols;      // 64, 128 or 256
  int32_t strips;          // ceil(h_out / strip_cols)
  int32_t ksplit, kc;      // K split: plane g covers rows [g*kc, (g+1)*kc) of W and A_k
  int32_t base_grid;       // workgroups of the base product (a multiple of 8)
  int32_t shrink_grid;     // LoRA shrink workgroups before them (n_rows * ksplit, rounded up to 8; 0: none)
  int32_t packed_ksteps;   // 0: W row-major; else W in the packed layout with this many 32-row k-steps
  int64_t plane_stride;    // floats between partial planes of Y (n_rows * h_out)
  const int32_t* seg_indptr;
  const int32_t* lora_idx;
  const uint16_t* X;       // [n_rows, h_in]
  const uint16_t* W;       // [h_in, h_out] row-major, or packed (packed_ksteps > 0)
  const uint64_t* A_ptrs;  // [num_loras] -> A_k [h_in, rank]
  const uint64_t* B_ptrs;  // [num_loras] -> B_k [rank, h_out]
  float* vpartials;        // [ksplit][n_rows][rank] (null: no LoRA term)
  uint64_t* row_b;         // [n_rows] B_k of each row, 0 without a LoRA term (written by the shrink)
  float* partials;         // [ksplit][n_rows][h_out]
  uint16_t* Y;             // [n_rows, h_out], written rounded (when Yf is null)
  float* Yf;               // null, or [n_rows, h_out] fp32, written unrounded instead of Y
};

// Partials then epilogue (two launches).
hipError_t launch_base(int dtype, int rank, const BaseParams& p, hipStream_t stream);
// W [h_in, h_out] row-major -> the packed layout (one launch).
hipError_t launch_base_pack(const uint16_t* W, int h_in, int h_out, uint16_t* Wp, hipStream_t stream);

}  // namespace sgmv
