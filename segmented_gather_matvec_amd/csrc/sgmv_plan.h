// sgmv_plan.h - host-side interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Rows of A_k covered by one pass of the shrink loop and columns of B_k covered
// by one pass of the expand loop (two 128-bit loads per thread per pass).
constexpr int vec_rows_per_pass(int rank) { return 256 * 2 * 8 / rank; }
constexpr int vec_cols_per_pass(int rank) { return 256 * 2 * 8 / rank; }

// Launch one vector kernel; returns the HIP error of the launch.
hipError_t launch_vec(int dtype, int rank, int rb, int mode, const VecParams& p, hipStream_t stream);

// One-launch decode kernel (shrink, on-chip hand-off, expand).
// A_k rows (one 128-bit vector each) per thread.  Ranks 32 and 64 take 8, so
// that H1 = 4096 needs 16 splits instead of 32 (a rank-64 batch of 32 rows
// then fits on the device at once: 9.9 us instead of 23.6 us on the two-launch
// route); rank 16 is fastest at 4 (8 was 0.1-0.8 us slower on every batch).
constexpr int decode_rows_per_thread(int rank) { return rank >= 32 ? 8 : 4; }
constexpr int kDecodeLanesPerColumn = 4;  // lanes sharing one 8-column vector of B_k
constexpr int decode_max_kc(int rank) { return decode_rows_per_thread(rank) * 256 / (rank / 8); }
constexpr int decode_max_cw() { return 256 / kDecodeLanesPerColumn * 8; }

// One projection of a batched call (its own LoRA tables and output); the
// projection of a workgroup is blockIdx.y.
constexpr int kMaxProjections = 4;
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
  int32_t pad_;
  const int32_t* seg_indptr;
  const int32_t* lora_idx;
  const int32_t* row_idx;  // null, or row of X / Y of each sorted row
  uint64_t* slots;      // projection 0: [num_units][splits][parts][RB*rank] tagged partials
  int64_t slot_stride;  // words between the slot areas of consecutive projections
  const uint16_t* X;
  Projection proj[kMaxProjections];
};

bool decode_supported(int rank, int rb);
// Launches num_proj projections (blockIdx.y).
hipError_t launch_decode(int dtype, int rank, int rb, const DecodeParams& p, int num_proj, hipStream_t stream);
// Workgroups of the decode kernel variant that fit on the device at once (0 if
// unknown).
// small: at most 64 LoRAs; map: a row map; het: rank or scale tables.
int decode_resident_capacity(int dtype, int rank, int rb, bool small, bool map, bool het);

// Matrix-core kernels for long segments: shrink (+ reduce of the H1 split),
// then expand.
constexpr int kMfmaRowsPerTile = 64;      // rows of one segment per shrink / expand workgroup
constexpr int kMfmaColsPerTile = 128;     // output columns per expand chunk
constexpr int kMfmaKChunk = 256;          // H1 granule of the shrink's split

struct MfmaParams {
  int32_t n_rows, h_in, h_out, num_segs, num_loras;
  int32_t num_units64, direct_units64;  // units of <= 64 rows of one segment
  int32_t ksplit, kc, chunks_per_wg;
  // Expand tiles of expand_rows (16 or 64) rows of one segment: num_units_x of them.
  int32_t expand_rows, num_units_x, direct_units_x, pad_;
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

bool mfma_supported(int rank);
// Shrink into the partial planes, then reduce them into V (two launches).
hipError_t launch_mfma_shrink(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream);
hipError_t launch_mfma_expand(int dtype, int rank, const MfmaParams& p, int num_proj, hipStream_t stream);

// Base projection with the LoRA term (batches of at most kBaseMaxRows rows):
// split-K partial planes of X @ W on the matrix cores (strips of strip_cols
// columns) and of V = X @ A_k in one launch, then an epilogue that sums them,
// adds V @ B_k and rounds once.
constexpr int kBaseMaxRows = 64;
constexpr int kBaseStageRows = 128;  // W rows per pipeline stage (kc is a multiple)
// LDS of the packed-W partial kernel's X chunk (16-bit elements, 64 KiB):
// rows (16 per row tile) x K chunk may not exceed it.
constexpr int kBasePackedXElems = 32768;

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
  uint16_t* Y;             // [n_rows, h_out], written
};

// Partials then epilogue (two launches).
hipError_t launch_base(int dtype, int rank, const BaseParams& p, hipStream_t stream);
// W [h_in, h_out] row-major -> the packed layout (one launch).
hipError_t launch_base_pack(const uint16_t* W, int h_in, int h_out, uint16_t* Wp, hipStream_t stream);

}  // namespace sgmv
