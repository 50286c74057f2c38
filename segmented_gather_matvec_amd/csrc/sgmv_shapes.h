// sgmv_shapes.h - tile shapes of the libsgmv kernels that the host planners
// need, and the shapes each kernel family takes.  Plain C++ (no HIP): the
// host-only planning and validation code includes it too.
#pragma once

namespace sgmv {

constexpr int kWorkgroupThreads = 256;  // every kernel runs 4 wave64s per workgroup

// Vector kernels: rows of A_k covered by one pass of the shrink loop and
// columns of B_k covered by one pass of the expand loop (two 128-bit loads per
// thread per pass).
constexpr int vec_rows_per_pass(int rank) { return kWorkgroupThreads * 2 * 8 / rank; }
constexpr int vec_cols_per_pass(int rank) { return kWorkgroupThreads * 2 * 8 / rank; }

// One-launch decode kernel.  A_k rows (one 128-bit vector each) per thread.
// Ranks 32 and 64 take 8, so that H1 = 4096 needs 16 splits instead of 32 (a
// rank-64 batch of 32 rows then fits on the device at once: 9.9 us instead of
// 23.6 us on the two-launch route); rank 16 is fastest at 4 (8 was 0.1-0.8 us
// slower on every batch).
constexpr int decode_rows_per_thread(int rank) { return rank >= 32 ? 8 : 4; }
constexpr int kDecodeLanesPerColumn = 4;  // lanes sharing one 8-column vector of B_k
constexpr int decode_max_kc(int rank) { return decode_rows_per_thread(rank) * kWorkgroupThreads / (rank / 8); }
constexpr int decode_max_cw() { return kWorkgroupThreads / kDecodeLanesPerColumn * 8; }
// Instantiated (rank, rows per unit) pairs of the decode kernel: one output of
// V per thread.
constexpr bool decode_supported(int rank, int rb) {
  return rank * rb <= kWorkgroupThreads && (rb == 1 || rb == 4 || rb == 16);
}

// Projections of one batched call (blockIdx.y).
constexpr int kMaxProjections = 4;

// Matrix-core kernels for long segments.
constexpr int kMfmaRowsPerTile = 64;   // rows of one segment per shrink / expand workgroup
constexpr int kMfmaColsPerTile = 128;  // output columns per expand chunk
constexpr int kMfmaKChunk = 256;       // H1 granule of the shrink's split
constexpr bool mfma_supported(int rank) { return rank == 16 || rank == 32 || rank == 64; }

// Base projection with the LoRA term (batches of at most kBaseMaxRows rows).
constexpr int kBaseMaxRows = 128;  // SGMV_BASE_MAX_ROWS
constexpr int kBaseStageRows = 128;  // W rows per pipeline stage (kc is a multiple)
// LDS of the packed-W partial kernel's X chunk (16-bit elements): 64 KiB up
// to 64 rows, 128 KiB above (a K chunk of 512 at 128 rows; 256 took 42.1
// instead of 38.5 us per call at 128 rows, H = 4096).  Rows (16 per row tile)
// x K chunk may not exceed it.
constexpr int kBasePackedXElems = 32768;
constexpr int base_packed_x_elems(int rows) { return rows > 64 ? 2 * kBasePackedXElems : kBasePackedXElems; }

}  // namespace sgmv
