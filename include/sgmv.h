/*
 * sgmv.h - C ABI of libsgmv: Segmented Gather Matrix-Vector multiplication
 * (SGMV) for multi-LoRA batches on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The Punica README (page "Punica：多 LoRA 模型统一服务框架",
 * LoRA paragraph) gives a LoRA pair as A [H1, r] and B [r, H2] beside a
 * pretrained weight W [H1, H2]; a row vector x run through the finetuned layer
 * gives x@(W + A@B) = x@W + x@A@B.  The multi-LoRA paragraph of the same page
 * batches rows X = (x_1..x_n) where every row carries its own LoRA model, so
 * the layer output is X@W plus, row by row, x_i @ A_{id(i)} @ B_{id(i)}; its
 * SGMV paragraph names the kernel that computes that second term.  This
 * library computes only that LoRA term and adds it onto a Y that already holds
 * the caller's X@W:
 *
 *     for every segment s, k = lora_idx[s], rows i in [seg_indptr[s], seg_indptr[s+1]):
 *         V[i, :]  = X[i, :] @ A_k                 (shrink, fp32 result)
 *         Y[i, :] += V[i, :] @ B_k                 (expand)
 *
 * Rows are grouped into segments: contiguous row ranges that share one LoRA
 * ("Segmented"), whose weights are fetched through per-LoRA pointer tables
 * ("Gather").  No LoRA scale factor appears in the pages' formula; the scale
 * is 1 and a caller folds any alpha/r into B.
 *
 * Layouts (all row-major, contiguous, the logical shapes of the LoRA
 * paragraph with row-vector inputs):
 *   X   [n_rows, h_in]    dtype            (read)
 *   A_k [h_in,  rank]     dtype            (read; A_ptrs[k] points to it)
 *   B_k [rank,  h_out]    dtype            (read; B_ptrs[k] points to it)
 *   V   [n_rows, rank]    float32          (written by sgmv_shrink, read by sgmv_expand)
 *   Y   [n_rows, h_out]   dtype            (read-modify-write)
 *   seg_indptr [num_segs+1], lora_idx [num_segs]   int32
 *   A_ptrs, B_ptrs [num_loras]  arrays of device pointers (uint64)
 *
 * Memory: every pointer passed to a device entry point (X, V, Y, A_ptrs,
 * B_ptrs, the matrices they point to, seg_indptr, lora_idx, workspace) is
 * DEVICE memory on the current HIP device, owned by the caller; it must stay
 * alive until the stream work finishes.  X, V and Y must not alias each
 * other.  The library allocates nothing and keeps no per-call state.
 *
 * Precision: inputs are fp16 or bf16; products and sums are fp32; Y is
 * rounded once (round-to-nearest-even) from fp32 (Y + addend) on store.
 *
 * Segment metadata preconditions (device-resident, so not checked by the
 * device entry points; sgmv_check_segments checks a host copy):
 *   seg_indptr[0] = 0, seg_indptr non-decreasing, seg_indptr[num_segs] <= n_rows,
 *   every segment length <= max_seg_len, 0 <= lora_idx[s] < num_loras.
 * Segments may come in any LoRA order and a LoRA id may appear in several
 * segments; empty segments are no-ops; rows at or past seg_indptr[num_segs]
 * are left untouched.  A violated precondition gives unspecified values in
 * Y / V but no out-of-bounds access beyond what the pointer tables allow.
 *
 * Errors: every entry point returns sgmv_status_t and never throws.  Argument
 * checks run on the host before any HIP call; a launch failure returns
 * SGMV_ERR_HIP.  Device entry points are asynchronous on `stream` (a
 * hipStream_t; NULL = the default stream) and never synchronise.
 */
#ifndef SGMV_H
#define SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sgmv_status {
  SGMV_OK = 0,
  SGMV_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad metadata (host checks) */
  SGMV_ERR_UNSUPPORTED = 2,  /* rank, dtype, alignment or size outside what the kernels take */
  SGMV_ERR_WORKSPACE = 3,    /* workspace missing or smaller than sgmv_workspace_bytes */
  SGMV_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} sgmv_status_t;

typedef enum sgmv_dtype {
  SGMV_F16 = 0,   /* IEEE binary16 */
  SGMV_BF16 = 1   /* bfloat16 (upper half of binary32) */
} sgmv_dtype_t;

/* Kernel family.  AUTO picks per call from max_seg_len and rank; the others
 * force one family (tests use them to pin every variant to the oracle). */
typedef enum sgmv_variant {
  SGMV_VARIANT_AUTO = 0,
  SGMV_VARIANT_VECTOR = 1,  /* split-K vector kernels, one launch per stage */
  SGMV_VARIANT_FUSED = 2,   /* sgmv_lora_apply only: one persistent launch, shrink->expand handoff on chip */
  SGMV_VARIANT_MFMA = 3     /* matrix-core kernels for long (prefill) segments */
} sgmv_variant_t;

/* Largest hidden size (h_in, h_out) the kernels' plans take; larger sizes
 * give SGMV_ERR_UNSUPPORTED. */
#define SGMV_MAX_HIDDEN (1 << 20)

/* Host-side shape summary; the host never reads device memory to plan. */
typedef struct sgmv_problem {
  int32_t dtype;        /* sgmv_dtype_t */
  int32_t n_rows;       /* rows of X, V and Y (>= 0) */
  int32_t h_in;         /* H1: columns of X, rows of A_k; multiple of 8, <= SGMV_MAX_HIDDEN */
  int32_t h_out;        /* H2: columns of Y and B_k; multiple of 8, <= SGMV_MAX_HIDDEN */
  int32_t rank;         /* r: one of 8, 16, 32, 64 */
  int32_t num_loras;    /* entries of A_ptrs / B_ptrs (>= 1 when num_segs > 0) */
  int32_t num_segs;     /* S (>= 0); 0 makes every device call a no-op */
  int32_t max_seg_len;  /* upper bound on every segment's length, 0..n_rows */
  int32_t variant;      /* sgmv_variant_t */
  int32_t splits;       /* workgroups sharing one row block of a segment (split-K
                           factor of the vector kernels); 0 picks it automatically */
} sgmv_problem_t;

/* Size of the leading area of every workspace that holds the kernels'
 * arrival counters.  It must be zero-filled before the workspace's first use;
 * every call that completes leaves it zero again.
 *
 * Workspace layout (one projection's slice; sizes from sgmv_workspace_bytes):
 *   [0, SGMV_WS_COUNTER_BYTES)  arrival counters of the two-launch route
 *   then                        that route's split partials and V, or the
 *                               matrix-core route's partial planes and V
 *   then                        the one-launch decode route's tagged partial
 *                               slots: an area no other route writes, so a
 *                               stale word there is always a tag of an
 *                               earlier decode launch, never another route's
 *                               data.
 *   then                        the matrix-core expand's lead area (V as tagged
 *                               words, or one flag per row block), for the same
 *                               reason also written by no other route.
 * Only the counter area must be zero before first use; the rest may hold
 * anything.  A call that does not complete (a kernel killed part way, a
 * device reset) can leave counters non-zero, after which two-launch calls on
 * that workspace give unspecified results: zero the counter area again before
 * reusing a workspace after such a failure.  The decode route and the
 * matrix-core route need no reset: their hand-offs carry a per-launch tag. */
#define SGMV_WS_COUNTER_BYTES ((size_t)1 << 20)

/* Human-readable name of a status code (static string, never NULL). */
const char* sgmv_status_str(sgmv_status_t status);

/* Host-only segment builder (no device access).  Groups the n requests of a
 * batch by LoRA id, as the multi-LoRA paragraph of the Punica README
 * requires (every input row bound to its own LoRA), into the segments of the
 * SGMV paragraph.  Order: ascending LoRA id, ties by request index (a stable
 * sort), only non-empty segments.
 *   req_lora   [n]      in:  LoRA id of request i, each in [0, num_loras)
 *   perm       [n]      out: perm[j] = request index placed at sorted row j
 *   seg_indptr [n+1]    out: capacity n+1; first *num_segs+1 entries written
 *   lora_idx   [n]      out: capacity n;   first *num_segs entries written
 *   num_segs, max_seg_len  out scalars
 * n = 0 gives num_segs = 0, seg_indptr[0] = 0, max_seg_len = 0.
 * Returns SGMV_ERR_INVALID_ARG for null pointers (other than arrays of an
 * n = 0 call), n < 0, num_loras < 1, or an id outside [0, num_loras); outputs
 * are then unspecified.  Runs in O(n + num_loras) time. */
sgmv_status_t sgmv_build_segments(const int32_t* req_lora, int32_t n, int32_t num_loras,
                                  int32_t* perm, int32_t* seg_indptr, int32_t* lora_idx,
                                  int32_t* num_segs, int32_t* max_seg_len);

/* Host-only check of a problem description: sizes, rank, dtype, variant. */
sgmv_status_t sgmv_check_problem(const sgmv_problem_t* problem);

/* Host-only check of a HOST copy of the segment metadata against the
 * preconditions listed above (num_segs, n_rows, max_seg_len and num_loras
 * taken from *problem). */
sgmv_status_t sgmv_check_segments(const sgmv_problem_t* problem, const int32_t* seg_indptr_host,
                                  const int32_t* lora_idx_host);

/* Workspace bytes that sgmv_shrink / sgmv_lora_apply need for *problem
 * (always >= SGMV_WS_COUNTER_BYTES). */
sgmv_status_t sgmv_workspace_bytes(const sgmv_problem_t* problem, size_t* bytes);

/* Kernel route that sgmv_lora_apply takes for a problem on the current HIP
 * device.  The SGMV paragraph of the Punica README describes one kernel for
 * every batch shape; here the route is chosen from the segment lengths: the
 * one-launch kernel while its grid fits on the device at once (decode-shaped
 * batches), the matrix-core kernels when some segment is long (prefill), else
 * the vector kernels. */
typedef enum sgmv_route {
  SGMV_ROUTE_NONE = 0,    /* nothing to do (no rows or segments) */
  SGMV_ROUTE_DECODE = 1,  /* one launch: shrink, on-chip exchange, expand */
  SGMV_ROUTE_MFMA = 2,    /* matrix-core shrink, then matrix-core expand, whose launch also sums the shrink's split partials
                             (in its first, lead workgroups) */
  SGMV_ROUTE_VECTOR = 3   /* split-K vector shrink, then vector expand */
} sgmv_route_t;

typedef struct sgmv_plan_info {
  int32_t route;          /* sgmv_route_t */
  int32_t launches;       /* kernel launches per sgmv_lora_apply call */
  int32_t rows_per_unit;  /* rows of one segment block (decode and vector routes) or of
                             one shrink tile (matrix-core route) */
  int32_t units;          /* segment blocks planned (an upper bound: empty ones exit at once) */
  int32_t splits;         /* workgroups that share one block (decode, vector) or
                             partial planes of the H1 split (matrix-core) */
  int32_t grid;           /* workgroups of the first launch */
} sgmv_plan_info_t;

/* Host-only: the plan sgmv_lora_apply would run for *problem on the current
 * device (the decode route depends on the device's occupancy; without a
 * usable device it is never chosen).  A batched call with a row map or rank /
 * scale tables launches a kernel variant whose occupancy may differ, so its
 * plan may differ too.  When the decode route's units do not all fit on the
 * device at once, it launches the largest co-resident grid (grid < units *
 * splits) once per pass over them (launches > 1).
 * No device memory is touched. */
sgmv_status_t sgmv_query_plan(const sgmv_problem_t* problem, sgmv_plan_info_t* info);

/* Shrink: V[i, :] = X[i, :] @ A_{lora_idx[s]} for every covered row i
 * (Punica README, LoRA paragraph: the x@A factor of x@A@B).  V rows not
 * covered by a segment are left untouched.  ws: device workspace of at least
 * sgmv_workspace_bytes bytes whose counter area is zero (see above). */
sgmv_status_t sgmv_shrink(const sgmv_problem_t* problem, const void* X, const void* const* A_ptrs,
                          float* V, const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                          size_t ws_bytes, void* stream);

/* Expand: Y[i, :] += V[i, :] @ B_{lora_idx[s]} for every covered row i
 * (the trailing @B factor), V in fp32, one rounding of Y on store. */
sgmv_status_t sgmv_expand(const sgmv_problem_t* problem, const float* V, const void* const* B_ptrs,
                          void* Y, const int32_t* seg_indptr, const int32_t* lora_idx,
                          void* stream);

/* Fused apply: Y[i, :] += (X[i, :] @ A_k) @ B_k, the whole LoRA term of the
 * multi-LoRA paragraph, with the fp32 intermediate kept in the workspace or
 * on chip.  Same workspace contract as sgmv_shrink.
 *
 * Device sharing (decode route, SGMV_ROUTE_DECODE of sgmv_query_plan): the
 * workgroups of one unit wait for each other's partial sums, and the grid is
 * sized from the device's occupancy so that all of them are resident at once
 * when the launch has the device to itself.  Precondition: no other
 * decode-route launch runs concurrently on the same device (another stream,
 * another process), and no other work holds the CUs that the launch needs.
 * If that is broken, a waiting workgroup gives up after the wait limit
 * (sgmv_set_wait_limit, default 1 s), leaves its part of Y untouched and sets
 * SGMV_DEVICE_ERR_WAIT_TIMEOUT in the device error word
 * (sgmv_take_device_errors): the kernel always ends, and the error is
 * reported instead of a hang.  On the matrix-core route with more than one
 * split partial per row, the expand launch's first workgroups (lowest ids,
 * dispatched first; they wait for nothing) sum them, and the other workgroups
 * wait for their rows' sums under the same bound and error word.  Calls on
 * one workspace must not overlap. */
sgmv_status_t sgmv_lora_apply(const sgmv_problem_t* problem, const void* X,
                              const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                              const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                              size_t ws_bytes, void* stream);

/* Fused apply with the segment metadata and the LoRA pointer tables on the
 * host: the segments the host builder produced for a batch (Punica README,
 * SGMV paragraph: a batch grouped into segments, each gathering its own
 * LoRA's weights) need not be copied to the device first.  Same result, bit
 * for bit, as sgmv_lora_apply on device copies of the same arrays.  The
 * library gathers each segment's A_k and B_k pointers on the host and passes
 * them with the segment bounds in the kernel's arguments, so the kernel reads
 * no metadata from device memory before its first weight load (one dependent
 * memory trip fewer than sgmv_lora_apply).
 *   A_ptrs_host, B_ptrs_host  [num_loras]     host arrays of device pointers
 *   seg_indptr_host           [num_segs + 1]  host arrays, checked as by
 *   lora_idx_host             [num_segs]      sgmv_check_segments
 * The host arrays are read during the call only.  Only for calls that the
 * one-launch decode route takes (decode-shaped batches) with at most
 * SGMV_HOST_META_MAX_SEGS segments; otherwise SGMV_ERR_UNSUPPORTED and nothing
 * is launched (use sgmv_lora_apply).  A null A_k or B_k of a segment gives
 * SGMV_ERR_INVALID_ARG, one not 16-byte aligned SGMV_ERR_UNSUPPORTED.
 * Workspace (sgmv_workspace_bytes), stream and device-sharing rules as for
 * sgmv_lora_apply. */
#define SGMV_HOST_META_MAX_SEGS 64
sgmv_status_t sgmv_lora_apply_host_meta(const sgmv_problem_t* problem, const void* X,
                                        const void* const* A_ptrs_host, const void* const* B_ptrs_host,
                                        void* Y, const int32_t* seg_indptr_host,
                                        const int32_t* lora_idx_host, void* ws, size_t ws_bytes,
                                        void* stream);

/* Bound on how long a workgroup waits for partial sums made by other
 * workgroups of the same launch (the one-launch decode route, and the
 * matrix-core expand when its lead workgroups sum the split partials), in
 * microseconds (process wide, applies to later calls; default 1000000).  0
 * makes every such wait give up at once: those workgroups then exit without
 * updating Y and set SGMV_DEVICE_ERR_WAIT_TIMEOUT (a test hook for the
 * give-up path).
 * SGMV_ERR_INVALID_ARG for a negative value.  Host only. */
sgmv_status_t sgmv_set_wait_limit(int64_t microseconds);

/* Device error bits of the current HIP device. */
#define SGMV_DEVICE_ERR_WAIT_TIMEOUT 1u  /* a wait for another workgroup's partial sums gave up: Y of that call is unspecified */

/* Synchronises the current device (hipDeviceSynchronize), then reads and
 * clears its device error word: *flags gets the SGMV_DEVICE_ERR_* bits set by
 * every kernel that ended since the last read (0: none).  SGMV_ERR_HIP when
 * the device cannot be queried. */
sgmv_status_t sgmv_take_device_errors(uint32_t* flags);

/* ---- For callers that cannot allocate ----
 *
 * sgmv_lora_apply without a workspace argument, for callers that cannot call
 * hipMalloc or hand over device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its workspace is a
 * static device array of the library, SGMV_NOALLOC_MAX_WORKSPACE bytes on
 * every GPU the library runs on, held until the process ends.  Same
 * arguments, results, preconditions and errors as sgmv_lora_apply, plus
 * SGMV_ERR_WORKSPACE when sgmv_workspace_bytes(problem) exceeds
 * SGMV_NOALLOC_MAX_WORKSPACE.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other host threads) race on it
 * and give unspecified results (decode-route calls may also report
 * SGMV_DEVICE_ERR_WAIT_TIMEOUT); serialise them.  The array keeps the last
 * call's contents; the call itself clears what must start at zero (with a
 * fill kernel on `stream`, on the two-launch route only). */
#define SGMV_NOALLOC_MAX_WORKSPACE ((size_t)16 << 20)
sgmv_status_t sgmv_lora_apply_noalloc(const sgmv_problem_t* problem, const void* X,
                                      const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                                      const int32_t* seg_indptr, const int32_t* lora_idx, void* stream);

/* One projection of a batched apply: its own LoRA tables and output.  All
 * pointers are device pointers, as in sgmv_lora_apply.
 *
 * Heterogeneous ranks (ranks != NULL).  The Punica discussion page
 * ("Punica: Serving multiple LoRA finetuned LLM as one", the question on LoRAs
 * with different ranks) answers that padding every LoRA to one rank costs
 * little because the kernels are not compute bound.  Here the padding is
 * virtual: LoRA k keeps its own rank r_k = ranks[k] (a multiple of 8 in
 * [0, problem->rank]; 0 means the LoRA adds nothing) and its compact storage,
 * A_k [h_in, r_k] and B_k [r_k, h_out] row-major, and the kernels treat ranks
 * r_k .. problem->rank - 1 as zero without reading them.  problem->rank is the
 * largest rank (the compiled tile width).  A LoRA of rank 0 may have null
 * table entries; rank values outside [0, problem->rank] are clamped and rounded
 * down to a multiple of 8 (not an error: the values live on the device).
 *
 * Per-LoRA scale (scales != NULL): the term becomes
 * scales[k] * (x @ A_k) @ B_k, the usual alpha / r factor of LoRA, which is
 * otherwise folded into B_k by the caller.  It multiplies the fp32
 * intermediate x @ A_k before the expand. */
typedef struct sgmv_projection {
  const void* const* A_ptrs;  /* [num_loras] pointers to A_k [h_in, r_k] */
  const void* const* B_ptrs;  /* [num_loras] pointers to B_k [r_k, h_out] */
  void* Y;                    /* [n_rows, h_out], read-modify-write */
  const int32_t* ranks;       /* NULL (every r_k = problem->rank) or [num_loras] int32 */
  const float* scales;        /* NULL (every scale 1) or [num_loras] fp32 */
} sgmv_projection_t;

#define SGMV_MAX_PROJECTIONS 4

/* Batched apply: Y_p[row(i), :] += (X[row(i), :] @ A_{p,k}) @ B_{p,k} for
 * every projection p < num_projections and every covered (sorted) row i.  The multi-LoRA
 * paragraph of the Punica README applies a LoRA per row to a layer's input;
 * the projections of one layer that read the same input (for instance the
 * query, key and value projections of an attention layer, each with its own
 * LoRA pair per model) share X, the shapes and the segments, and run here as
 * one call (one launch per stage instead of one per projection).
 *   projections  HOST array of num_projections (1..SGMV_MAX_PROJECTIONS)
 *                descriptors; the Y buffers must not alias X or each other.
 *   row_idx      NULL (row(i) = i: X and Y are in segment order), or a DEVICE
 *                int32 [n_rows] row map, row(i) = row_idx[i]: the sorted row i
 *                of the segments is row row_idx[i] of X and of every Y.  With the
 *                builder's perm as row_idx the caller keeps X and Y in request
 *                order and skips both permutes (the gather and scatter of rows
 *                happen in the kernels).  Precondition (not checked on the
 *                device): the entries of row_idx[0 .. seg_indptr[S]) are
 *                distinct and in [0, n_rows).
 *   ws           device workspace of at least
 *                (num_projections - 1) * round_up(W, 256) + W bytes, where W is
 *                sgmv_workspace_bytes(problem): projection p uses the slice at
 *                p * round_up(W, 256), whose counter area must be zero (zero
 *                the whole workspace once).
 * Same preconditions, precision and error conventions as sgmv_lora_apply,
 * which is this call with one projection and no row map. */
sgmv_status_t sgmv_lora_apply_batched(const sgmv_problem_t* problem, const void* X,
                                      const sgmv_projection_t* projections, int32_t num_projections,
                                      const int32_t* seg_indptr, const int32_t* lora_idx,
                                      const int32_t* row_idx, void* ws, size_t ws_bytes, void* stream);

/* ---- Base projection with the LoRA term (decode-sized batches) ----
 *
 * Punica README, LoRA paragraph: a row vector x gets the output x@W + x@A@B;
 * multi-LoRA paragraph: X@W is one product for the whole batch and every row
 * adds its own LoRA term.  sgmv_base_lora_apply computes, for every row
 * i < n_rows,
 *     Y[i, :] = X[i, :] @ W + (X[i, :] @ A_k) @ B_k     (k = lora_idx[s], i in segment s)
 *     Y[i, :] = X[i, :] @ W                            (i covered by no segment)
 * with the sum kept in fp32 and rounded once to the input format.  Y is
 * written, not accumulated.
 *   W       device [h_in, h_out] row-major, same format as X, 16-byte aligned.
 *   X, Y    device [n_rows, h_in] and [n_rows, h_out]; Y must not alias X or W.
 *   A_ptrs, B_ptrs, seg_indptr, lora_idx  as for sgmv_lora_apply (may be NULL
 *           when num_segs == 0 or max_seg_len == 0: then Y = X @ W).
 *   ws      device workspace of sgmv_base_workspace_bytes bytes (any contents;
 *           it holds the fp32 partial planes of V and of X @ W).
 * Supported: n_rows <= SGMV_BASE_MAX_ROWS (SGMV_ERR_UNSUPPORTED above; a
 * prefill-sized base projection is a dense GEMM for a GEMM library, followed by
 * sgmv_lora_apply);
 * ranks, formats and alignment as for sgmv_lora_apply.  Two launches (split-K
 * partial products of X @ W on the matrix cores together with the partial
 * planes of V = X @ A_k; an epilogue that sums them, adds V @ B_k and rounds);
 * asynchronous on `stream`.  Same metadata preconditions and error
 * conventions as sgmv_lora_apply. */
/* Largest batch (rows) the base projection entry points take. */
#define SGMV_BASE_MAX_ROWS 128

sgmv_status_t sgmv_base_workspace_bytes(const sgmv_problem_t* problem, size_t* bytes);
sgmv_status_t sgmv_base_lora_apply(const sgmv_problem_t* problem, const void* X, const void* W,
                                   const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                                   const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                                   size_t ws_bytes, void* stream);

/* Base projection from a packed copy of W.  The base weight of a layer does
 * not change while a server runs, so it can be rearranged once into the
 * operand order of the matrix cores; sgmv_base_lora_apply_packed then streams
 * it with fully coalesced loads straight into the MFMA operands (no LDS
 * staging of W; over 32 rows, X is staged once per workgroup).  It computes
 * what sgmv_base_lora_apply computes, to the same bound.  The outputs are
 * bitwise equal whenever both calls split K alike.  That holds unless the call
 * has over 32 rows and the row-major call's K chunk exceeds 512 rows of W.
 * The packed call then takes a shorter chunk and more partial planes.
 *
 * Packed layout (16-bit elements, either format): kst = ceil(h_in / 128) * 4
 * k-steps of 32 rows; ceil(h_out / 16) rounded up to an even count of
 * 16-column blocks.  Block (nb, ks) is 512 elements at offset
 * (nb * kst + ks) * 512; its elements 8 L + e (L = 16 q + m, e = 0..7) hold
 * W[32 ks + 8 q + e][16 nb + m], or 0 past the matrix.
 *
 * sgmv_base_packed_weight_bytes: size of the packed copy for h_in, h_out > 0
 *   (SGMV_ERR_INVALID_ARG otherwise; SGMV_ERR_UNSUPPORTED above SGMV_MAX_HIDDEN).
 * sgmv_base_pack_weight: W device [h_in, h_out] row-major, 2-byte aligned ->
 *   Wp device, 16-byte aligned, wp_bytes >= sgmv_base_packed_weight_bytes
 *   (SGMV_ERR_WORKSPACE below it).  One launch, asynchronous on `stream`; W is
 *   not modified and the caller owns both buffers.
 * sgmv_base_lora_apply_packed: the arguments of sgmv_base_lora_apply with Wp,
 *   the packed copy of W for problem->h_in and problem->h_out, in place of W
 *   (16-byte aligned); same workspace size, limits and errors. */
sgmv_status_t sgmv_base_packed_weight_bytes(int32_t h_in, int32_t h_out, size_t* bytes);
sgmv_status_t sgmv_base_pack_weight(const void* W, int32_t h_in, int32_t h_out, void* Wp, size_t wp_bytes,
                                    void* stream);
sgmv_status_t sgmv_base_lora_apply_packed(const sgmv_problem_t* problem, const void* X, const void* Wp,
                                          const void* const* A_ptrs, const void* const* B_ptrs, void* Y,
                                          const int32_t* seg_indptr, const int32_t* lora_idx, void* ws,
                                          size_t ws_bytes, void* stream);

/* One shard of a row-parallel (H1-split) base layer: the same product written
 * as an unrounded fp32 partial.  The LoRA paragraph's output x@W + x@A@B is
 * linear in x over any split of H1 into slices g: x@W = sum_g x_g@W_g and
 * x@A@B = (sum_g x_g@A_g)@B = sum_g (x_g@A_g)@B.  A device holding slice g of a
 * layer whose input is split along H1 computes
 *     Yp[i, :] = X_g[i, :] @ W_g + (X_g[i, :] @ A_{k,g}) @ B_k      (fp32, written)
 * for every row i (rows no segment covers get X_g[i, :] @ W_g), and the layer's
 * existing all-reduce sums the shards' Yp; rounding the sum once to the input
 * format gives the one-rounding output of sgmv_base_lora_apply.
 *   problem   h_in = the slice's width, h_out = the full H2; other fields as for
 *             sgmv_base_lora_apply (n_rows <= SGMV_BASE_MAX_ROWS).
 *   X, W      device X_g [n_rows, h_in] and W_g [h_in, h_out] (rows of W in the
 *             slice), row-major, or W_g in the packed layout of
 *             sgmv_base_pack_weight when w_packed = 1 (0: row-major).
 *   A_ptrs    [num_loras] device pointers to A_{k,g}, the slice's rows of A_k:
 *             [h_in, rank] row-major (A_k's own storage at row offset g * h_in).
 *   B_ptrs    [num_loras] device pointers to the whole B_k [rank, h_out].
 *   Yp        device fp32 [n_rows, h_out], 16-byte aligned, written.
 *   ws        as for sgmv_base_lora_apply (sgmv_base_workspace_bytes).
 * Errors as for sgmv_base_lora_apply; SGMV_ERR_INVALID_ARG for w_packed other
 * than 0 or 1. */
sgmv_status_t sgmv_base_lora_apply_partial(const sgmv_problem_t* problem, const void* X, const void* W,
                                           int32_t w_packed, const void* const* A_ptrs,
                                           const void* const* B_ptrs, float* Yp, const int32_t* seg_indptr,
                                           const int32_t* lora_idx, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SGMV_H */
