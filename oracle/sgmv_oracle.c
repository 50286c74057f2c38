/*
 * sgmv_oracle.c - plain fp64 reference of the SGMV LoRA term.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the benchmark's CPU
 * baseline call this; the library's compute path never does.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * Follows the Punica README (page "Punica：多 LoRA 模型统一服务框架"):
 *  - LoRA paragraph: A is [H1, r], B is [r, H2], a row vector x gets
 *    x@A@B added to x@W; evaluated here in that association, (x@A)@B.
 *  - multi-LoRA paragraph: every row of the batch uses its own LoRA pair, and
 *    the LoRA term is added on top of the base output X@W (held in Y0).
 *  - SGMV paragraph: rows come grouped in segments that share one LoRA; a
 *    segment s covers rows [seg_indptr[s], seg_indptr[s+1]) and uses LoRA
 *    lora_idx[s].
 * Every fp16/bf16 input is decoded exactly to double; all sums are fp64 in
 * ascending index order; nothing is blocked, fused or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_binary16(uint16_t bits) {
  const int sign = bits >> 15;
  const int expo = (bits >> 10) & 0x1f;
  const int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24);             /* subnormal: frac * 2^(1-15-10) */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(1024 + frac), expo - 25); /* (1.frac) * 2^(expo-15) */
  }
  return sign ? -mag : mag;
}

/* bfloat16 is the upper 16 bits of an IEEE binary32 value. */
static double decode_bfloat16(uint16_t bits) {
  const uint32_t word = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

static double decode(int dtype, uint16_t bits) {
  return dtype == ORACLE_BF16 ? decode_bfloat16(bits) : decode_binary16(bits);
}

void oracle_decode(int dtype, const uint16_t* in, double* out, int64_t count) {
  for (int64_t i = 0; i < count; ++i) out[i] = decode(dtype, in[i]);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Checks the segment metadata and returns, for every row, its segment (or -1
 * when no segment covers it).  Returns NULL on invalid metadata. */
static int32_t* row_segments(int32_t n_rows, const int32_t* seg_indptr, const int32_t* lora_idx,
                             int32_t num_segs, int32_t num_loras) {
  if (n_rows < 0 || num_segs < 0) return NULL;
  int32_t* seg_of_row = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  if (!seg_of_row) return NULL;
  for (int32_t i = 0; i < n_rows; ++i) seg_of_row[i] = -1;
  if (num_segs > 0 && seg_indptr[0] != 0) goto bad;
  for (int32_t s = 0; s < num_segs; ++s) {
    const int32_t lo = seg_indptr[s], hi = seg_indptr[s + 1];
    if (hi < lo || hi > n_rows) goto bad;
    if (lora_idx[s] < 0 || lora_idx[s] >= num_loras) goto bad;
    for (int32_t i = lo; i < hi; ++i) seg_of_row[i] = s;
  }
  return seg_of_row;
bad:
  free(seg_of_row);
  return NULL;
}

/* v[j] = sum_h x[h] * A[h, j], h ascending. */
static void row_shrink(int dtype, int32_t h_in, int32_t rank, const uint16_t* x_row,
                       const uint16_t* a, double* v) {
  for (int32_t j = 0; j < rank; ++j) {
    double acc = 0.0;
    for (int32_t h = 0; h < h_in; ++h)
      acc += decode(dtype, x_row[h]) * decode(dtype, a[(int64_t)h * rank + j]);
    v[j] = acc;
  }
}

/* y[c] = y0[c] + scale * sum_j v[j] * B[j, c], j ascending. */
static void row_expand(int dtype, int32_t rank, int32_t h_out, const double* v,
                       const uint16_t* b, const uint16_t* y0_row, double scale, double* y) {
  for (int32_t c = 0; c < h_out; ++c) {
    double acc = 0.0;
    for (int32_t j = 0; j < rank; ++j) acc += v[j] * decode(dtype, b[(int64_t)j * h_out + c]);
    y[c] = decode(dtype, y0_row[c]) + scale * acc;
  }
}

/*
 * Shrink: V[i, :] = X[i, :] @ A_{lora_idx[s]} for each covered row i.
 * row_mask (nullable) limits the work to rows with a non-zero mask byte.
 * Uncovered or masked-out rows of V are not written.
 * Returns 0, or -1 on invalid metadata.
 */
int oracle_sgmv_shrink(int dtype, int32_t n_rows, int32_t h_in, int32_t rank,
                       const uint16_t* X, const uint16_t* const* A, int32_t num_loras,
                       const int32_t* seg_indptr, const int32_t* lora_idx, int32_t num_segs,
                       const uint8_t* row_mask, double* V, int nthreads) {
  int32_t* seg_of_row = row_segments(n_rows, seg_indptr, lora_idx, num_segs, num_loras);
  if (!seg_of_row) return -1;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    const int32_t s = seg_of_row[i];
    if (s < 0 || (row_mask && !row_mask[i])) continue;
    row_shrink(dtype, h_in, rank, X + (int64_t)i * h_in, A[lora_idx[s]], V + (int64_t)i * rank);
  }
  free(seg_of_row);
  return 0;
}

/*
 * Expand: Y[i, :] = Y0[i, :] + V[i, :] @ B_{lora_idx[s]} for each covered
 * row i, with V given in fp64.  Uncovered rows get Y = Y0 exactly; masked-out
 * rows are not written.  Returns 0, or -1 on invalid metadata.
 */
int oracle_sgmv_expand(int dtype, int32_t n_rows, int32_t h_out, int32_t rank, const double* V,
                       const uint16_t* const* B, int32_t num_loras, const int32_t* seg_indptr,
                       const int32_t* lora_idx, int32_t num_segs, const uint16_t* Y0,
                       const uint8_t* row_mask, double* Y, int nthreads) {
  int32_t* seg_of_row = row_segments(n_rows, seg_indptr, lora_idx, num_segs, num_loras);
  if (!seg_of_row) return -1;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    if (row_mask && !row_mask[i]) continue;
    const int32_t s = seg_of_row[i];
    double* y = Y + (int64_t)i * h_out;
    const uint16_t* y0 = Y0 + (int64_t)i * h_out;
    if (s < 0) {
      for (int32_t c = 0; c < h_out; ++c) y[c] = decode(dtype, y0[c]);
      continue;
    }
    row_expand(dtype, rank, h_out, V + (int64_t)i * rank, B[lora_idx[s]], y0, 1.0, y);
  }
  free(seg_of_row);
  return 0;
}

/*
 * Whole LoRA term: Y[i, :] = Y0[i, :] + s_k * (X[i, :] @ A_k) @ B_k, k the
 * LoRA of row i's segment, the intermediate kept in fp64.
 *   ranks  (nullable) rank r_k of each LoRA: A_k is [h_in, r_k] and B_k is
 *          [r_k, h_out]; NULL means every LoRA has rank `rank`.  A LoRA of
 *          rank 0 adds nothing.  The Punica discussion page ("Punica: Serving
 *          multiple LoRA finetuned LLM as one", the question on LoRAs with
 *          different ranks) treats such LoRAs as padded to one rank: padding
 *          with zero columns of A and zero rows of B leaves the term unchanged,
 *          which is what a rank table expresses.
 *   scales (nullable) s_k of each LoRA; NULL means 1.
 * V (nullable, [n_rows, rank]) receives the unscaled fp64 intermediate of
 * covered rows, zero past r_k.  Uncovered rows get Y = Y0 exactly.
 * Returns 0, or -1 on invalid metadata, a rank outside [0, rank], or
 * allocation failure.
 */
int oracle_sgmv_apply(int dtype, int32_t n_rows, int32_t h_in, int32_t h_out, int32_t rank,
                      const int32_t* ranks, const double* scales, const uint16_t* X,
                      const uint16_t* const* A, const uint16_t* const* B, int32_t num_loras,
                      const int32_t* seg_indptr, const int32_t* lora_idx, int32_t num_segs,
                      const uint16_t* Y0, const uint8_t* row_mask, double* Y, double* V,
                      int nthreads) {
  int32_t* seg_of_row = row_segments(n_rows, seg_indptr, lora_idx, num_segs, num_loras);
  if (!seg_of_row) return -1;
  int bad = rank <= 0 || rank > 4096;
  for (int32_t k = 0; ranks && k < num_loras; ++k) bad |= ranks[k] < 0 || ranks[k] > rank;
  if (bad) {
    free(seg_of_row);
    return -1;
  }
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    if (row_mask && !row_mask[i]) continue;
    const int32_t s = seg_of_row[i];
    double* y = Y + (int64_t)i * h_out;
    const uint16_t* y0 = Y0 + (int64_t)i * h_out;
    if (s < 0) {
      for (int32_t c = 0; c < h_out; ++c) y[c] = decode(dtype, y0[c]);
      continue;
    }
    double v[4096];
    const int32_t k = lora_idx[s];
    const int32_t rk = ranks ? ranks[k] : rank;
    row_shrink(dtype, h_in, rk, X + (int64_t)i * h_in, A[k], v);
    row_expand(dtype, rk, h_out, v, B[k], y0, scales ? scales[k] : 1.0, y);
    if (V)
      for (int32_t j = 0; j < rank; ++j) V[(int64_t)i * rank + j] = j < rk ? v[j] : 0.0;
  }
  free(seg_of_row);
  return 0;
}

/*
 * Base projection plus the LoRA term.  The LoRA paragraph gives a row vector x
 * the output x@W + x@A@B; the multi-LoRA paragraph computes X@W for the whole
 * batch and adds each row's own LoRA term:
 *   Y[i, c] = sum_h X[i, h] * W[h, c]  (h ascending)
 *             + [row i covered] sum_j v[j] * B_k[j, c]  (j ascending),
 *   v[j] = sum_h X[i, h] * A_k[h, j],  k the LoRA of row i's segment.
 * W is [h_in, h_out] row-major.  A row no segment covers gets the base term
 * only.  Every output's base sum runs over h in ascending order (the loop
 * below walks W row by row and keeps h_out running sums).  row_mask
 * (nullable) limits the work to rows with a non-zero mask byte; masked-out
 * rows are not written.  Returns 0, or -1 on invalid metadata.
 */
int oracle_sgmv_base_apply(int dtype, int32_t n_rows, int32_t h_in, int32_t h_out, int32_t rank,
                           const uint16_t* X, const uint16_t* W, const uint16_t* const* A,
                           const uint16_t* const* B, int32_t num_loras, const int32_t* seg_indptr,
                           const int32_t* lora_idx, int32_t num_segs, const uint8_t* row_mask,
                           double* Y, int nthreads) {
  int32_t* seg_of_row = row_segments(n_rows, seg_indptr, lora_idx, num_segs, num_loras);
  if (!seg_of_row) return -1;
  if (rank <= 0 || rank > 4096) {
    free(seg_of_row);
    return -1;
  }
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t i = 0; i < n_rows; ++i) {
    if (row_mask && !row_mask[i]) continue;
    double* y = Y + (int64_t)i * h_out;
    const uint16_t* x_row = X + (int64_t)i * h_in;
    for (int32_t c = 0; c < h_out; ++c) y[c] = 0.0;
    for (int32_t h = 0; h < h_in; ++h) {  /* base: running sums over h */
      const double xh = decode(dtype, x_row[h]);
      const uint16_t* w_row = W + (int64_t)h * h_out;
      for (int32_t c = 0; c < h_out; ++c) y[c] += xh * decode(dtype, w_row[c]);
    }
    const int32_t s = seg_of_row[i];
    if (s < 0) continue;
    double v[4096];
    const int32_t k = lora_idx[s];  /* LoRA of the row's segment */
    row_shrink(dtype, h_in, rank, x_row, A[k], v);
    for (int32_t c = 0; c < h_out; ++c) {
      double acc = 0.0;
      for (int32_t j = 0; j < rank; ++j)  /* LoRA term: v @ B_k */
        acc += v[j] * decode(dtype, B[k][(int64_t)j * h_out + c]);
      y[c] += acc;
    }
  }
  free(seg_of_row);
  return 0;
}
