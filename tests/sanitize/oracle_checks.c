/*
 * oracle_checks.c - drives the C oracle (oracle/sgmv_oracle.c) over seeded
 * random, extreme and malformed inputs.  tests/test_host_sanitizers.py builds
 * it together with the oracle under the address and undefined-behaviour
 * sanitizers; any report, or a failed check, fails the test.  The checks are
 * the oracle's own contract: malformed segment metadata is rejected, valid
 * metadata is accepted, and the whole-term entry point agrees bit for bit
 * with its shrink followed by its expand.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_decode(int dtype, const uint16_t* in, double* out, int64_t count);
int oracle_sgmv_shrink(int dtype, int32_t n_rows, int32_t h_in, int32_t rank, const uint16_t* X,
                       const uint16_t* const* A, int32_t num_loras, const int32_t* seg_indptr,
                       const int32_t* lora_idx, int32_t num_segs, const uint8_t* row_mask, double* V,
                       int nthreads);
int oracle_sgmv_expand(int dtype, int32_t n_rows, int32_t h_out, int32_t rank, const double* V,
                       const uint16_t* const* B, int32_t num_loras, const int32_t* seg_indptr,
                       const int32_t* lora_idx, int32_t num_segs, const uint16_t* Y0,
                       const uint8_t* row_mask, double* Y, int nthreads);
int oracle_sgmv_apply(int dtype, int32_t n_rows, int32_t h_in, int32_t h_out, int32_t rank,
                      const int32_t* ranks, const double* scales, const uint16_t* X,
                      const uint16_t* const* A, const uint16_t* const* B, int32_t num_loras,
                      const int32_t* seg_indptr, const int32_t* lora_idx, int32_t num_segs,
                      const uint16_t* Y0, const uint8_t* row_mask, double* Y, double* V, int nthreads);
int oracle_sgmv_base_apply(int dtype, int32_t n_rows, int32_t h_in, int32_t h_out, int32_t rank,
                           const uint16_t* X, const uint16_t* W, const uint16_t* const* A,
                           const uint16_t* const* B, int32_t num_loras, const int32_t* seg_indptr,
                           const int32_t* lora_idx, int32_t num_segs, const uint8_t* row_mask,
                           double* Y, int nthreads);

static int failures = 0;
#define CHECK(c)                                                                      \
  do {                                                                                \
    if (!(c)) {                                                                       \
      if (failures < 20) fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                                     \
    }                                                                                 \
  } while (0)

static uint64_t rs = 88172645463325252ull;
static uint64_t next(void) { /* xorshift64 */
  rs ^= rs << 13;
  rs ^= rs >> 7;
  rs ^= rs << 17;
  return rs;
}
static uint16_t small_value(int dtype) {
  /* finite values of modest size: sign, exponent near the bias, any fraction */
  const uint16_t sign = (uint16_t)((next() & 1) << 15);
  if (dtype == 0) return (uint16_t)(sign | ((12 + next() % 6) << 10) | (next() & 0x3ff));
  return (uint16_t)(sign | ((124 + next() % 6) << 7) | (next() & 0x7f));
}

static int metadata_ok(int32_t n, const int32_t* seg, const int32_t* lidx, int32_t S, int32_t P) {
  if (S < 0) return 0;
  if (S > 0 && seg[0] != 0) return 0;
  for (int32_t s = 0; s < S; ++s) {
    if (seg[s + 1] < seg[s] || seg[s + 1] > n) return 0;
    if (lidx[s] < 0 || lidx[s] >= P) return 0;
  }
  return 1;
}

static void decode_all(void) {
  uint16_t* in = malloc(65536 * sizeof(uint16_t));
  double* out = malloc(65536 * sizeof(double));
  for (int i = 0; i < 65536; ++i) in[i] = (uint16_t)i;
  for (int d = 0; d < 2; ++d) {
    oracle_decode(d, in, out, 65536);
    CHECK(out[0] == 0.0 && out[0x8000] == 0.0 && signbit(out[0x8000]));
    CHECK(d == 0 ? out[0x3c00] == 1.0 : out[0x3f80] == 1.0);
  }
  free(in);
  free(out);
}

static void random_calls(void) {
  for (int trial = 0; trial < 600; ++trial) {
    const int dtype = (int)(next() % 2);
    const int32_t n = (int32_t)(next() % 12), h_in = 8 * (1 + (int32_t)(next() % 6)),
                  h_out = 8 * (1 + (int32_t)(next() % 6)), rank = 8 * (1 + (int32_t)(next() % 4)),
                  P = 1 + (int32_t)(next() % 4);
    const int32_t S = (int32_t)(next() % 5);
    int32_t seg[6], lidx[6];
    int32_t at = 0;
    seg[0] = 0;
    for (int32_t s = 0; s < S; ++s) {
      at += (int32_t)(next() % 4);
      seg[s + 1] = at;
      lidx[s] = (int32_t)(next() % (uint64_t)P);
    }
    /* one field in three broken on purpose */
    if (next() % 3 == 0 && S > 0) {
      const int32_t s = (int32_t)(next() % (uint64_t)S);
      switch (next() % 5) {
        case 0: seg[0] = 1 + (int32_t)(next() % 3); break;
        case 1: seg[s + 1] = seg[s] - 1; break;
        case 2: lidx[s] = -1; break;
        case 3: lidx[s] = P; break;
        default: seg[S] = n + 1 + (int32_t)(next() % 3); break;
      }
    }
    uint16_t* X = malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1) * (size_t)h_in);
    uint16_t* Y0 = malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1) * (size_t)h_out);
    uint16_t* W = malloc(sizeof(uint16_t) * (size_t)h_in * (size_t)h_out);
    const uint16_t* A[4];
    const uint16_t* B[4];
    int32_t ranks[4];
    double scales[4];
    for (int32_t k = 0; k < P; ++k) {
      uint16_t* a = malloc(sizeof(uint16_t) * (size_t)h_in * (size_t)rank);
      uint16_t* b = malloc(sizeof(uint16_t) * (size_t)rank * (size_t)h_out);
      for (int64_t i = 0; i < (int64_t)h_in * rank; ++i) a[i] = small_value(dtype);
      for (int64_t i = 0; i < (int64_t)rank * h_out; ++i) b[i] = small_value(dtype);
      A[k] = a;
      B[k] = b;
      ranks[k] = rank;
      scales[k] = 1.0;
    }
    for (int64_t i = 0; i < (int64_t)n * h_in; ++i) X[i] = small_value(dtype);
    for (int64_t i = 0; i < (int64_t)n * h_out; ++i) Y0[i] = small_value(dtype);
    for (int64_t i = 0; i < (int64_t)h_in * h_out; ++i) W[i] = small_value(dtype);
    const size_t ny = (size_t)(n > 0 ? n : 1) * (size_t)h_out, nv = (size_t)(n > 0 ? n : 1) * (size_t)rank;
    double *Y1 = malloc(sizeof(double) * ny), *Y2 = malloc(sizeof(double) * ny), *Y3 = malloc(sizeof(double) * ny);
    double *V1 = malloc(sizeof(double) * nv), *V2 = malloc(sizeof(double) * nv);
    for (size_t i = 0; i < nv; ++i) V1[i] = V2[i] = 0.0;
    const int ok = metadata_ok(n, seg, lidx, S, P);
    const int threads = 1 + (int)(next() % 3);
    const int rc1 = oracle_sgmv_apply(dtype, n, h_in, h_out, rank, (next() % 2) ? ranks : NULL,
                                      (next() % 2) ? scales : NULL, X, A, B, P, seg, lidx, S, Y0, NULL, Y1, V1,
                                      threads);
    const int rc2 = oracle_sgmv_shrink(dtype, n, h_in, rank, X, A, P, seg, lidx, S, NULL, V2, threads);
    const int rc3 = oracle_sgmv_expand(dtype, n, h_out, rank, V2, B, P, seg, lidx, S, Y0, NULL, Y2, threads);
    const int rc4 = oracle_sgmv_base_apply(dtype, n, h_in, h_out, rank, X, W, A, B, P, seg, lidx, S, NULL, Y3,
                                           threads);
    CHECK((rc1 == 0) == ok && (rc2 == 0) == ok && (rc3 == 0) == ok && (rc4 == 0) == ok);
    if (ok) {
      CHECK(memcmp(Y1, Y2, sizeof(double) * (size_t)n * (size_t)h_out) == 0);
      for (int32_t s = 0; s < S; ++s)
        for (int32_t i = seg[s]; i < seg[s + 1]; ++i)
          CHECK(memcmp(V1 + (int64_t)i * rank, V2 + (int64_t)i * rank, sizeof(double) * (size_t)rank) == 0);
      for (size_t i = 0; i < (size_t)n * (size_t)h_out; ++i) CHECK(isfinite(Y3[i]));
    }
    for (int32_t k = 0; k < P; ++k) {
      free((void*)A[k]);
      free((void*)B[k]);
    }
    free(X); free(Y0); free(W); free(Y1); free(Y2); free(Y3); free(V1); free(V2);
  }
}

static void bad_ranks(void) {
  uint16_t x[8] = {0}, a[64] = {0}, b[64] = {0}, y0[8] = {0};
  const uint16_t* A[1] = {a};
  const uint16_t* B[1] = {b};
  int32_t seg[2] = {0, 1}, lidx[1] = {0};
  double y[8];
  int32_t r1[1] = {9}, r2[1] = {-1};
  CHECK(oracle_sgmv_apply(0, 1, 8, 8, 8, r1, NULL, x, A, B, 1, seg, lidx, 1, y0, NULL, y, NULL, 1) == -1);
  CHECK(oracle_sgmv_apply(0, 1, 8, 8, 8, r2, NULL, x, A, B, 1, seg, lidx, 1, y0, NULL, y, NULL, 1) == -1);
  CHECK(oracle_sgmv_apply(0, 1, 8, 8, 0, NULL, NULL, x, A, B, 1, seg, lidx, 1, y0, NULL, y, NULL, 1) == -1);
  CHECK(oracle_sgmv_apply(0, 1, 8, 8, 8, NULL, NULL, x, A, B, 1, seg, lidx, -1, y0, NULL, y, NULL, 1) == -1);
  CHECK(oracle_sgmv_base_apply(0, 1, 8, 8, 5000, x, x, A, B, 1, seg, lidx, 1, NULL, y, 1) == -1);
}

int main(void) {
  decode_all();
  random_calls();
  bad_ranks();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle checks ok\n");
  return 0;
}
