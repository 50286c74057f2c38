// host_checks.cpp - drives the host-only part of libsgmv (segment builder,
// problem and metadata checks, kernel plans, workspace layout) over seeded
// random, extreme and malformed inputs.  tests/test_host_sanitizers.py builds
// it together with segmented_gather_matvec_amd/csrc/sgmv_host.cpp under the
// address and undefined-behaviour sanitizers; any report, or a failed check,
// fails the test.  Exit status 0 means every check held.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <numeric>
#include <random>
#include <vector>

#include "sgmv.h"
#include "sgmv_host.h"

using namespace sgmv_host;

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      if (failures < 20) std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

// The builder against a plain stable sort (ascending id, ties by request).
static void builder_random(std::mt19937_64& rng) {
  for (int trial = 0; trial < 3000; ++trial) {
    const int n = (int)(rng() % 300);
    int32_t P;
    switch (rng() % 4) {
      case 0: P = 1; break;
      case 1: P = 1 + (int32_t)(rng() % 64); break;
      case 2: P = 1 + (int32_t)(rng() % 5000); break;
      default: P = INT32_MAX - (int32_t)(rng() % 1000); break;  // the sparse-id path
    }
    std::vector<int32_t> ids((size_t)n);
    for (auto& v : ids) v = (int32_t)(rng() % (uint64_t)P);
    if (P > 64 && n > 0 && rng() % 2) ids[0] = P - 1;
    std::vector<int32_t> perm((size_t)n + 1, -7), seg((size_t)n + 1, -7), lidx((size_t)n + 1, -7);
    int32_t S = -1, mx = -1;
    const sgmv_status_t st = sgmv_build_segments(n ? ids.data() : nullptr, n, P, n ? perm.data() : nullptr,
                                                 seg.data(), n ? lidx.data() : nullptr, &S, &mx);
    CHECK(st == SGMV_OK);
    std::vector<int32_t> ref((size_t)n);
    std::iota(ref.begin(), ref.end(), 0);
    std::stable_sort(ref.begin(), ref.end(), [&](int32_t a, int32_t b) { return ids[(size_t)a] < ids[(size_t)b]; });
    for (int j = 0; j < n; ++j) CHECK(perm[(size_t)j] == ref[(size_t)j]);
    int32_t s = 0, longest = 0;
    CHECK(seg[0] == 0);
    for (int j = 0; j < n; ++j) {
      if (j > 0 && ids[(size_t)ref[(size_t)j]] != ids[(size_t)ref[(size_t)j - 1]]) {
        CHECK(seg[(size_t)s + 1] == j);
        longest = std::max(longest, j - seg[(size_t)s]);
        ++s;
      }
      CHECK(lidx[(size_t)s] == ids[(size_t)ref[(size_t)j]]);
    }
    if (n > 0) {
      CHECK(seg[(size_t)s + 1] == n);
      longest = std::max(longest, n - seg[(size_t)s]);
      ++s;
    }
    CHECK(S == s);
    CHECK(mx == longest);
  }
}

static void builder_malformed(std::mt19937_64& rng) {
  int32_t ids[8] = {0, 1, 2, 3, 0, 1, 2, 3};
  int32_t perm[8], seg[9], lidx[8], S, mx;
  CHECK(sgmv_build_segments(ids, -1, 4, perm, seg, lidx, &S, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(ids, 8, 0, perm, seg, lidx, &S, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(ids, 8, INT32_MIN, perm, seg, lidx, &S, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(nullptr, 8, 4, perm, seg, lidx, &S, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(ids, 8, 4, nullptr, seg, lidx, &S, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(ids, 8, 4, perm, nullptr, lidx, &S, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(ids, 8, 4, perm, seg, nullptr, &S, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(ids, 8, 4, perm, seg, lidx, nullptr, &mx) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(ids, 8, 4, perm, seg, lidx, &S, nullptr) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_build_segments(nullptr, 0, 4, nullptr, seg, nullptr, &S, &mx) == SGMV_OK && S == 0 && mx == 0);
  for (int trial = 0; trial < 2000; ++trial) {
    int32_t bad[8];
    for (int i = 0; i < 8; ++i) bad[i] = (int32_t)(rng() % 4);
    const int at = (int)(rng() % 8);
    const int32_t P = 1 + (int32_t)(rng() % 4);
    switch (rng() % 4) {
      case 0: bad[at] = -1 - (int32_t)(rng() % 100); break;
      case 1: bad[at] = INT32_MIN; break;
      case 2: bad[at] = P + (int32_t)(rng() % 100); break;
      default: bad[at] = INT32_MAX; break;
    }
    CHECK(sgmv_build_segments(bad, 8, P, perm, seg, lidx, &S, &mx) == SGMV_ERR_INVALID_ARG);
  }
}

static int32_t pick(std::mt19937_64& rng, const std::vector<int32_t>& common) {
  const uint64_t r = rng() % 10;
  if (r < 6) return common[(size_t)(rng() % common.size())];
  if (r < 8) return (int32_t)(rng() % 20000);
  return (int32_t)(uint32_t)rng();
}

// Every problem description, valid or not, must be checked without a trap;
// the valid ones must plan consistently.
static void problems(std::mt19937_64& rng) {
  const std::vector<int32_t> sizes = {INT32_MIN, -8, -1, 0, 1, 7, 8, 16, 24, 64, 128, 4096, 5120, 11008,
                                      13824, 2147483640, INT32_MAX};
  const std::vector<int32_t> small = {INT32_MIN, -1, 0, 1, 2, 3, 8, 16, 32, 64, 100, 1000, INT32_MAX};
  int valid = 0;
  for (int trial = 0; trial < 40000; ++trial) {
    sgmv_problem_t p;
    p.dtype = pick(rng, {-1, 0, 1, 2});
    p.n_rows = pick(rng, small);
    p.h_in = pick(rng, sizes);
    p.h_out = pick(rng, sizes);
    p.rank = pick(rng, {-16, 0, 7, 8, 16, 24, 32, 64, 128});
    p.num_loras = pick(rng, small);
    p.num_segs = pick(rng, small);
    p.max_seg_len = pick(rng, small);
    p.variant = pick(rng, {-1, 0, 1, 2, 3, 4});
    p.splits = pick(rng, {-1, 0, 1, 2, 3, 7, 16, 64, 512, 4096, INT32_MAX});
    if (rng() % 2) {  // bias towards valid descriptions
      p.dtype = (int32_t)(rng() % 2);
      p.rank = 8 << (rng() % 4);
      p.n_rows = (int32_t)(rng() % 6000);
      p.max_seg_len = p.n_rows ? (int32_t)(rng() % ((uint64_t)p.n_rows + 1)) : 0;
      p.num_segs = (int32_t)(rng() % 400);
      p.num_loras = 1 + (int32_t)(rng() % 100);
      p.variant = (int32_t)(rng() % 4);
      if (rng() % 2) p.splits = 0;
      if (rng() % 2) p.h_in = 8 * (1 + (int32_t)(rng() % 2000));
      if (rng() % 2) p.h_out = 8 * (1 + (int32_t)(rng() % 2000));
    }
    const sgmv_status_t st = sgmv_check_problem(&p);
    size_t bytes = 0, base_bytes = 0;
    CHECK(sgmv_workspace_bytes(&p, &bytes) == st);
    const sgmv_status_t bst = sgmv_base_workspace_bytes(&p, &base_bytes);
    if (st != SGMV_OK) {
      CHECK(bst == st);
      continue;
    }
    ++valid;
    CHECK(bytes >= SGMV_WS_COUNTER_BYTES);
    // the plans cover the problem
    const VecPlan v = plan_vec(p, kTargetWorkgroups);
    CHECK(v.splits >= 1 && v.kc % 8 == 0 && v.cw % 8 == 0);
    CHECK((int64_t)v.kc * v.splits >= p.h_in && (int64_t)v.cw * v.splits >= p.h_out);
    CHECK(2 * v.num_units <= kCounterSlots);
    DecodePlan c[3];
    const int nc = decode_candidates(p, c);
    for (int i = 0; i < nc; ++i) {
      CHECK(c[i].supported && c[i].splits >= 1);
      CHECK((int64_t)c[i].kc * c[i].splits >= p.h_in && (int64_t)c[i].cw * c[i].splits >= p.h_out);
      CHECK(c[i].kc <= sgmv::decode_max_kc(p.rank) && c[i].cw <= sgmv::decode_max_cw());
      CHECK(c[i].grid == c[i].round_units * c[i].splits && c[i].round_units >= c[i].num_units);
    }
    if (sgmv::mfma_supported(p.rank)) {
      const MfmaPlan m = plan_mfma(p);
      CHECK(m.ksplit >= 1 && m.kc % sgmv::kMfmaKChunk == 0);
      CHECK((int64_t)m.ksplit * m.kc >= p.h_in && (int64_t)(m.ksplit - 1) * m.kc < p.h_in);
      CHECK(m.chunks_per_wg >= 1 && (m.expand_rows == 16 || m.expand_rows == 32 || m.expand_rows == 64));
      CHECK(m.expand_rows != 32 || p.rank <= 16);
    }
    // the decode slots, then the matrix-core lead area, sit after every other
    // route's area and do not overlap
    const WsLayout w = apply_ws_layout(p);
    CHECK(w.total == bytes);
    CHECK(w.decode_off % 256 == 0 && w.lead_off % 256 == 0);
    CHECK(w.decode_off >= vec_ws_bytes(v, p.rank) + v_area_bytes(p));
    if (sgmv::mfma_supported(p.rank))
      CHECK(w.decode_off >= SGMV_WS_COUNTER_BYTES + plan_mfma(p).partial_bytes + v_area_bytes(p));
    CHECK(w.lead_off >= w.decode_off + decode_slot_bytes(p));
    CHECK(w.total == w.lead_off + (sgmv::mfma_supported(p.rank) ? plan_mfma(p).vt_bytes : 0));
    if (sgmv::mfma_supported(p.rank) && plan_mfma(p).lead)
      CHECK(plan_mfma(p).vt_bytes >= (size_t)p.n_rows * p.rank * 8 &&
            plan_mfma(p).vt_bytes >= (size_t)plan_mfma(p).lead_blocks * 4);
    // base projection
    if (p.n_rows > sgmv::kBaseMaxRows) {
      CHECK(bst == SGMV_ERR_UNSUPPORTED);
    } else {
      CHECK(bst == SGMV_OK);
      for (int packed = 0; packed < 2; ++packed) {
        const BasePlan b = plan_base(p, packed != 0);
        CHECK(b.ksplit >= 1 && (int64_t)b.ksplit * b.kc >= p.h_in && b.kc % sgmv::kBaseStageRows == 0);
        CHECK(b.base_grid % 8 == 0 && b.base_grid >= b.strips * b.ksplit);
        CHECK(b.v_off >= b.b_off && b.p_off >= b.v_off && b.total >= b.p_off && b.total <= base_bytes);
      }
    }
  }
  CHECK(valid > 5000);
  CHECK(sgmv_check_problem(nullptr) == SGMV_ERR_INVALID_ARG);
  size_t b = 0;
  CHECK(sgmv_workspace_bytes(nullptr, &b) == SGMV_ERR_INVALID_ARG);
}

// Metadata checks against a direct evaluation of the preconditions.
static void segments(std::mt19937_64& rng) {
  const std::vector<int32_t> vals = {INT32_MIN, -5, -1, 0, 1, 2, 3, 4, 5, 8, 9, 100, INT32_MAX - 1, INT32_MAX};
  for (int trial = 0; trial < 40000; ++trial) {
    sgmv_problem_t p{};
    p.num_segs = (int32_t)(rng() % 6);
    p.n_rows = pick(rng, vals);
    p.max_seg_len = pick(rng, vals);
    p.num_loras = pick(rng, vals);
    std::vector<int32_t> seg((size_t)p.num_segs + 1), lidx((size_t)p.num_segs + 1);
    int32_t at = 0;
    for (auto& x : seg) x = (rng() % 3) ? (at += (int32_t)(rng() % 4)) : pick(rng, vals);
    if (rng() % 2) seg[0] = 0;
    for (auto& x : lidx) x = (rng() % 3) ? (int32_t)(rng() % 5) : pick(rng, vals);
    bool ok = p.num_segs >= 0 && seg[0] == 0;
    for (int32_t s = 0; ok && s < p.num_segs; ++s) {
      const int64_t len = (int64_t)seg[(size_t)s + 1] - seg[(size_t)s];
      ok = len >= 0 && len <= p.max_seg_len && lidx[(size_t)s] >= 0 && lidx[(size_t)s] < p.num_loras;
    }
    ok = ok && seg[(size_t)p.num_segs] <= p.n_rows;
    CHECK((sgmv_check_segments(&p, seg.data(), lidx.data()) == SGMV_OK) == ok);
  }
  sgmv_problem_t p{};
  p.num_segs = 1;
  int32_t seg[2] = {0, 1};
  CHECK(sgmv_check_segments(nullptr, seg, seg) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_check_segments(&p, nullptr, seg) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_check_segments(&p, seg, nullptr) == SGMV_ERR_INVALID_ARG);
}

static void packed_sizes(std::mt19937_64& rng) {
  const std::vector<int32_t> vals = {INT32_MIN, -1, 0, 1, 8, 15, 16, 17, 127, 128, 129, 4096, 11008,
                                     2147483640, INT32_MAX};
  for (int trial = 0; trial < 20000; ++trial) {
    const int32_t hi = pick(rng, vals), ho = pick(rng, vals);
    size_t bytes = 0;
    const sgmv_status_t st = sgmv_base_packed_weight_bytes(hi, ho, &bytes);
    if (hi <= 0 || ho <= 0) {
      CHECK(st == SGMV_ERR_INVALID_ARG);
    } else if (st == SGMV_OK) {
      // every element of W has a slot
      CHECK(bytes >= (size_t)hi * (size_t)ho * 2u);
      CHECK(bytes % 1024 == 0);
    } else {
      CHECK(st == SGMV_ERR_UNSUPPORTED);
    }
  }
  size_t b = 0;
  CHECK(sgmv_base_packed_weight_bytes(16, 16, nullptr) == SGMV_ERR_INVALID_ARG);
  CHECK(sgmv_base_packed_weight_bytes(4096, 4096, &b) == SGMV_OK && b == 4096u * 4096u * 2u);
}

int main() {
  std::mt19937_64 rng(20241203);
  builder_random(rng);
  builder_malformed(rng);
  problems(rng);
  segments(rng);
  packed_sizes(rng);
  for (int s = 0; s < 8; ++s) CHECK(sgmv_status_str((sgmv_status_t)s) != nullptr);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
