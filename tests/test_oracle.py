"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

The pages (Punica README, page "Punica：多 LoRA 模型统一服务框架") print no numeric
SGMV example, so the oracle is pinned by: a hand-derived closed-form example,
the merge identity x@(W + A@B) = x@W + x@A@B of the LoRA paragraph, the
Identical-popularity case reducing to one dense product, the per-row
definition of the multi-LoRA paragraph (segments change nothing), linearity,
empty-segment / split / permutation invariances, exact decoding of every
fp16 / bf16 bit pattern, and brute force on the tiny workload.  Every check
here uses numpy / torch CPU routines or hand-written expectations, never the
oracle's own C code, as the reference side.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def np_decode(bits, dtype):
    """Independent decode: numpy's float16 and torch's bfloat16 conversions."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def brute_force(dtype, X, A, B, seg_indptr, lora_idx, Y0):
    """Per-row numpy evaluation of Y0 + (x @ A_k) @ B_k from the page's definition."""
    Xd, Y = np_decode(X, dtype), np_decode(Y0, dtype).copy()
    for s in range(len(lora_idx)):
        k = lora_idx[s]
        Ak, Bk = np_decode(A[k], dtype), np_decode(B[k], dtype)
        for i in range(seg_indptr[s], seg_indptr[s + 1]):
            Y[i] = Y[i] + (Xd[i] @ Ak) @ Bk
    return Y


def rand_case(seed, n=8, h_in=32, h_out=24, rank=4, P=4, dtype="f16"):
    rng = np.random.default_rng(seed)
    X = workloads.to_bits(rng.standard_normal((n, h_in), dtype=np.float32), dtype)
    A = workloads.to_bits(rng.standard_normal((P, h_in, rank), dtype=np.float32) * 0.2, dtype)
    B = workloads.to_bits(rng.standard_normal((P, rank, h_out), dtype=np.float32) * 0.5, dtype)
    Y0 = workloads.to_bits(rng.standard_normal((n, h_out), dtype=np.float32), dtype)
    return rng, X, A, B, Y0


# ---------------------------------------------------------------- decoding

def test_decode_every_f16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got, ref = oracle.decode(bits, "f16"), np_decode(bits, "f16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_every_bf16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got, ref = oracle.decode(bits, "bf16"), np_decode(bits, "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_decode_known_values():
    # binary16 landmarks from the IEEE 754 format definition
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x3555: 0.333251953125}
    for b, v in cases.items():
        assert oracle.decode(np.array([b], np.uint16), "f16")[0] == v
    # bfloat16 landmarks (upper half of binary32)
    for b, v in {0x3F80: 1.0, 0xC040: -3.0, 0x0001: 2.0 ** -133, 0x7F7F: 3.3895313892515355e38}.items():
        assert oracle.decode(np.array([b], np.uint16), "bf16")[0] == v


# ---------------------------------------------------------------- closed form

def test_golden_closed_form_example():
    with open(os.path.join(GOLDEN, "closed_form_two_loras.json")) as f:
        g = json.load(f)
    dt = g["dtype"]
    X = workloads.to_bits(np.array(g["X"], np.float32), dt)
    A = workloads.to_bits(np.array(g["A"], np.float32), dt)
    B = workloads.to_bits(np.array(g["B"], np.float32), dt)
    Y0 = workloads.to_bits(np.array(g["Y0"], np.float32), dt)
    Y, V = oracle.sgmv_apply(dt, X, A, B, g["seg_indptr"], g["lora_idx"], Y0, want_v=True)
    assert np.array_equal(Y, np.array(g["Y_expected"], np.float64))
    for i, v in enumerate(g["V_expected"]):
        if v is None:
            assert np.isnan(V[i]).all()
        else:
            assert np.array_equal(V[i], np.array(v, np.float64))
    Vs = oracle.sgmv_shrink(dt, X, A, g["seg_indptr"], g["lora_idx"])
    assert np.array_equal(Vs[:3], V[:3])


def test_merge_identity_of_lora_paragraph():
    """x@(W + A_k@B_k) == x@W + oracle term, row by row (tiny dense brute force)."""
    rng, X, A, B, _ = rand_case(11, n=8, h_in=32, h_out=32, rank=4, P=4)
    ids = rng.integers(0, 4, size=8)
    perm, seg, lidx, _ = oracle.build_segments(ids, 4)
    Xs = X[perm]
    zero = np.zeros((8, 32), np.uint16)
    term = oracle.sgmv_apply("f16", Xs, A, B, seg, lidx, zero)
    W = rng.standard_normal((32, 32))
    Xd = np_decode(Xs, "f16")
    for j, i in enumerate(perm):
        k = ids[i]
        merged = Xd[j] @ (W + np_decode(A[k], "f16") @ np_decode(B[k], "f16"))
        unmerged = Xd[j] @ W + term[j]
        np.testing.assert_allclose(unmerged, merged, rtol=1e-12, atol=1e-12 * np.abs(merged).max())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_identical_popularity_is_one_dense_product(dtype):
    """All rows on one LoRA: the term equals (X@A)@B and X@(A@B) as dense matmuls."""
    _, X, A, B, Y0 = rand_case(12, n=16, h_in=64, h_out=40, rank=8, P=1, dtype=dtype)
    Y = oracle.sgmv_apply(dtype, X, A, B, [0, 16], [0], Y0)
    Xd, Ad, Bd, Y0d = (np_decode(t, dtype) for t in (X, A[0], B[0], Y0))
    scale = np.abs(Y).max()
    np.testing.assert_allclose(Y, Y0d + (Xd @ Ad) @ Bd, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(Y, Y0d + Xd @ (Ad @ Bd), rtol=0, atol=1e-12 * scale)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_workload_brute_force(dtype):
    w = workloads.tiny()
    X, A, B, Y0 = w.X, w.A, w.B, w.Y0
    if dtype == "bf16":  # same draws, bf16 rounding
        X, A, B = (workloads.to_bits(np_decode(t, "f16").astype(np.float32), "bf16") for t in (X, A, B))
    Y = oracle.sgmv_apply(dtype, X, A, B, w.seg_indptr, w.lora_idx, Y0)
    ref = brute_force(dtype, X, A, B, w.seg_indptr, w.lora_idx, Y0)
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------- invariances

def test_segments_equal_per_row_definition():
    """Builder-sorted segments, un-permuted, give exactly the per-row result
    (each row alone in its own one-row segment, in request order)."""
    rng, X, A, B, Y0 = rand_case(13, n=20, P=5)
    ids = rng.integers(0, 5, size=20)
    perm, seg, lidx, _ = oracle.build_segments(ids, 5)
    Ys = oracle.sgmv_apply("f16", X[perm], A, B, seg, lidx, Y0[perm])
    per_row = oracle.sgmv_apply("f16", X, A, B, np.arange(21), ids, Y0)
    unperm = np.empty_like(Ys)
    unperm[perm] = Ys
    assert np.array_equal(unperm, per_row)


def test_linearity_in_segment_rows_and_weights():
    rng, X, A, B, Y0 = rand_case(14, n=10, P=3)
    seg, lidx = [0, 4, 7, 10], [2, 0, 1]
    zero = np.zeros_like(Y0)
    base = oracle.sgmv_apply("f16", X, A, B, seg, lidx, zero)
    # doubling the rows of segment 1 doubles exactly its term, others bit-identical
    X2 = X.copy()
    X2[4:7] = workloads.to_bits(np_decode(X[4:7], "f16").astype(np.float32) * 2, "f16")
    dbl = oracle.sgmv_apply("f16", X2, A, B, seg, lidx, zero)
    assert np.array_equal(dbl[4:7], 2 * base[4:7])
    assert np.array_equal(dbl[:4], base[:4]) and np.array_equal(dbl[7:], base[7:])
    # doubling B_0 doubles exactly the rows that use LoRA 0 (segment 1)
    B2 = B.copy()
    B2[0] = workloads.to_bits(np_decode(B[0], "f16").astype(np.float32) * 2, "f16")
    dblb = oracle.sgmv_apply("f16", X, A, B2, seg, lidx, zero)
    assert np.array_equal(dblb[4:7], 2 * base[4:7]) and np.array_equal(dblb[:4], base[:4])
    # additivity in X with small-integer rows (sums exact in fp16)
    X1 = rng.integers(-8, 9, size=X.shape).astype(np.float32)
    X3 = rng.integers(-8, 9, size=X.shape).astype(np.float32)
    t1 = oracle.sgmv_apply("f16", workloads.to_bits(X1, "f16"), A, B, seg, lidx, zero)
    t3 = oracle.sgmv_apply("f16", workloads.to_bits(X3, "f16"), A, B, seg, lidx, zero)
    t13 = oracle.sgmv_apply("f16", workloads.to_bits(X1 + X3, "f16"), A, B, seg, lidx, zero)
    np.testing.assert_allclose(t13, t1 + t3, rtol=0, atol=1e-12 * np.abs(t13).max())


def test_empty_segments_change_nothing():
    _, X, A, B, Y0 = rand_case(15, n=9, P=4)
    seg, lidx = [0, 3, 5, 9], [1, 3, 0]
    ref = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0)
    seg_e, lidx_e = [0, 0, 3, 3, 3, 5, 9, 9], [2, 1, 0, 3, 3, 0, 1]
    assert np.array_equal(oracle.sgmv_apply("f16", X, A, B, seg_e, lidx_e, Y0), ref)


def test_split_segment_changes_nothing():
    _, X, A, B, Y0 = rand_case(16, n=9, P=4)
    ref = oracle.sgmv_apply("f16", X, A, B, [0, 3, 9], [1, 2], Y0)
    split = oracle.sgmv_apply("f16", X, A, B, [0, 2, 3, 7, 9], [1, 1, 2, 2], Y0)
    assert np.array_equal(split, ref)


def test_segment_permutation_permutes_rows():
    _, X, A, B, Y0 = rand_case(17, n=9, P=4)
    seg, lidx = [0, 3, 5, 9], [1, 3, 0]
    ref = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0)
    order = [2, 0, 1]
    rows = np.concatenate([np.arange(seg[s], seg[s + 1]) for s in order])
    seg_p = np.concatenate([[0], np.cumsum([seg[s + 1] - seg[s] for s in order])])
    got = oracle.sgmv_apply("f16", X[rows], A, B, seg_p, [lidx[s] for s in order], Y0[rows])
    assert np.array_equal(got, ref[rows])


def test_uncovered_rows_keep_base_output():
    _, X, A, B, Y0 = rand_case(18, n=8, P=2)
    Y = oracle.sgmv_apply("f16", X, A, B, [0, 2, 5], [1, 0], Y0)
    assert np.array_equal(Y[5:], np_decode(Y0[5:], "f16"))
    Y_none = oracle.sgmv_apply("f16", X, A, B, [0], [], Y0)
    assert np.array_equal(Y_none, np_decode(Y0, "f16"))


def test_shrink_then_expand_equals_apply():
    _, X, A, B, Y0 = rand_case(19, n=8, P=3)
    seg, lidx = [0, 2, 3, 8], [2, 2, 0]
    V = oracle.sgmv_shrink("f16", X, A, seg, lidx)
    Y = oracle.sgmv_expand("f16", V, B, seg, lidx, Y0)
    assert np.array_equal(Y, oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0))


def test_row_mask_computes_only_listed_rows():
    _, X, A, B, Y0 = rand_case(20, n=8, P=3)
    seg, lidx = [0, 4, 8], [1, 2]
    full = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0)
    mask = np.zeros(8, np.uint8)
    mask[[1, 6]] = 1
    part = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0, row_mask=mask)
    assert np.array_equal(part[[1, 6]], full[[1, 6]])
    assert np.isnan(part[[0, 2, 3, 4, 5, 7]]).all()


@pytest.mark.parametrize("seg,lidx", [([1, 2], [0]), ([0, 3, 2], [0, 0]), ([0, 9], [0]),
                                      ([0, 2], [5]), ([0, 2], [-1])])
def test_invalid_metadata_is_rejected(seg, lidx):
    _, X, A, B, Y0 = rand_case(21, n=8, P=2)
    with pytest.raises(ValueError):
        oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0)


def test_integer_exact_inputs_give_integer_results():
    rng = np.random.default_rng(22)
    X, A, B, Y0 = workloads.integer_exact(rng, 6, 128, 64, 16, 3, "f16", nnz_per_col=8, y0_bound=64)
    Y = oracle.sgmv_apply("f16", X, A, B, [0, 2, 6], [2, 0], Y0)
    assert np.array_equal(Y, np.round(Y)) and np.abs(Y).max() <= 2048
    # the values are exact fp16 integers: the same bits as a direct cast
    assert np.array_equal(workloads.to_bits(Y.astype(np.float32), "f16").view(np.float16).astype(np.float64), Y)


# ---------------------------------------------------------------- ranks and scales
# The Punica discussion page ("Punica: Serving multiple LoRA finetuned LLM as
# one", the question on LoRAs with different ranks) handles mixed ranks by
# padding every LoRA to one rank.  Padding A_k with zero columns and B_k with
# zero rows leaves x @ A_k @ B_k unchanged, so a LoRA of rank r_k must give what
# the uniform-rank path (pinned above) gives on the zero-padded pair.

def het_case(seed, dtype="f16", ranks=(8, 0, 16, 24), R=32, n=10, h_in=48, h_out=40):
    rng = np.random.default_rng(seed)
    X = workloads.to_bits(rng.standard_normal((n, h_in), dtype=np.float32), dtype)
    Y0 = workloads.to_bits(rng.standard_normal((n, h_out), dtype=np.float32), dtype)
    A = [workloads.to_bits(rng.standard_normal((h_in, r), dtype=np.float32) * 0.2, dtype) for r in ranks]
    B = [workloads.to_bits(rng.standard_normal((r, h_out), dtype=np.float32) * 0.5, dtype) for r in ranks]
    Ap = [np.zeros((h_in, R), np.uint16) for _ in ranks]
    Bp = [np.zeros((R, h_out), np.uint16) for _ in ranks]
    for k, r in enumerate(ranks):
        Ap[k][:, :r] = A[k]
        Bp[k][:r, :] = B[k]
    seg, lidx = [0, 3, 5, 9, 10], [2, 1, 0, 3]
    return X, A, B, Ap, Bp, Y0, seg, lidx


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rank_table_equals_zero_padding(dtype):
    X, A, B, Ap, Bp, Y0, seg, lidx = het_case(30, dtype)
    het, V = oracle.sgmv_apply(dtype, X, A, B, seg, lidx, Y0, rank=32, want_v=True)
    pad, Vp = oracle.sgmv_apply(dtype, X, Ap, Bp, seg, lidx, Y0, want_v=True)
    assert np.array_equal(het, pad)
    assert np.array_equal(V, Vp)  # V is zero past each LoRA's rank
    # and both agree with the per-row definition evaluated by numpy
    assert np.allclose(het, brute_force(dtype, X, Ap, Bp, seg, lidx, Y0), rtol=1e-12, atol=1e-12)


def test_rank_zero_lora_adds_nothing():
    X, A, B, Ap, Bp, Y0, seg, lidx = het_case(31)
    Y = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0, rank=32)
    rows = range(seg[1], seg[2])  # segment 1 uses LoRA 1, of rank 0
    assert np.array_equal(Y[list(rows)], np_decode(Y0, "f16")[list(rows)])


def test_scale_multiplies_the_term_only():
    # Integer-exact inputs and power-of-two scales: every value is exact, so
    # Y(s) - Y0 equals s * (Y(1) - Y0) bit for bit, and the base output is not
    # scaled.
    rng = np.random.default_rng(32)
    X, A, B, Y0 = workloads.integer_exact(rng, 6, 128, 64, 16, 3, "f16", nnz_per_col=8, y0_bound=64)
    seg, lidx = [0, 2, 3, 6], [2, 0, 1]
    scales = np.array([0.5, 4.0, -0.25])
    one = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0)
    got = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0, scales=scales)
    y0 = np_decode(Y0, "f16")
    for s in range(3):
        rows = slice(seg[s], seg[s + 1])
        assert np.array_equal(got[rows] - y0[rows], scales[lidx[s]] * (one[rows] - y0[rows]))
    assert not np.array_equal(one, y0)  # the term is not zero


# ---------------------------------------------------------------- base projection + LoRA term

def base_case(seed, n=8, h_in=32, h_out=24, rank=4, P=3, dtype="f16"):
    rng, X, A, B, _ = rand_case(seed, n, h_in, h_out, rank, P, dtype)
    W = workloads.to_bits(rng.standard_normal((h_in, h_out), dtype=np.float32) * 0.2, dtype)
    return X, W, A, B


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_base_apply_with_zero_weight_is_the_lora_term(dtype):
    """W = 0: the base term vanishes and Y is sgmv_apply's result on Y0 = 0, bit for bit."""
    X, W, A, B = base_case(40, dtype=dtype)
    seg, lidx = [0, 3, 4, 8], [2, 0, 2]
    got = oracle.sgmv_base_apply(dtype, X, np.zeros_like(W), A, B, seg, lidx)
    ref = oracle.sgmv_apply(dtype, X, A, B, seg, lidx, np.zeros((8, 24), np.uint16))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_base_apply_without_segments_is_a_matmul(dtype):
    """No segment: Y = X @ W, against numpy's fp64 product of the decoded operands."""
    X, W, A, B = base_case(41, h_in=40, h_out=24, dtype=dtype)
    got = oracle.sgmv_base_apply(dtype, X, W, A, B, [0], [])
    np.testing.assert_allclose(got, np_decode(X, dtype) @ np_decode(W, dtype), rtol=1e-12, atol=1e-12)


def test_base_apply_identity_weight_adds_the_input():
    """W = I (h_in = h_out): Y = X + the LoRA term, i.e. sgmv_apply with Y0 = X, bit for bit."""
    X, W, A, B = base_case(42, h_in=24, h_out=24)
    eye = workloads.to_bits(np.eye(24, dtype=np.float32), "f16")
    seg, lidx = [0, 5, 8], [1, 0]
    assert np.array_equal(oracle.sgmv_base_apply("f16", X, eye, A, B, seg, lidx),
                          oracle.sgmv_apply("f16", X, A, B, seg, lidx, X))


def test_base_apply_uncovered_rows_get_the_base_term_only():
    X, W, A, B = base_case(43)
    got = oracle.sgmv_base_apply("f16", X, W, A, B, [0, 2, 5], [1, 0])
    base = oracle.sgmv_base_apply("f16", X, W, A, B, [0], [])
    assert np.array_equal(got[5:], base[5:])
    assert not np.allclose(got[:5], base[:5])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_base_apply_brute_force(dtype):
    """Per-row numpy evaluation of x @ W + (x @ A_k) @ B_k (h_in != h_out, LoRAs reused)."""
    X, W, A, B = base_case(44, h_in=40, h_out=24, dtype=dtype)
    seg, lidx = [0, 1, 4, 6], [2, 2, 0]
    got = oracle.sgmv_base_apply(dtype, X, W, A, B, seg, lidx)
    Xd = np_decode(X, dtype)
    ref = Xd @ np_decode(W, dtype)
    for s in range(len(lidx)):
        Ak, Bk = np_decode(A[lidx[s]], dtype), np_decode(B[lidx[s]], dtype)
        for i in range(seg[s], seg[s + 1]):
            ref[i] += (Xd[i] @ Ak) @ Bk
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_base_apply_row_mask_computes_only_listed_rows():
    X, W, A, B = base_case(45)
    seg, lidx = [0, 4, 8], [1, 2]
    full = oracle.sgmv_base_apply("f16", X, W, A, B, seg, lidx)
    mask = np.zeros(8, np.uint8)
    mask[[2, 7]] = 1
    part = oracle.sgmv_base_apply("f16", X, W, A, B, seg, lidx, row_mask=mask)
    assert np.array_equal(part[[2, 7]], full[[2, 7]])
    assert np.isnan(part[[0, 1, 3, 4, 5, 6]]).all()


# ---------------------------------------------------------------- builder

def test_builder_golden_examples():
    with open(os.path.join(GOLDEN, "builder_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        perm, seg, lidx, mx = oracle.build_segments(c["req_lora"], c["num_loras"])
        assert perm == c["perm"] and seg == c["seg_indptr"] and lidx == c["lora_idx"]
        assert mx == c["max_seg_len"]


@pytest.mark.parametrize("seed", range(5))
def test_builder_matches_numpy_stable_sort(seed):
    rng = np.random.default_rng(100 + seed)
    n, P = int(rng.integers(1, 300)), int(rng.integers(1, 70))
    ids = rng.integers(0, P, size=n)
    perm, seg, lidx, mx = oracle.build_segments(ids, P)
    assert np.array_equal(perm, np.argsort(ids, kind="stable"))
    counts = np.bincount(ids, minlength=P)
    present = np.nonzero(counts)[0]
    assert np.array_equal(lidx, present)
    assert np.array_equal(np.diff(seg), counts[present]) and seg[-1] == n
    assert mx == counts.max()


def test_builder_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.build_segments([0, 3], 3)
    with pytest.raises(ValueError):
        oracle.build_segments([-1], 3)
