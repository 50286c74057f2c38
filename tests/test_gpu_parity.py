"""GPU parity of libsgmv against the fp64 oracle, through the C ABI.

Bar: every element within |gpu - ref| <= 1e-3 + 1e-2*|ref| of the unrounded
fp64 oracle; integer-exact inputs (every partial sum an exact fp32 integer,
every output exact in fp16/bf16) must match bit for bit in every variant;
segment metadata from the library's builder must equal the oracle's builder.
Workloads follow the Punica README's popularity cases (page "Punica：多 LoRA
模型统一服务框架", throughput paragraph) and the shapes listed per test.
"""
import numpy as np
import pytest

import oracle
import segmented_gather_matvec_amd as sg
import workloads
from tests.gpu_cases import DeviceCall, assert_close, assert_close_f32, to_bits, to_device

pytestmark = pytest.mark.gpu

APPLY_VARIANTS = [sg.SGMV_VARIANT_AUTO, sg.SGMV_VARIANT_VECTOR, sg.SGMV_VARIANT_FUSED,
                  sg.SGMV_VARIANT_MFMA]


def expect_unsupported(call):
    """The matrix-core kernels take ranks 16, 32 and 64 only."""
    with pytest.raises(sg.SgmvError) as e:
        call.apply()
    assert e.value.status == sg.SGMV_ERR_UNSUPPORTED


def mfma_rank_ok(variant, rank):
    return variant != sg.SGMV_VARIANT_MFMA or rank in (16, 32, 64)


def run_workload(w, variant=sg.SGMV_VARIANT_AUTO, splits=0):
    """Run a Workload (builder applied when it carries per-request ids)."""
    X, Y0 = w.X, w.Y0
    if w.req_lora is not None:
        perm, seg, lidx, _ = sg.sgmv_build_segments(w.req_lora, w.num_loras)
        operm, oseg, olidx, _ = oracle.build_segments(w.req_lora, w.num_loras)
        assert perm.tolist() == operm and seg.tolist() == oseg and lidx.tolist() == olidx
        X, Y0 = X[perm], Y0[perm]
    else:
        seg, lidx = w.seg_indptr, w.lora_idx
    call = DeviceCall(w.dtype, X, w.A, w.B, Y0, seg, lidx, variant=variant, splits=splits)
    return call


# ------------------------------------------------------------ workloads of the pages' study

@pytest.mark.parametrize("variant", APPLY_VARIANTS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny(variant, dtype):
    w = workloads.tiny()
    if dtype == "bf16":
        w.dtype = "bf16"
        w.X, w.A, w.B = (workloads.to_bits(oracle.decode(t, "f16").astype(np.float32), "bf16")
                         for t in (w.X, w.A, w.B))
    call = run_workload(w, variant)
    if not mfma_rank_ok(variant, 8):
        return expect_unsupported(call)
    assert_close(to_bits(call.apply()), call.oracle_apply(), dtype)
    assert call.counters_clear()


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
def test_decode_distinct_h4096_r16_b32(variant):
    call = run_workload(workloads.decode_distinct(), variant)
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")
    assert call.counters_clear()


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 64, 512])
@pytest.mark.parametrize("variant", [sg.SGMV_VARIANT_VECTOR, sg.SGMV_VARIANT_FUSED])
def test_decode_distinct_any_split(splits, variant):
    call = run_workload(workloads.decode_distinct(), variant, splits)
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")
    assert call.counters_clear()


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
@pytest.mark.parametrize("kind,n", [("identical", 32), ("identical", 64), ("uniform", 32),
                                    ("uniform", 64), ("skewed", 32), ("skewed", 64)])
def test_popularity_sweep(kind, n, variant):
    call = run_workload(workloads.popularity(kind, n), variant)
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")
    assert call.counters_clear()


@pytest.mark.parametrize("kind,n", [("identical", 32), ("uniform", 64), ("skewed", 64)])
def test_popularity_auto_takes_one_launch_route(kind, n):
    """Decode-shaped batches run the one-launch kernel with one-row blocks."""
    call = run_workload(workloads.popularity(kind, n))
    info = sg.sgmv_query_plan(call.problem)
    assert (info.route, info.launches, info.rows_per_unit) == (sg.SGMV_ROUTE_DECODE, 1, 1), info.as_dict()


@pytest.mark.parametrize("kind,n,splits,rows_per_unit", [
    ("identical", 32, 128, 4), ("identical", 32, 256, 16), ("identical", 64, 128, 16),
    ("skewed", 32, 64, None), ("uniform", 64, 32, None), ("skewed", 64, 48, None)])
def test_popularity_larger_row_blocks(kind, n, splits, rows_per_unit):
    """Forcing more splits pushes the one-launch kernel to 4- and 16-row blocks
    (the plans that larger batches get), or off it when no plan fits on the
    device at once; the result must not change.  (32 one-row units of 128
    splits exceed the 2048 workgroups a 256-CU device can ever hold at once;
    the 16-row cases also exceed what the 4-row kernel's occupancy holds.)"""
    call = run_workload(workloads.popularity(kind, n), sg.SGMV_VARIANT_FUSED, splits)
    info = sg.sgmv_query_plan(call.problem)
    if rows_per_unit is not None:
        assert (info.route, info.rows_per_unit) == (sg.SGMV_ROUTE_DECODE, rows_per_unit), info.as_dict()
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")
    assert call.counters_clear()


@pytest.mark.parametrize("case", ["distinct_b512", "distinct_b100_h1024_splits32", "skewed_b64_splits64",
                                  "uniform_b32_splits128"])
def test_decode_passes_when_units_exceed_the_device(case):
    """When the units of a decode-shaped batch do not all fit on the device at
    once, the decode kernel is launched in passes, each over the next units with
    the largest co-resident grid; the result must equal the oracle, and the plan
    must be that multi-pass one."""
    if case == "distinct_b512":
        call = run_workload(workloads.decode_distinct(n=512), sg.SGMV_VARIANT_AUTO)
    elif case == "distinct_b100_h1024_splits32":
        call = run_workload(workloads.decode_distinct(n=100, h=1024), sg.SGMV_VARIANT_FUSED, 32)
    elif case == "skewed_b64_splits64":
        call = run_workload(workloads.popularity("skewed", 64), sg.SGMV_VARIANT_FUSED, 64)
    else:
        call = run_workload(workloads.popularity("uniform", 32), sg.SGMV_VARIANT_FUSED, 128)
    info = sg.sgmv_query_plan(call.problem)
    assert info.route == sg.SGMV_ROUTE_DECODE, info.as_dict()
    assert info.launches > 1 and info.grid < info.units * info.splits, info.as_dict()
    rows = None if call.Xh.shape[0] <= 128 else np.r_[0:8, 120:136, call.Xh.shape[0] - 8:call.Xh.shape[0]]
    mask = None
    if rows is not None:
        mask = np.zeros(call.Xh.shape[0], np.uint8)
        mask[rows] = 1
    ref = call.oracle_apply(row_mask=mask)
    assert_close(to_bits(call.apply()), ref, "f16", rows=rows)


def _batched_case(w, variant, nproj, seed):
    """nproj projections of one workload's rows: projection 0 uses the workload's
    weights and Y0; the others draw their own (seeded) weights and Y0."""
    rng = np.random.default_rng(seed)
    call = run_workload(w, variant)
    projs = [(call.A, call.B, call.Y, call.A_ptrs, call.B_ptrs, call.Ah, call.Bh, call.Y0h)]
    P, h_in, r = call.Ah.shape
    h_out = call.Bh.shape[2]
    for _ in range(nproj - 1):
        Ah = workloads.to_bits((rng.standard_normal((P, h_in, r)) * h_in ** -0.5).astype(np.float32), w.dtype)
        Bh = workloads.to_bits((rng.standard_normal((P, r, h_out)) * r ** -0.5).astype(np.float32), w.dtype)
        Y0h = workloads.to_bits(rng.standard_normal(call.Y0h.shape).astype(np.float32), w.dtype)
        A, B, Y = to_device(Ah, w.dtype), to_device(Bh, w.dtype), to_device(Y0h, w.dtype)
        projs.append((A, B, Y, sg.pointer_table(A), sg.pointer_table(B), Ah, Bh, Y0h))
    return call, projs


@pytest.mark.parametrize("case", ["distinct3", "distinct_b64_4", "distinct_b128_4", "skewed3", "mixed2_mfma",
                                  "distinct3_vector"])
def test_batched_projections_match_oracle_and_single_calls(case):
    """sgmv_lora_apply_batched: every projection equals the oracle, and equals
    (bitwise) a separate sgmv_lora_apply of that projection.  Distinct b128 with
    4 projections (4096 workgroups) exceeds what the device holds at once and
    runs the per-projection fallback."""
    import torch
    w, variant, nproj = {
        "distinct3": (workloads.decode_distinct(), sg.SGMV_VARIANT_AUTO, 3),
        "distinct_b64_4": (workloads.decode_distinct(n=64), sg.SGMV_VARIANT_AUTO, 4),
        "distinct_b128_4": (workloads.decode_distinct(n=128), sg.SGMV_VARIANT_AUTO, 4),
        "skewed3": (workloads.popularity("skewed", 32), sg.SGMV_VARIANT_AUTO, 3),
        "mixed2_mfma": (workloads.mixed(64, seed=464, pairs=((512, 1376),), lo=16, hi=100)[0],
                        sg.SGMV_VARIANT_MFMA, 2),
        "distinct3_vector": (workloads.decode_distinct(), sg.SGMV_VARIANT_VECTOR, 3),
    }[case]
    call, projs = _batched_case(w, variant, nproj, seed=77)
    ws = torch.zeros(sg.batched_workspace_bytes(call.problem, nproj), dtype=torch.uint8, device="cuda")
    sg.sgmv_lora_apply_batched(call.problem, call.X, [(a, b, y) for (_, _, y, a, b, *_rest) in projs],
                               call.seg_d, call.lidx_d, ws)
    torch.cuda.synchronize()
    got = [to_bits(pj[2]).copy() for pj in projs]
    for i, (_, _, Y, A_ptrs, B_ptrs, Ah, Bh, Y0h) in enumerate(projs):
        ref = oracle.sgmv_apply(w.dtype, call.Xh, Ah, Bh, call.seg, call.lidx, Y0h)
        assert_close(got[i], ref, w.dtype, what=f"projection {i}")
        Y.copy_(to_device(Y0h, w.dtype))
        ws1 = sg.new_workspace(call.problem)
        sg.sgmv_lora_apply(call.problem, call.X, A_ptrs, B_ptrs, Y, call.seg_d, call.lidx_d, ws1)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(Y), got[i]), f"projection {i}: batched != single call"


@pytest.mark.parametrize("case", ["distinct", "skewed", "identical_rb4", "identical_rb16", "skewed_vector",
                                  "mixed_mfma_random_map"])
def test_row_map_gathers_and_scatters_rows(case):
    """With row_idx the kernels read X and update Y in request order: the result
    equals the oracle on the sorted rows, scattered back through the map, and
    rows outside the map keep their values."""
    import torch
    if case == "mixed_mfma_random_map":
        w = workloads.mixed(16, seed=416, pairs=((512, 1376),), lo=16, hi=100)[0]
        seg, lidx = np.asarray(w.seg_indptr, np.int32), np.asarray(w.lora_idx, np.int32)
        n = w.X.shape[0]
        perm = np.random.default_rng(3).permutation(n + 7)[: n].astype(np.int32)  # rows among n + 7
        X = np.zeros((n + 7, w.X.shape[1]), np.uint16); X[perm] = w.X
        Y0 = workloads.to_bits(np.random.default_rng(4).standard_normal((n + 7, w.Y0.shape[1])).astype(np.float32),
                               w.dtype)
        variant, splits = sg.SGMV_VARIANT_MFMA, 0
    else:
        kind, n, variant, splits = {"distinct": ("distinct", 32, sg.SGMV_VARIANT_AUTO, 0),
                                    "skewed": ("skewed", 64, sg.SGMV_VARIANT_AUTO, 0),
                                    "identical_rb4": ("identical", 32, sg.SGMV_VARIANT_FUSED, 64),
                                    "identical_rb16": ("identical", 64, sg.SGMV_VARIANT_FUSED, 128),
                                    "skewed_vector": ("skewed", 32, sg.SGMV_VARIANT_VECTOR, 0)}[case]
        w = workloads.popularity(kind, n) if kind != "distinct" else workloads.decode_distinct()
        if w.req_lora is None:  # Distinct: requests in a shuffled order
            w.req_lora = np.random.default_rng(5).permutation(w.num_loras)[: w.X.shape[0]].astype(np.int32)
        perm, seg, lidx, _ = sg.sgmv_build_segments(w.req_lora, w.num_loras)
        X, Y0 = w.X, w.Y0                    # request order
    call = DeviceCall(w.dtype, X, w.A, w.B, Y0, seg, lidx, variant=variant, splits=splits)
    ws = sg.new_workspace(call.problem)
    sg.sgmv_lora_apply_batched(call.problem, call.X, [(call.A_ptrs, call.B_ptrs, call.Y)], call.seg_d,
                               call.lidx_d, ws, row_idx=torch.from_numpy(np.ascontiguousarray(perm)).cuda())
    torch.cuda.synchronize()
    ref_sorted = oracle.sgmv_apply(w.dtype, X[perm], w.A, w.B, seg, lidx, Y0[perm])
    ref = oracle.decode(Y0, w.dtype)
    ref[perm] = ref_sorted
    assert_close(to_bits(call.Y), ref, w.dtype, what=case)


@pytest.mark.parametrize("variant", [sg.SGMV_VARIANT_AUTO, sg.SGMV_VARIANT_VECTOR, sg.SGMV_VARIANT_MFMA])
@pytest.mark.parametrize("rank", [16, 64])
def test_mixed_prefill_decode_reduced(rank, variant):
    """Config-4 layout (8 prefill + 24 one-row segments, 16 LoRAs, bf16) with prefill
    lengths 16..100 and hidden sizes 512/1376, small enough for a full comparison."""
    for w in workloads.mixed(rank, seed=400 + rank, pairs=((512, 1376), (1376, 512)), lo=16, hi=100):
        call = run_workload(w, variant)
        assert_close(to_bits(call.apply()), call.oracle_apply(), "bf16", what=w.name)


@pytest.mark.parametrize("rank", [16, 64])
def test_mixed_prefill_decode_full_size_sampled(rank):
    """Config 4 at full size (Llama-7B MLP shapes, ~4.6k rows), oracle on sampled rows."""
    for w in workloads.mixed(rank):
        call = run_workload(w)
        got = to_bits(call.apply())
        rng = np.random.default_rng(7)
        seg = call.seg
        rows = set(int(r) for r in rng.choice(call.Xh.shape[0], size=24, replace=False))
        for s in range(len(seg) - 1):       # first and last row of every segment
            if seg[s + 1] > seg[s]:
                rows.update((int(seg[s]), int(seg[s + 1] - 1)))
        rows = np.array(sorted(rows))
        mask = np.zeros(call.Xh.shape[0], np.uint8)
        mask[rows] = 1
        ref = call.oracle_apply(row_mask=mask)
        assert_close(got, ref, "bf16", rows=rows, what=w.name)


# ------------------------------------------------------------ bit-exact pins

INT_EXACT = {("f16", 8): (64, 512), ("f16", 16): (64, 512), ("f16", 32): (32, 512),
             ("f16", 64): (16, 512), ("bf16", 8): (16, 64), ("bf16", 16): (8, 64),
             ("bf16", 32): (4, 64), ("bf16", 64): (2, 64)}


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
@pytest.mark.parametrize("dtype,rank", sorted(INT_EXACT))
def test_integer_exact_inputs_bitwise(dtype, rank, variant):
    m, c = INT_EXACT[(dtype, rank)]
    rng = np.random.default_rng(1000 + rank)
    X, A, B, Y0 = workloads.integer_exact(rng, 24, 256, 264, rank, 4, dtype, m, c)
    seg, lidx = [0, 5, 5, 6, 9, 17, 24], [3, 1, 0, 3, 2, 1]
    call = DeviceCall(dtype, X, A, B, Y0, seg, lidx, variant=variant)
    if not mfma_rank_ok(variant, rank):
        return expect_unsupported(call)
    got = oracle.decode(to_bits(call.apply()), dtype)
    assert np.array_equal(got, call.oracle_apply())


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
def test_integer_exact_full_decode_shape(variant):
    rng = np.random.default_rng(2024)
    X, A, B, Y0 = workloads.integer_exact(rng, 32, 4096, 4096, 16, 32, "f16", 64, 512)
    call = DeviceCall("f16", X, A, B, Y0, np.arange(33), np.arange(32)[::-1].copy(), variant=variant)
    assert np.array_equal(oracle.decode(to_bits(call.apply()), "f16"), call.oracle_apply())


@pytest.mark.parametrize("variant", [sg.SGMV_VARIANT_AUTO, sg.SGMV_VARIANT_VECTOR, sg.SGMV_VARIANT_MFMA])
def test_integer_exact_shrink_bitwise(variant):
    rng = np.random.default_rng(77)
    X, A, B, Y0 = workloads.integer_exact(rng, 40, 512, 64, 32, 3, "bf16", 4, 64)
    seg, lidx = [0, 1, 21, 40], [2, 0, 1]
    call = DeviceCall("bf16", X, A, B, Y0, seg, lidx, variant=variant)
    V = call.shrink().cpu().numpy().astype(np.float64)
    assert np.array_equal(V, oracle.sgmv_shrink("bf16", X, A, seg, lidx))


@pytest.mark.parametrize("rank,h_in,launches", [(16, 4096, 2), (64, 8192, 2)])
def test_integer_exact_many_planes_bitwise(rank, h_in, launches):
    """A long H1 on full 64-row tiles: 16 partial planes at rank 16 and 11 at
    rank 64, summed by the lead workgroups of the expand launch (row-block
    flags); the standalone shrink's reduce launch is checked on the same
    planes.  Integer inputs make every result exact, so every way of summing
    the planes must give the oracle's bits."""
    rng = np.random.default_rng(5000 + rank)
    m, c = INT_EXACT[("bf16", rank)]
    X, A, B, Y0 = workloads.integer_exact(rng, 256, h_in, 256, rank, 3, "bf16", m, c)
    call = DeviceCall("bf16", X, A, B, Y0, [0, 128, 256], [2, 0], variant=sg.SGMV_VARIANT_MFMA)
    info = sg.sgmv_query_plan(call.problem)
    assert (info.route, info.launches) == (sg.SGMV_ROUTE_MFMA, launches), info.as_dict()
    assert info.splits > 8, info.as_dict()
    assert np.array_equal(oracle.decode(to_bits(call.apply()), "bf16"), call.oracle_apply())
    V = call.shrink().cpu().numpy().astype(np.float64)
    assert np.array_equal(V, oracle.sgmv_shrink("bf16", X, A, [0, 128, 256], [2, 0]))


# ------------------------------------------------------------ edge cases

def rand_inputs(seed, n, h_in, h_out, rank, P, dtype="f16"):
    rng = np.random.default_rng(seed)
    X = workloads.to_bits(rng.standard_normal((n, h_in), dtype=np.float32), dtype)
    A = workloads.to_bits(rng.standard_normal((P, h_in, rank), dtype=np.float32) / np.sqrt(h_in), dtype)
    B = workloads.to_bits(rng.standard_normal((P, rank, h_out), dtype=np.float32) / np.sqrt(rank), dtype)
    Y0 = workloads.to_bits(rng.standard_normal((n, h_out), dtype=np.float32), dtype)
    return X, A, B, Y0


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
def test_empty_unsorted_repeated_segments_and_uncovered_rows(variant):
    X, A, B, Y0 = rand_inputs(1, 20, 256, 128, 16, 5)
    seg, lidx = [0, 0, 3, 3, 4, 9, 9, 15], [4, 2, 2, 0, 1, 3, 2]   # rows 15.. uncovered
    call = DeviceCall("f16", X, A, B, Y0, seg, lidx, variant=variant)
    got = to_bits(call.apply())
    assert_close(got, call.oracle_apply(), "f16")
    assert np.array_equal(got[15:], Y0[15:])
    assert call.counters_clear()


@pytest.mark.parametrize("layout", ["full_tiles", "short_tiles"])
def test_split_sum_in_the_expand_launch_with_empty_unsorted_segments_and_uncovered_rows(layout):
    """The matrix-core route with several H1 planes (their sum done by lead
    workgroups of the expand launch: row-block flags for full tiles, tagged V
    words for short ones, one float4 or one float2 per thread), on a batch with
    empty, repeated and unsorted segments, rows that no segment covers (left
    untouched), and H1 / H2 that are not multiples of the tile sizes."""
    if layout == "full_tiles":
        n, h_in, seg, lidx = 150, 4104, [0, 0, 70, 70, 71, 130], [4, 2, 2, 0, 3]
    else:
        n, h_in = 90, 8200
        seg = [0, 3, 3, 10, 17, 20, 20, 31, 35, 44, 50, 61, 62, 75, 80]
        lidx = [1, 4, 0, 2, 3, 3, 0, 1, 4, 2, 2, 0, 1, 3]
    X, A, B, Y0 = rand_inputs(30 + len(seg), n, h_in, 1000, 64, 5, "bf16")
    call = DeviceCall("bf16", X, A, B, Y0, seg, lidx, variant=sg.SGMV_VARIANT_MFMA)
    info = sg.sgmv_query_plan(call.problem)
    assert info.route == sg.SGMV_ROUTE_MFMA and info.splits > 1 and info.launches == 2, info.as_dict()
    end = seg[-1]
    for _ in range(2):  # the second call finds the first call's V words and flags in the workspace
        call.reset_y()
        got = to_bits(call.apply())
        assert_close(got, call.oracle_apply(), "bf16")
        assert np.array_equal(got[end:], Y0[end:])
    assert sg.sgmv_take_device_errors() == 0


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
def test_no_segments_is_a_no_op(variant):
    X, A, B, Y0 = rand_inputs(2, 8, 64, 64, 16, 2)
    call = DeviceCall("f16", X, A, B, Y0, [0], [], variant=variant)
    assert np.array_equal(to_bits(call.apply()), Y0)
    call2 = DeviceCall("f16", X, A, B, Y0, [0, 0, 0], [1, 0], variant=variant)
    assert np.array_equal(to_bits(call2.apply()), Y0)


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
@pytest.mark.parametrize("h_in,h_out", [(8, 8), (24, 40), (4104, 1000), (11008, 8)])
def test_ragged_hidden_sizes(h_in, h_out, variant):
    X, A, B, Y0 = rand_inputs(3, 6, h_in, h_out, 16, 3, "bf16")
    call = DeviceCall("bf16", X, A, B, Y0, [0, 2, 3, 6], [2, 0, 1], variant=variant)
    assert_close(to_bits(call.apply()), call.oracle_apply(), "bf16")


@pytest.mark.parametrize("row_map", [False, True])
@pytest.mark.parametrize("rank", [16, 32, 64])
@pytest.mark.parametrize("h_in,dtype", [(40, "bf16"), (4104, "f16"), (4104, "bf16")])
def test_full_row_tiles(h_in, dtype, rank, row_map):
    """Segments long enough for full 64-row tiles (at least 32 rows per tile on
    average, where the matrix-core shrink stages X through LDS), with a ragged
    H1 (40 = a stage of 128 holding 5 vectors; 4104 = 32 stages plus 8), every
    rank, in segment order and through a row map among spare rows."""
    import torch
    n, h_out, P = 200, 264, 3
    seg, lidx = [0, 130, 131, 200], [2, 0, 1]
    tiles = sum(-(-(b - a) // 64) for a, b in zip(seg, seg[1:]))
    assert n >= 32 * tiles
    Xs, A, B, Y0s = rand_inputs(11 + rank, n, h_in, h_out, rank, P, dtype)
    if row_map:
        perm = np.random.default_rng(rank).permutation(n + 5)[:n].astype(np.int32)
        X = np.zeros((n + 5, h_in), np.uint16); X[perm] = Xs
        Y0 = workloads.to_bits(np.random.default_rng(9).standard_normal((n + 5, h_out)).astype(np.float32), dtype)
        Y0[perm] = Y0s
    else:
        X, Y0 = Xs, Y0s
    call = DeviceCall(dtype, X, A, B, Y0, seg, lidx, variant=sg.SGMV_VARIANT_MFMA)
    assert sg.sgmv_query_plan(call.problem).route == sg.SGMV_ROUTE_MFMA
    row_idx = torch.from_numpy(perm).cuda() if row_map else None
    sg.sgmv_lora_apply_batched(call.problem, call.X, [(call.A_ptrs, call.B_ptrs, call.Y)], call.seg_d,
                               call.lidx_d, call.ws, row_idx=row_idx)
    torch.cuda.synchronize()
    ref_sorted = oracle.sgmv_apply(dtype, Xs, A, B, np.asarray(seg, np.int32), np.asarray(lidx, np.int32), Y0s)
    if row_map:
        ref = oracle.decode(Y0, dtype)
        ref[perm] = ref_sorted
    else:
        ref = ref_sorted
    assert_close(to_bits(call.Y), ref, dtype, what=f"h_in {h_in} rank {rank}")


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
@pytest.mark.parametrize("rank", [8, 32, 64])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_ranks(rank, dtype, variant):
    X, A, B, Y0 = rand_inputs(4 + rank, 40, 1024, 768, rank, 6, dtype)
    seg, lidx = [0, 1, 2, 6, 7, 23, 24, 40], [5, 0, 3, 3, 1, 2, 4]
    call = DeviceCall(dtype, X, A, B, Y0, seg, lidx, variant=variant)
    if not mfma_rank_ok(variant, rank):
        return expect_unsupported(call)
    assert_close(to_bits(call.apply()), call.oracle_apply(), dtype)


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
def test_one_long_segment(variant):
    X, A, B, Y0 = rand_inputs(5, 300, 512, 256, 16, 2)
    call = DeviceCall("f16", X, A, B, Y0, [0, 300], [1], variant=variant)
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")


@pytest.mark.parametrize("variant", APPLY_VARIANTS)
def test_many_segments_more_than_a_wave(variant):
    # 150 segments mixing lengths 0..3 (unit lookup scans segments 64 at a time)
    rng = np.random.default_rng(6)
    lens = rng.integers(0, 4, size=150)
    seg = np.concatenate([[0], np.cumsum(lens)])
    n = int(seg[-1]) + 5
    X, A, B, Y0 = rand_inputs(6, n, 128, 64, 16, 7)
    call = DeviceCall("f16", X, A, B, Y0, seg, rng.integers(0, 7, size=150), variant=variant)
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")


def test_max_seg_len_bound_above_actual():
    """max_seg_len is an upper bound: a looser bound must not change the result."""
    X, A, B, Y0 = rand_inputs(8, 12, 256, 256, 16, 3)
    seg, lidx = [0, 2, 3, 12], [1, 0, 2]
    ref = None
    for bound in (9, 12):
        call = DeviceCall("f16", X, A, B, Y0, seg, lidx, max_seg_len=bound)
        got = to_bits(call.apply())
        ref = call.oracle_apply() if ref is None else ref
        assert_close(got, ref, "f16")


# ------------------------------------------------------------ the separate stages

@pytest.mark.parametrize("variant", [sg.SGMV_VARIANT_AUTO, sg.SGMV_VARIANT_MFMA])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("rank", [8, 16, 64])
def test_shrink_matches_oracle(dtype, rank, variant):
    if not mfma_rank_ok(variant, rank):
        pytest.skip("matrix-core kernels take ranks 16, 32, 64 (error path covered elsewhere)")
    X, A, B, Y0 = rand_inputs(9, 30, 2048, 64, rank, 4, dtype)
    seg, lidx = [0, 1, 9, 9, 25], [3, 0, 1, 2]           # rows 25..29 uncovered
    call = DeviceCall(dtype, X, A, B, Y0, seg, lidx, variant=variant)
    V = call.shrink().cpu().numpy()
    ref = oracle.sgmv_shrink(dtype, X, A, seg, lidx)
    assert_close_f32(V[:25].astype(np.float64), ref[:25])
    assert np.isnan(V[25:]).all()


@pytest.mark.parametrize("variant", [sg.SGMV_VARIANT_AUTO, sg.SGMV_VARIANT_VECTOR, sg.SGMV_VARIANT_MFMA])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_expand_matches_oracle(dtype, variant):
    import torch
    X, A, B, Y0 = rand_inputs(10, 30, 64, 3000, 32, 4, dtype)
    seg, lidx = [0, 7, 8, 20], [1, 3, 0]
    rng = np.random.default_rng(11)
    Vh = rng.standard_normal((30, 32)).astype(np.float32)
    call = DeviceCall(dtype, X, A, B, Y0, seg, lidx, variant=variant)
    got = to_bits(call.expand(torch.from_numpy(Vh).cuda()))
    ref = oracle.sgmv_expand(dtype, Vh.astype(np.float64), B, seg, lidx, Y0)
    assert_close(got, ref, dtype)
    assert np.array_equal(got[20:], Y0[20:])


def test_results_are_deterministic():
    call = run_workload(workloads.popularity("skewed", 64), sg.SGMV_VARIANT_AUTO)
    first = to_bits(call.apply())
    for _ in range(3):
        call.reset_y()
        assert np.array_equal(to_bits(call.apply()), first)


def test_back_to_back_calls_share_workspace():
    """Calls of different shapes on one workspace (counters must come back to zero)."""
    import torch
    calls = [run_workload(workloads.decode_distinct(seed=30 + i, n=8 + 8 * i, h=1024)) for i in range(3)]
    nbytes = max(sg.sgmv_workspace_bytes(c.problem) for c in calls)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for c in calls:
            c.ws = ws
            c.reset_y()
            assert_close(to_bits(c.apply()), c.oracle_apply(), "f16")
    assert bool((ws[: sg.SGMV_WS_COUNTER_BYTES] == 0).all().item())


# ------------------------------------------------------------ 13B full-model shapes

@pytest.mark.parametrize("row_layout", ["segment_order", "row_map"])
def test_llama13b_layer_sampled(row_layout):
    """One layer of the 13B full-model sweep at its real shapes: q, k, v (5120 -> 5120)
    batched in one call, o alone, gate and up (5120 -> 13824) batched, down
    (13824 -> 5120) alone; r = 64, bf16, 64 LoRAs per projection, 256 decode rows
    with truncated Zipf(1.5) LoRA ids (a request keeps its LoRA in every projection),
    segments from the library's builder (checked against the oracle's).  Weights
    and activations are drawn on the device from seeded generators; every
    projection is compared element by element with the fp64 oracle on the first
    and last row of every segment plus 24 random rows.  In "row_map" the
    activations stay in request order and the kernels gather / scatter rows
    through the builder's perm."""
    import torch
    n, rank, P = 256, 64, 64
    ids = workloads.full_model_ids(seed=5, n=n, pool=P)
    perm, seg, lidx, mx = sg.sgmv_build_segments(ids, P)
    operm, oseg, olidx, omx = oracle.build_segments(ids, P)
    assert (perm.tolist(), seg.tolist(), lidx.tolist(), mx) == (operm, oseg, olidx, omx)
    used = sorted(set(int(k) for k in lidx))
    seg_d = torch.from_numpy(seg).cuda()
    lidx_d = torch.from_numpy(lidx).cuda()
    perm_d = torch.from_numpy(np.ascontiguousarray(perm)).cuda() if row_layout == "row_map" else None
    # sorted row j holds request perm[j]: with a row map, X / Y rows stay in request order
    order = perm if row_layout == "row_map" else np.arange(n)
    rng = np.random.default_rng(13)
    sample = set(int(r) for r in rng.choice(n, 24, replace=False))
    for s in range(len(seg) - 1):
        sample.update((int(seg[s]), int(seg[s + 1]) - 1))
    mask = np.zeros(n, np.uint8)
    mask[sorted(sample)] = 1
    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    shapes = {name: (h_in, h_out) for (name, h_in, h_out) in workloads.LLAMA13B_PROJ}
    names = [name for (name, _, _) in workloads.LLAMA13B_PROJ]
    layer = 7
    for gi, grp in enumerate(groups):
        h_in, h_out = shapes[grp[0]]
        X = workloads.device_normal((n, h_in), 1.0, "bf16", 880000 + 4 * layer + gi)
        projs, host = [], []
        for name in grp:
            seed = workloads.full_model_weight_seed(layer, names.index(name))
            A = workloads.device_normal((P, h_in, rank), h_in ** -0.5, "bf16", seed * 2)
            B = workloads.device_normal((P, rank, h_out), rank ** -0.5, "bf16", seed * 2 + 1)
            Y = workloads.device_normal((n, h_out), 1.0, "bf16", 890000 + 7 * layer + names.index(name))
            host.append((Y, to_bits(Y), [to_bits(A[k]) if k in used else np.zeros((1, 1), np.uint16)
                                         for k in range(P)],
                         [to_bits(B[k]) if k in used else np.zeros((1, 1), np.uint16) for k in range(P)]))
            projs.append((sg.pointer_table(A), sg.pointer_table(B), Y, A, B))
        prob = sg.make_problem("bf16", n, h_in, h_out, rank, P, len(lidx), mx)
        assert sg.sgmv_query_plan(prob).route == sg.SGMV_ROUTE_MFMA
        ws = torch.zeros(sg.batched_workspace_bytes(prob, len(grp)), dtype=torch.uint8, device="cuda")
        Xh = to_bits(X)
        sg.sgmv_lora_apply_batched(prob, X, [(a, b, y) for (a, b, y, _, _) in projs], seg_d, lidx_d, ws,
                                   row_idx=perm_d)
        torch.cuda.synchronize()
        for name, (Y, Y0h, Ah, Bh) in zip(grp, host):
            # the oracle works on sorted rows: sorted row j is activation row order[j]
            ref = oracle.sgmv_apply("bf16", Xh[order], Ah, Bh, seg, lidx, Y0h[order], row_mask=mask)
            got = to_bits(Y)[order]
            assert_close(got, ref, "bf16", rows=mask.astype(bool), what=f"{row_layout} {name}")
            assert np.isfinite(oracle.decode(to_bits(Y), "bf16")).all()


@pytest.mark.parametrize("variant", [sg.SGMV_VARIANT_MFMA, sg.SGMV_VARIANT_VECTOR, sg.SGMV_VARIANT_AUTO])
def test_f16_large_intermediate(variant):
    """fp16 inputs whose intermediate V = x @ A_k exceeds fp16's range (|V| up to
    ~1e5, the term itself and Y in range): every route keeps V in fp32 or, on the
    matrix cores, splits a power-of-two scaled copy of it, so every route meets
    the oracle bound; rows with small V share the tiles."""
    rng = np.random.default_rng(55)
    n, h_in, h_out, rank, P = 48, 512, 256, 16, 3
    Xf = rng.standard_normal((n, h_in)).astype(np.float32)
    Xf[24:] *= 1e-3                                  # small-V rows beside the large ones
    Af = (rng.standard_normal((P, h_in, rank)) * 4000.0).astype(np.float32)
    Bf = (rng.standard_normal((P, rank, h_out)) * 1e-3).astype(np.float32)
    Y0f = rng.standard_normal((n, h_out)).astype(np.float32)
    X, A, B, Y0 = (workloads.to_bits(a, "f16") for a in (Xf, Af, Bf, Y0f))
    seg, lidx = [0, 20, 21, 48], [2, 0, 1]
    call = DeviceCall("f16", X, A, B, Y0, seg, lidx, variant=variant)
    _, V = oracle.sgmv_apply("f16", X, A, B, seg, lidx, Y0, want_v=True)
    assert np.nanmax(np.abs(V)) > 65504.0
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")
