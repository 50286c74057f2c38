"""Parity of sgmv_base_lora_apply (Y = X @ W + per-row LoRA term, rounded once)
against the fp64 oracle, through the C ABI.

Cases cover: one row per LoRA (the decode batch of the headline shape, full
size), repeated LoRAs, rows no segment covers, no segments at all (Y = X @ W),
a single row, 64, 96 and 128 rows, ragged K (h_in not a multiple of the 128-row stage) and
ragged column strips (h_out not a multiple of 128), both formats, every rank,
and integer-valued inputs whose result is exact (compared bit for bit).  The
row-parallel shard entry point (sgmv_base_lora_apply_partial) is checked shard by
shard against the oracle on each H1 slice, summed against the whole product,
and, with one slice, rounded against sgmv_base_lora_apply bit for bit."""
import numpy as np
import pytest

import oracle
import segmented_gather_matvec_amd as sg
import workloads
from tests.gpu_cases import assert_close, assert_close_f32, i32, to_bits, to_device

pytestmark = pytest.mark.gpu


def packed_layout(W):
    """The packed layout, built with numpy from its definition: block (nb, ks) holds
    W[32 ks + 8 q + e][16 nb + m] at element 8 (16 q + m) + e; zero past the matrix."""
    h_in, h_out = W.shape
    kst = -(-h_in // 128) * 4
    nbp = -(-(-(-h_out // 16)) // 2) * 2
    Wpad = np.zeros((kst * 32, nbp * 16), np.uint16)
    Wpad[:h_in, :h_out] = W
    t = Wpad.reshape(kst, 4, 8, nbp, 16)           # [ks][q][e][nb][m]
    return t.transpose(3, 0, 1, 4, 2).reshape(-1)  # [nb][ks][q][m][e]


def run_base(dtype, X, W, A, B, seg, lidx, Y_fill=None, packed=False):
    import torch
    n, h_in = X.shape
    P, _, rank = A.shape
    h_out = W.shape[1]
    seg = np.asarray(seg, np.int32)
    lidx = np.asarray(lidx, np.int32)
    mx = int(np.diff(seg).max()) if len(seg) > 1 else 0
    prob = sg.make_problem(dtype, n, h_in, h_out, rank, P, len(lidx), mx)
    Xd, Wd, Ad, Bd = (to_device(a, dtype) for a in (X, W, A, B))
    Y = torch.full((n, h_out), float("nan") if Y_fill is None else Y_fill, dtype=Xd.dtype, device="cuda")
    ws = torch.full((sg.sgmv_base_workspace_bytes(prob),), 0xA5, dtype=torch.uint8, device="cuda")  # any contents
    fn = sg.sgmv_base_lora_apply
    if packed:
        Wd = sg.pack_base_weight(Wd)
        fn = sg.sgmv_base_lora_apply_packed
    fn(prob, Xd, Wd, sg.pointer_table(Ad), sg.pointer_table(Bd), Y,
       i32(seg if seg.size else [0]), i32(lidx if lidx.size else [0]), ws)
    torch.cuda.synchronize()
    return to_bits(Y), prob, (Xd, Wd, Ad, Bd, Y, ws, seg, lidx)


def make_case(seed, dtype, n, h_in, h_out, rank, P, layout):
    rng = np.random.default_rng(seed)
    X, A, B, _ = workloads._values(rng, n, h_in, h_out, rank, P, dtype)
    W = workloads.base_weight(rng, h_in, h_out, dtype)
    if layout == "distinct":                  # row i -> LoRA i
        seg, lidx = list(range(n + 1)), list(range(n))
    elif layout == "skewed":                  # builder-sorted Zipf ids
        ids = np.minimum(rng.zipf(1.5, size=n) - 1, P - 1).astype(np.int32)
        perm, seg, lidx, _ = sg.sgmv_build_segments(ids, P)
        X = X[perm]
        seg, lidx = seg.tolist(), lidx.tolist()
    elif layout == "tail_uncovered":          # rows past 2n/3 have no LoRA
        cut = 2 * n // 3
        seg, lidx = [0, cut // 2, cut], [P - 1, 0]
    elif layout == "none":
        seg, lidx = [0], []
    else:
        raise ValueError(layout)
    return X, W, A, B, seg, lidx


CASES = {
    # name: (seed, dtype, n, h_in, h_out, rank, P, layout)
    "distinct_b32_h4096_r16": (2, "f16", 32, 4096, 4096, 16, 32, "distinct"),
    "skewed_b64_bf16_r64": (3, "bf16", 64, 1024, 1376, 64, 16, "skewed"),
    "tail_uncovered_ragged": (4, "f16", 20, 520, 264, 8, 4, "tail_uncovered"),
    "no_segments_bf16": (5, "bf16", 7, 384, 512, 32, 2, "none"),
    "one_row_r32": (6, "bf16", 1, 2048, 1024, 32, 3, "distinct"),
    "distinct_b64_f16_r8": (7, "f16", 64, 256, 2056, 8, 64, "distinct"),
    # 40 rows (four row tiles) over many strips: the packed kernel's LDS cap on
    # the X chunk (512 k) cuts the K chunk below the row-major call's 640
    "capped_chunk_b40_bf16_r32": (9, "bf16", 40, 2560, 8200, 32, 6, "skewed"),
    # eight row tiles (65..128 rows): the packed kernel stages 128 rows of X
    # (K chunk up to 512, the row-major call's chunk here)
    "distinct_b128_f16_r16": (10, "f16", 128, 4096, 4096, 16, 128, "distinct"),
    "skewed_b96_bf16_r64": (11, "bf16", 96, 1536, 1032, 64, 24, "skewed"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_base_apply_matches_oracle(name):
    seed, dtype, n, h_in, h_out, rank, P, layout = CASES[name]
    X, W, A, B, seg, lidx = make_case(seed, dtype, n, h_in, h_out, rank, P, layout)
    got, _, _ = run_base(dtype, X, W, A, B, seg, lidx)
    ref = oracle.sgmv_base_apply(dtype, X, W, A, B, seg, lidx)
    assert_close(got, ref, dtype, what=name)


@pytest.mark.parametrize("shape", [(520, 264), (1024, 1376), (4096, 4096), (8, 24)])
def test_packed_weight_layout_bit_exact(shape):
    """sgmv_base_pack_weight writes exactly the documented layout (bit for bit)."""
    import torch
    rng = np.random.default_rng(sum(shape))
    W = workloads.base_weight(rng, shape[0], shape[1], "bf16")
    Wd = to_device(W, "bf16")
    Wp = torch.full((sg.sgmv_base_packed_weight_bytes(*shape) // 2,), 12345, dtype=torch.int16,
                    device="cuda").view(torch.bfloat16)  # every element must be written
    sg.sgmv_base_pack_weight(Wd, Wp)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(Wp), packed_layout(W))


@pytest.mark.parametrize("name", sorted(CASES))
def test_packed_base_apply_matches_oracle_and_row_major_call(name):
    """The packed entry point meets the oracle bound.  Where both calls split K alike (every
    case but the capped one, whose packed call takes 5 planes against 4) it also equals the
    row-major call bit for bit: the same MFMA operands in the same order."""
    seed, dtype, n, h_in, h_out, rank, P, layout = CASES[name]
    X, W, A, B, seg, lidx = make_case(seed, dtype, n, h_in, h_out, rank, P, layout)
    got, _, _ = run_base(dtype, X, W, A, B, seg, lidx, packed=True)
    assert_close(got, oracle.sgmv_base_apply(dtype, X, W, A, B, seg, lidx), dtype, what=name)
    row_major, _, _ = run_base(dtype, X, W, A, B, seg, lidx)
    if not name.startswith("capped"):
        assert np.array_equal(got, row_major)


def test_base_apply_integer_inputs_bit_exact():
    """X, W, B in {-1, 0, 1}, A with 8 entries of +-1 per column: every partial sum is
    an integer far inside fp32's exact range and the result is exact in fp16, so
    the device result equals the oracle's bit for bit."""
    rng = np.random.default_rng(11)
    n, h_in, h_out, rank, P = 24, 384, 392, 16, 5
    X, A, B, _ = workloads.integer_exact(rng, n, h_in, h_out, rank, P, "f16", nnz_per_col=8, y0_bound=0)
    Wf = np.zeros((h_in, h_out), np.float32)
    for c in range(h_out):
        rows = rng.choice(h_in, size=12, replace=False)
        Wf[rows, c] = rng.choice([-1.0, 1.0], size=12)
    W = workloads.to_bits(Wf, "f16")
    seg, lidx = [0, 5, 6, 14, 20], [4, 0, 4, 2]   # rows 20.. uncovered
    ref = oracle.sgmv_base_apply("f16", X, W, A, B, seg, lidx)
    for packed in (False, True):
        got, _, _ = run_base("f16", X, W, A, B, seg, lidx, packed=packed)
        assert np.array_equal(oracle.decode(got, "f16"), ref), packed


def test_base_apply_repeated_calls_and_shared_workspace():
    """Two calls in a row on one workspace (the second with fewer rows and other
    weights) each match the oracle: nothing stale leaks between calls."""
    import torch
    dtype = "bf16"
    X, W, A, B, seg, lidx = make_case(21, dtype, 48, 768, 640, 16, 8, "skewed")
    got1, prob1, dev1 = run_base(dtype, X, W, A, B, seg, lidx)
    assert_close(got1, oracle.sgmv_base_apply(dtype, X, W, A, B, seg, lidx), dtype, what="first")
    X2, W2, A2, B2, seg2, lidx2 = make_case(22, dtype, 9, 768, 640, 16, 12, "distinct")
    ws = dev1[5]
    seg2a, lidx2a = np.asarray(seg2, np.int32), np.asarray(lidx2, np.int32)
    prob2 = sg.make_problem(dtype, 9, 768, 640, 16, 12, len(lidx2a), 1)
    assert sg.sgmv_base_workspace_bytes(prob2) <= ws.numel()
    Xd, Wd, Ad, Bd = (to_device(a, dtype) for a in (X2, W2, A2, B2))
    Y = torch.full((9, 640), float("nan"), dtype=Xd.dtype, device="cuda")
    sg.sgmv_base_lora_apply(prob2, Xd, Wd, sg.pointer_table(Ad), sg.pointer_table(Bd), Y, i32(seg2a),
                            i32(lidx2a), ws)
    torch.cuda.synchronize()
    assert_close(to_bits(Y), oracle.sgmv_base_apply(dtype, X2, W2, A2, B2, seg2, lidx2), dtype, what="second")


# ------------------------------------------------------------ row-parallel shards

def run_partial(dtype, X, W, A_dev, lo, hi, B, seg, lidx, packed=False):
    """sgmv_base_lora_apply_partial on the K slice [lo, hi) of X, W and every A_k
    (A_dev: the whole stacked A on the device, [P, h_in, rank]); fp32 Yp as float64."""
    import torch
    n, h_in = X.shape
    P, _, rank = A_dev.shape
    h_out = W.shape[1]
    seg = np.asarray(seg, np.int32)
    lidx = np.asarray(lidx, np.int32)
    mx = int(np.diff(seg).max()) if len(seg) > 1 else 0
    prob = sg.make_problem(dtype, n, hi - lo, h_out, rank, P, len(lidx), mx)
    Xg = to_device(np.ascontiguousarray(X[:, lo:hi]), dtype)
    Wg = to_device(np.ascontiguousarray(W[lo:hi]), dtype)
    if packed:
        Wg = sg.pack_base_weight(Wg)
    # A_{k,g}: rows lo..hi-1 of A_k, addressed inside A_k's own storage
    A_tab = (A_dev.data_ptr() + (torch.arange(P, device="cuda", dtype=torch.int64) * h_in + lo) * rank * 2).contiguous()
    Bd = to_device(B, dtype)
    Yp = torch.full((n, h_out), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((sg.sgmv_base_workspace_bytes(prob),), 0x5A, dtype=torch.uint8, device="cuda")
    sg.sgmv_base_lora_apply_partial(prob, Xg, Wg, A_tab, sg.pointer_table(Bd), Yp, i32(seg if seg.size else [0]),
                                    i32(lidx if lidx.size else [0]), ws, w_packed=packed)
    torch.cuda.synchronize()
    return Yp.cpu().numpy().astype(np.float64)


SHARD_CASES = ["distinct_b32_h4096_r16", "skewed_b64_bf16_r64", "tail_uncovered_ragged", "no_segments_bf16"]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("name", SHARD_CASES)
def test_row_parallel_shards_sum_to_the_whole_product(name, packed):
    """Two H1 slices of the inputs (as two devices of a row-parallel layer hold
    them): each shard's fp32 partial equals the oracle on that slice, and the
    shards sum to the oracle's whole product (X @ W + per-row LoRA term)."""
    seed, dtype, n, h_in, h_out, rank, P, layout = CASES[name]
    X, W, A, B, seg, lidx = make_case(seed, dtype, n, h_in, h_out, rank, P, layout)
    A_dev = to_device(A, dtype)
    cut = (h_in // 2 + 7) // 8 * 8
    total = np.zeros((n, h_out))
    for lo, hi in ((0, cut), (cut, h_in)):
        Yp = run_partial(dtype, X, W, A_dev, lo, hi, B, seg, lidx, packed=packed)
        ref = oracle.sgmv_base_apply(dtype, np.ascontiguousarray(X[:, lo:hi]), np.ascontiguousarray(W[lo:hi]),
                                     np.ascontiguousarray(A[:, lo:hi, :]), B, seg, lidx)
        assert_close_f32(Yp, ref, what=f"{name} shard [{lo}, {hi})")
        total += Yp
    assert_close_f32(total, oracle.sgmv_base_apply(dtype, X, W, A, B, seg, lidx), what=f"{name} sum")


@pytest.mark.parametrize("packed", [False, True])
def test_one_shard_rounded_equals_the_rounded_call(packed):
    """With the whole H1 as its one slice, the shard's fp32 output rounded once
    (nearest even) is bit for bit the output of sgmv_base_lora_apply: the same
    partial planes, summed in the same order, before the one rounding."""
    import torch
    name = "skewed_b64_bf16_r64"
    seed, dtype, n, h_in, h_out, rank, P, layout = CASES[name]
    X, W, A, B, seg, lidx = make_case(seed, dtype, n, h_in, h_out, rank, P, layout)
    Yp = run_partial(dtype, X, W, to_device(A, dtype), 0, h_in, B, seg, lidx, packed=packed)
    rounded = to_bits(torch.from_numpy(Yp.astype(np.float32)).to(torch.bfloat16))
    got, _, _ = run_base(dtype, X, W, A, B, seg, lidx, packed=packed)
    assert np.array_equal(rounded, got)


def test_shards_of_integer_inputs_sum_exactly():
    """Integer-valued inputs: every shard is exact in fp32 and the shards sum to
    the oracle's whole product bit for bit."""
    rng = np.random.default_rng(12)
    n, h_in, h_out, rank, P = 24, 768, 392, 16, 5
    X, A, B, _ = workloads.integer_exact(rng, n, h_in, h_out, rank, P, "f16", nnz_per_col=8, y0_bound=0)
    Wf = np.zeros((h_in, h_out), np.float32)
    for c in range(h_out):
        rows = rng.choice(h_in, size=12, replace=False)
        Wf[rows, c] = rng.choice([-1.0, 1.0], size=12)
    W = workloads.to_bits(Wf, "f16")
    seg, lidx = [0, 5, 6, 14, 20], [4, 0, 4, 2]
    A_dev = to_device(A, "f16")
    total = np.zeros((n, h_out))
    for lo, hi in ((0, 256), (256, 512), (512, 768)):
        total += run_partial("f16", X, W, A_dev, lo, hi, B, seg, lidx)
    assert np.array_equal(total, oracle.sgmv_base_apply("f16", X, W, A, B, seg, lidx))
