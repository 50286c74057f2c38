"""Host-side tests of libsgmv's C ABI: no GPU needed, no kernel launched.

Covers: the shared library loads and exports every entry point declared in
include/sgmv.h; the host segment builder matches the oracle's stable-sort
builder bit for bit; argument checks return their status codes before any
HIP call.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle
import segmented_gather_matvec_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgmv.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sgmv_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    lib = sg.load_library()
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), f"{name} declared in sgmv.h but not exported"
    assert set(names) == set(sg.ENTRY_POINTS)


def test_problem_struct_layout_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct sgmv_problem \{(.*?)\} sgmv_problem_t;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [n for n, _ in sg.sgmv_problem_t._fields_]
    assert ctypes.sizeof(sg.sgmv_problem_t) == 4 * len(fields)
    assert f"SGMV_WS_COUNTER_BYTES ((size_t)1 << 20)" in src and sg.SGMV_WS_COUNTER_BYTES == 1 << 20


def test_plan_info_struct_layout_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct sgmv_plan_info \{(.*?)\} sgmv_plan_info_t;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == [n for n, _ in sg.sgmv_plan_info_t._fields_]
    assert ctypes.sizeof(sg.sgmv_plan_info_t) == 4 * len(fields)
    for name, val in [("SGMV_ROUTE_NONE", 0), ("SGMV_ROUTE_DECODE", 1), ("SGMV_ROUTE_MFMA", 2),
                      ("SGMV_ROUTE_VECTOR", 3)]:
        assert re.search(rf"{name} = {val}\b", src) and getattr(sg, name) == val


@pytest.mark.parametrize("kw,routes", [
    ({"num_segs": 0, "max_seg_len": 0}, {sg.SGMV_ROUTE_NONE}),
    ({"variant": sg.SGMV_VARIANT_VECTOR}, {sg.SGMV_ROUTE_VECTOR}),
    ({"variant": sg.SGMV_VARIANT_MFMA, "rank": 16}, {sg.SGMV_ROUTE_MFMA}),
    # the one-launch route needs the device's occupancy; without a GPU it is never taken
    ({}, {sg.SGMV_ROUTE_DECODE, sg.SGMV_ROUTE_VECTOR, sg.SGMV_ROUTE_MFMA}),
    ({"n_rows": 2048, "num_segs": 4, "max_seg_len": 1024, "rank": 64},
     {sg.SGMV_ROUTE_MFMA}),
])
def test_query_plan_routes(kw, routes):
    info = sg.sgmv_query_plan(good(**kw))
    assert info.route in routes
    if info.route == sg.SGMV_ROUTE_NONE:
        assert info.launches == 0 and info.grid == 0
    else:
        assert info.launches in {1: (1,), 2: (2, 3), 3: (2,)}[info.route]
        assert info.units >= 1 and info.splits >= 1 and info.grid >= 1
    with pytest.raises(sg.SgmvError):
        sg.sgmv_query_plan(good(rank=7))
    assert sg.load_library().sgmv_query_plan(ctypes.byref(good()), None) == sg.SGMV_ERR_INVALID_ARG


def test_projection_struct_layout_matches_header():
    src = open(HEADER).read()
    body = re.search(r"typedef struct sgmv_projection \{(.*?)\} sgmv_projection_t;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(\w+);", body)
    assert fields == [n for n, _ in sg.sgmv_projection_t._fields_]
    assert ctypes.sizeof(sg.sgmv_projection_t) == 8 * len(fields)
    assert re.search(r"#define SGMV_MAX_PROJECTIONS 4\b", src) and sg.SGMV_MAX_PROJECTIONS == 4
    m = re.search(r"#define SGMV_BASE_MAX_ROWS (\d+)\b", src)
    assert m and int(m.group(1)) == sg.SGMV_BASE_MAX_ROWS


def test_batched_apply_fails_fast_on_bad_arguments():
    """Host checks of sgmv_lora_apply_batched run before any HIP call."""
    lib = sg.load_library()
    p = good()
    fake = ctypes.c_void_p(0x10000)
    need = sg.sgmv_workspace_bytes(p)

    def call(projs, n, ws_bytes, X=fake, problem=p):
        arr = (sg.sgmv_projection_t * max(1, len(projs)))(*projs)
        return lib.sgmv_lora_apply_batched(ctypes.byref(problem), X, arr if projs else None, n, fake, fake, None,
                                           fake, ws_bytes, None)
    ok = sg.sgmv_projection_t(0x10000, 0x10000, 0x10000)
    assert call([], 0, need) == sg.SGMV_ERR_INVALID_ARG
    assert call([ok] * 5, 5, 5 * need) == sg.SGMV_ERR_INVALID_ARG            # more than SGMV_MAX_PROJECTIONS
    assert call([ok, sg.sgmv_projection_t(0x10000, None, 0x10000)], 2, 4 * need) == sg.SGMV_ERR_INVALID_ARG
    assert call([ok, sg.sgmv_projection_t(0x10000, 0x10000, 0x10002)], 2, 4 * need) == sg.SGMV_ERR_UNSUPPORTED
    # rank and scale tables must be 4-byte aligned
    assert call([sg.sgmv_projection_t(0x10000, 0x10000, 0x10000, 0x10002, None)], 1, need) == sg.SGMV_ERR_UNSUPPORTED
    assert call([sg.sgmv_projection_t(0x10000, 0x10000, 0x10000, None, 0x10001)], 1, need) == sg.SGMV_ERR_UNSUPPORTED
    assert call([ok, ok], 2, need) == sg.SGMV_ERR_WORKSPACE                    # one slice is not two
    assert call([ok, ok], 2, sg.batched_workspace_bytes(p, 2) - 1) == sg.SGMV_ERR_WORKSPACE
    assert call([ok], 1, need, X=None) == sg.SGMV_ERR_INVALID_ARG
    empty = good(num_segs=0, max_seg_len=0)
    assert call([ok, ok], 2, 0, problem=empty) == sg.SGMV_OK                  # nothing to do
    assert sg.batched_workspace_bytes(p, 1) == need
    assert sg.batched_workspace_bytes(p, 3) == 2 * ((need + 255) // 256 * 256) + need


def test_status_strings():
    for st in range(5):
        assert sg.sgmv_status_str(st).startswith("SGMV_")
    assert "UNKNOWN" in sg.sgmv_status_str(99)


# ------------------------------------------------------------------ builder

def test_builder_golden_examples():
    with open(os.path.join(GOLDEN, "builder_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        perm, seg, lidx, mx = sg.sgmv_build_segments(c["req_lora"], c["num_loras"])
        assert perm.tolist() == c["perm"]
        assert seg.tolist() == c["seg_indptr"]
        assert lidx.tolist() == c["lora_idx"]
        assert mx == c["max_seg_len"]


@pytest.mark.parametrize("seed", range(12))
def test_builder_matches_oracle_bit_exact(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 400))
    # dense pools take the counting sort, sparse pools the comparison sort
    P = int(rng.choice([1, 3, 50, 4096, 10_000_000]))
    ids = rng.integers(0, P, size=n)
    perm, seg, lidx, mx = sg.sgmv_build_segments(ids, P)
    operm, oseg, olidx, omx = oracle.build_segments(ids, P)
    assert perm.tolist() == operm and seg.tolist() == oseg and lidx.tolist() == olidx and mx == omx


@pytest.mark.parametrize("kind,n", [("identical", 32), ("uniform", 64), ("skewed", 64), ("skewed", 32)])
def test_builder_on_popularity_workloads(kind, n):
    import workloads
    w = workloads.popularity(kind, n)
    perm, seg, lidx, mx = sg.sgmv_build_segments(w.req_lora, w.num_loras)
    operm, oseg, olidx, omx = oracle.build_segments(w.req_lora, w.num_loras)
    assert perm.tolist() == operm and seg.tolist() == oseg and lidx.tolist() == olidx and mx == omx


@pytest.mark.parametrize("ids,P", [([0, 3], 3), ([-1], 3), ([0], 0)])
def test_builder_rejects_bad_ids(ids, P):
    with pytest.raises(sg.SgmvError) as e:
        sg.sgmv_build_segments(ids, P)
    assert e.value.status == sg.SGMV_ERR_INVALID_ARG


# ------------------------------------------------------------------ problem checks

def good(**kw):
    base = dict(dtype="f16", n_rows=32, h_in=4096, h_out=4096, rank=16, num_loras=32,
                num_segs=32, max_seg_len=1)
    base.update(kw)
    return sg.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, sg.SGMV_OK),
    ({"dtype": "bf16", "rank": 64}, sg.SGMV_OK),
    ({"rank": 8}, sg.SGMV_OK),
    ({"rank": 32}, sg.SGMV_OK),
    ({"rank": 12}, sg.SGMV_ERR_UNSUPPORTED),
    ({"rank": 128}, sg.SGMV_ERR_UNSUPPORTED),
    ({"dtype": 7}, sg.SGMV_ERR_UNSUPPORTED),
    ({"h_in": 4100}, sg.SGMV_ERR_UNSUPPORTED),
    ({"h_out": 12}, sg.SGMV_ERR_UNSUPPORTED),
    ({"h_in": 0}, sg.SGMV_ERR_INVALID_ARG),
    ({"n_rows": -1}, sg.SGMV_ERR_INVALID_ARG),
    ({"num_segs": -1}, sg.SGMV_ERR_INVALID_ARG),
    ({"max_seg_len": 33}, sg.SGMV_ERR_INVALID_ARG),
    ({"num_loras": 0}, sg.SGMV_ERR_INVALID_ARG),
    ({"variant": 9}, sg.SGMV_ERR_INVALID_ARG),
    ({"splits": -2}, sg.SGMV_ERR_INVALID_ARG),
    ({"num_segs": 0, "num_loras": 0, "max_seg_len": 0}, sg.SGMV_OK),
    ({"n_rows": 0, "num_segs": 0, "max_seg_len": 0}, sg.SGMV_OK),
])
def test_check_problem(kw, status):
    assert sg.sgmv_check_problem(good(**kw)) == status


def test_check_problem_null():
    assert sg.load_library().sgmv_check_problem(None) == sg.SGMV_ERR_INVALID_ARG


@pytest.mark.parametrize("seg,lidx,status", [
    ([0, 1, 2, 4], [0, 1, 2], sg.SGMV_OK),
    ([0, 0, 2, 4], [0, 1, 2], sg.SGMV_OK),           # empty segment
    ([1, 1, 2, 4], [0, 1, 2], sg.SGMV_ERR_INVALID_ARG),  # seg_indptr[0] != 0
    ([0, 2, 1, 4], [0, 1, 2], sg.SGMV_ERR_INVALID_ARG),  # decreasing
    ([0, 1, 2, 9], [0, 1, 2], sg.SGMV_ERR_INVALID_ARG),  # past n_rows
    ([0, 1, 2, 4], [0, 1, 5], sg.SGMV_ERR_INVALID_ARG),  # id out of range
    ([0, 1, 2, 4], [0, -1, 2], sg.SGMV_ERR_INVALID_ARG),
    ([0, 1, 4, 4], [0, 1, 2], sg.SGMV_ERR_INVALID_ARG),  # longer than max_seg_len
])
def test_check_segments(seg, lidx, status):
    p = sg.make_problem("f16", 8, 64, 64, 8, 4, 3, 2)
    assert sg.sgmv_check_segments(p, seg, lidx) == status


def test_workspace_bytes():
    p = good()
    nbytes = sg.sgmv_workspace_bytes(p)
    assert nbytes >= sg.SGMV_WS_COUNTER_BYTES + 32 * 16 * 4
    with pytest.raises(sg.SgmvError):
        sg.sgmv_workspace_bytes(good(rank=7))


@pytest.mark.parametrize("kw", [
    {"num_segs": 0, "max_seg_len": 0},
    {"n_rows": 0, "num_segs": 0, "max_seg_len": 0, "num_loras": 0},
    {"n_rows": 1, "num_segs": 1, "max_seg_len": 1, "num_loras": 1},
    {"n_rows": 5000, "num_segs": 3, "max_seg_len": 4000, "rank": 64, "h_in": 11008, "h_out": 8},
    {"n_rows": 4, "num_segs": 1, "max_seg_len": 4, "rank": 8, "h_in": 8, "h_out": 8},
    {"n_rows": 300, "num_segs": 300, "max_seg_len": 1, "rank": 32, "variant": 3},
])
@pytest.mark.parametrize("rank", [8, 16, 32, 64])
def test_workspace_bytes_degenerate_and_extreme_problems(kw, rank):
    """Planning every route must not fail (or trap) for empty, tiny or huge problems."""
    kw = dict(kw)
    kw.setdefault("rank", rank)
    if kw.get("variant") == 3 and kw["rank"] == 8:
        kw["rank"] = 16
    nbytes = sg.sgmv_workspace_bytes(good(**kw))
    assert nbytes >= sg.SGMV_WS_COUNTER_BYTES


def test_host_meta_entry_point_fails_fast_on_bad_host_metadata():
    """sgmv_lora_apply_host_meta checks its host arrays before any HIP call: null
    or misaligned arguments, metadata that breaks the segment preconditions, more
    segments than its kernel arguments carry, a null or misaligned A_k / B_k of a
    used LoRA, a missing or short workspace."""
    import numpy as np
    lib = sg.load_library()
    fake = ctypes.c_void_p(0x10000)    # aligned, never dereferenced on these paths
    odd = ctypes.c_void_p(0x10002)
    P = 4
    good_ptrs = [0x100000 * (k + 1) for k in range(P)]

    def run(p, seg, lidx, A=good_ptrs, B=good_ptrs, X=fake, Y=fake, ws=fake, nbytes=1 << 30):
        seg_a = None if seg is None else np.ascontiguousarray(seg, np.int32)
        lidx_a = np.ascontiguousarray(lidx if len(lidx) else [0], np.int32)
        A_a, B_a = np.ascontiguousarray(A, np.uint64), np.ascontiguousarray(B, np.uint64)
        return lib.sgmv_lora_apply_host_meta(ctypes.byref(p), X, A_a.ctypes.data, B_a.ctypes.data, Y,
                                             None if seg_a is None else seg_a.ctypes.data, lidx_a.ctypes.data,
                                             ws, nbytes, None)

    p = sg.make_problem("f16", 8, 256, 256, 16, P, 3, 4)
    seg, lidx = [0, 2, 6, 8], [3, 0, 1]
    assert run(p, seg, lidx, X=None) == sg.SGMV_ERR_INVALID_ARG
    assert run(p, seg, lidx, Y=None) == sg.SGMV_ERR_INVALID_ARG
    assert run(p, None, lidx) == sg.SGMV_ERR_INVALID_ARG
    assert run(p, seg, lidx, X=odd) == sg.SGMV_ERR_UNSUPPORTED
    assert run(p, seg, [3, 0, 4]) == sg.SGMV_ERR_INVALID_ARG          # LoRA id out of range
    assert run(p, [0, 2, 7, 8], lidx) == sg.SGMV_ERR_INVALID_ARG      # a segment longer than max_seg_len
    assert run(p, [0, 2, 6, 9], lidx) == sg.SGMV_ERR_INVALID_ARG      # past n_rows
    null_a = list(good_ptrs); null_a[0] = 0                            # LoRA 0 is used by segment 1
    assert run(p, seg, lidx, A=null_a) == sg.SGMV_ERR_INVALID_ARG
    odd_b = list(good_ptrs); odd_b[3] += 8                             # LoRA 3 is used by segment 0
    assert run(p, seg, lidx, B=odd_b) == sg.SGMV_ERR_UNSUPPORTED
    assert run(p, seg, lidx, ws=None, nbytes=0) == sg.SGMV_ERR_WORKSPACE
    assert run(p, seg, lidx, nbytes=sg.SGMV_WS_COUNTER_BYTES - 1) == sg.SGMV_ERR_WORKSPACE
    many = sg.SGMV_HOST_META_MAX_SEGS + 1
    pm = sg.make_problem("f16", many, 256, 256, 16, P, many, 1)
    assert run(pm, list(range(many + 1)), [0] * many) == sg.SGMV_ERR_UNSUPPORTED
    empty = sg.make_problem("f16", 8, 256, 256, 16, P, 0, 0)
    assert lib.sgmv_lora_apply_host_meta(ctypes.byref(empty), None, None, None, None, None, None, None, 0,
                                         None) == sg.SGMV_OK


def test_device_entry_points_fail_fast_on_bad_arguments():
    """Every status below is returned by host checks before any HIP call."""
    lib = sg.load_library()
    p = good()
    fake = ctypes.c_void_p(0x10000)    # aligned, never dereferenced on these paths
    odd = ctypes.c_void_p(0x10002)
    ws_need = sg.sgmv_workspace_bytes(p)
    # null pointers
    assert lib.sgmv_lora_apply(ctypes.byref(p), None, fake, fake, fake, fake, fake, fake, ws_need,
                               None) == sg.SGMV_ERR_INVALID_ARG
    assert lib.sgmv_shrink(ctypes.byref(p), fake, None, fake, fake, fake, fake, ws_need,
                           None) == sg.SGMV_ERR_INVALID_ARG
    assert lib.sgmv_expand(ctypes.byref(p), fake, fake, None, fake, fake, None) == sg.SGMV_ERR_INVALID_ARG
    # misaligned X / Y
    assert lib.sgmv_lora_apply(ctypes.byref(p), odd, fake, fake, fake, fake, fake, fake, ws_need,
                               None) == sg.SGMV_ERR_UNSUPPORTED
    assert lib.sgmv_expand(ctypes.byref(p), fake, fake, odd, fake, fake, None) == sg.SGMV_ERR_UNSUPPORTED
    # workspace missing / too small
    assert lib.sgmv_lora_apply(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, 0,
                               None) == sg.SGMV_ERR_WORKSPACE
    assert lib.sgmv_shrink(ctypes.byref(p), fake, fake, fake, fake, fake, fake, sg.SGMV_WS_COUNTER_BYTES,
                           None) == sg.SGMV_ERR_WORKSPACE
    # unsupported rank
    bad = good(rank=24)
    assert lib.sgmv_lora_apply(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake, ws_need,
                               None) == sg.SGMV_ERR_UNSUPPORTED
    # nothing to do: OK without touching any pointer
    empty = good(num_segs=0, max_seg_len=0)
    assert lib.sgmv_lora_apply(ctypes.byref(empty), None, None, None, None, None, None, None, 0,
                               None) == sg.SGMV_OK


def test_base_apply_fails_fast_on_bad_arguments():
    """sgmv_base_lora_apply: every status below comes from host checks before any HIP call."""
    lib = sg.load_library()
    p = good()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10002)
    need = sg.sgmv_base_workspace_bytes(p)
    call = lambda prob, X, W, Y, ws, nbytes, A=fake, B=fake: lib.sgmv_base_lora_apply(
        ctypes.byref(prob), X, W, A, B, Y, fake, fake, ws, nbytes, None)
    assert call(p, None, fake, fake, fake, need) == sg.SGMV_ERR_INVALID_ARG
    assert call(p, fake, None, fake, fake, need) == sg.SGMV_ERR_INVALID_ARG
    assert call(p, fake, fake, None, fake, need) == sg.SGMV_ERR_INVALID_ARG
    assert call(p, fake, fake, fake, fake, need, A=None) == sg.SGMV_ERR_INVALID_ARG
    assert call(p, fake, odd, fake, fake, need) == sg.SGMV_ERR_UNSUPPORTED
    assert call(p, fake, fake, fake, None, 0) == sg.SGMV_ERR_WORKSPACE
    assert call(p, fake, fake, fake, fake, need - 1) == sg.SGMV_ERR_WORKSPACE
    # more than SGMV_BASE_MAX_ROWS rows: a dense GEMM, not this entry point
    big = good(n_rows=sg.SGMV_BASE_MAX_ROWS + 1, num_segs=sg.SGMV_BASE_MAX_ROWS + 1)
    assert call(big, fake, fake, fake, fake, need) == sg.SGMV_ERR_UNSUPPORTED
    with pytest.raises(sg.SgmvError) as e:
        sg.sgmv_base_workspace_bytes(big)
    assert e.value.status == sg.SGMV_ERR_UNSUPPORTED
    # no rows: nothing to do
    none = good(n_rows=0, num_segs=0, max_seg_len=0)
    assert call(none, None, None, None, None, 0) == sg.SGMV_OK


def test_packed_base_entry_points_fail_fast():
    """sgmv_base_pack_weight / sgmv_base_lora_apply_packed: host checks before any HIP call."""
    lib = sg.load_library()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10001)
    need = sg.sgmv_base_packed_weight_bytes(520, 264)
    pack = lambda W, h_in, h_out, Wp, nbytes: lib.sgmv_base_pack_weight(W, h_in, h_out, Wp, nbytes, None)
    assert pack(None, 520, 264, fake, need) == sg.SGMV_ERR_INVALID_ARG
    assert pack(fake, 520, 264, None, need) == sg.SGMV_ERR_INVALID_ARG
    assert pack(fake, 0, 264, fake, need) == sg.SGMV_ERR_INVALID_ARG
    assert pack(fake, 520, -8, fake, need) == sg.SGMV_ERR_INVALID_ARG
    assert pack(fake, 520, 264, fake, need - 1) == sg.SGMV_ERR_WORKSPACE
    assert pack(odd, 520, 264, fake, need) == sg.SGMV_ERR_UNSUPPORTED
    assert pack(fake, 520, 264, ctypes.c_void_p(0x10008), need) == sg.SGMV_ERR_UNSUPPORTED
    out = ctypes.c_size_t(0)
    assert lib.sgmv_base_packed_weight_bytes(0, 8, ctypes.byref(out)) == sg.SGMV_ERR_INVALID_ARG
    p = good()
    ws = sg.sgmv_base_workspace_bytes(p)
    call = lambda prob, X, Wp, Y, nbytes: lib.sgmv_base_lora_apply_packed(
        ctypes.byref(prob), X, Wp, fake, fake, Y, fake, fake, fake, nbytes, None)
    assert call(p, fake, None, fake, ws) == sg.SGMV_ERR_INVALID_ARG
    assert call(p, fake, ctypes.c_void_p(0x10008), fake, ws) == sg.SGMV_ERR_UNSUPPORTED
    assert call(p, fake, fake, fake, ws - 1) == sg.SGMV_ERR_WORKSPACE
    assert call(good(n_rows=sg.SGMV_BASE_MAX_ROWS + 1, num_segs=sg.SGMV_BASE_MAX_ROWS + 1), fake, fake, fake,
                ws) == sg.SGMV_ERR_UNSUPPORTED


@pytest.mark.parametrize("h_in,h_out,blocks,ksteps", [(4096, 4096, 256, 128), (520, 264, 18, 20),
                                                      (8, 8, 2, 4), (11008, 4096, 256, 344)])
def test_packed_weight_size(h_in, h_out, blocks, ksteps):
    """1 KiB per (16-column block, 32-row k-step); blocks to an even count, k-steps to a multiple of 4."""
    assert sg.sgmv_base_packed_weight_bytes(h_in, h_out) == blocks * ksteps * 1024


@pytest.mark.parametrize("kw", [{}, {"h_out": 11008}, {"h_in": 13824, "h_out": 5120, "rank": 64},
                                {"n_rows": 1, "num_segs": 1}, {"n_rows": 64, "num_segs": 64},
                                {"n_rows": 128, "num_segs": 128}])
def test_base_workspace_covers_its_parts(kw):
    """The base workspace holds one fp32 partial plane of V and of Y per K split."""
    p = good(**kw)
    need = sg.sgmv_base_workspace_bytes(p)
    planes = need // (p.n_rows * (p.h_out + p.rank) * 4)
    assert planes >= 1
    assert need < (p.n_rows * p.h_out * 4) * (p.h_in // 128 + 1) + (64 << 20)


def test_wait_limit_and_device_error_entry_points_check_arguments():
    """The wait bound of the decode route and the device error query reject bad
    arguments on the host (no device touched)."""
    lib = sg.load_library()
    assert lib.sgmv_set_wait_limit(-1) == sg.SGMV_ERR_INVALID_ARG
    assert lib.sgmv_take_device_errors(None) == sg.SGMV_ERR_INVALID_ARG
    assert lib.sgmv_set_wait_limit(250000) == sg.SGMV_OK
    assert lib.sgmv_set_wait_limit(1000000) == sg.SGMV_OK
    with pytest.raises(sg.SgmvError) as e:
        sg.sgmv_set_wait_limit(-5)
    assert e.value.status == sg.SGMV_ERR_INVALID_ARG
    src = open(HEADER).read()
    assert re.search(r"#define SGMV_DEVICE_ERR_WAIT_TIMEOUT 1u", src)
    assert sg.SGMV_DEVICE_ERR_WAIT_TIMEOUT == 1
