"""sgmv_lora_apply_noalloc, the entry point for callers that cannot allocate,
against sgmv_lora_apply (the same kernels on a caller-owned workspace), through
the C ABI.  Two calls in a row on each route, the second on a smaller input,
must give bit-identical results to the workspace entry point, and both must
match the fp64 oracle within the parity bound; a problem whose workspace
exceeds the static scratch is rejected with SGMV_ERR_WORKSPACE.  Workloads:
the Punica README's decode batch (page "Punica：多 LoRA 模型统一服务框架",
throughput paragraph) and mixed prefill + decode segments."""
import ctypes

import numpy as np
import pytest

import segmented_gather_matvec_amd as sg
import workloads
from tests.gpu_cases import DeviceCall, assert_close, to_bits

pytestmark = pytest.mark.gpu


def _pair(w, variant):
    if w.req_lora is not None:
        perm, seg, lidx, _ = sg.sgmv_build_segments(w.req_lora, w.num_loras)
        X, Y0 = w.X[perm], w.Y0[perm]
    else:
        seg, lidx, X, Y0 = w.seg_indptr, w.lora_idx, w.X, w.Y0
    return DeviceCall(w.dtype, X, w.A, w.B, Y0, seg, lidx, variant=variant)


CASES = {
    # route: (larger input, smaller input)
    "decode": (lambda: workloads.decode_distinct(seed=21, n=64),
               lambda: workloads.decode_distinct(seed=22, n=8, h=1024), sg.SGMV_VARIANT_AUTO),
    "mfma": (lambda: workloads.mixed(64, seed=423, pairs=((1376, 512),), lo=16, hi=100)[0],
             lambda: workloads.mixed(16, seed=424, pairs=((512, 256),), lo=17, hi=40, n_prefill=2, n_decode=3)[0],
             sg.SGMV_VARIANT_MFMA),
    "vector": (lambda: workloads.popularity("skewed", 64, seed=25),
               lambda: workloads.popularity("uniform", 32, seed=26, h=512), sg.SGMV_VARIANT_VECTOR),
}


@pytest.mark.parametrize("route", sorted(CASES))
def test_noalloc_matches_workspace_entry_point(route):
    import torch
    big, small, variant = CASES[route]
    expect = {"decode": sg.SGMV_ROUTE_DECODE, "mfma": sg.SGMV_ROUTE_MFMA, "vector": sg.SGMV_ROUTE_VECTOR}[route]
    for make in (big, small):
        call = _pair(make(), variant)
        assert sg.sgmv_query_plan(call.problem).route == expect
        ref = to_bits(call.apply()).copy()            # caller-owned workspace
        call.reset_y()
        sg.sgmv_lora_apply_noalloc(call.problem, call.X, call.A_ptrs, call.B_ptrs, call.Y, call.seg_d,
                                   call.lidx_d)
        torch.cuda.synchronize()
        got = to_bits(call.Y)
        assert np.array_equal(got, ref), f"{route}: no-alloc result differs from the workspace entry point"
        assert_close(got, call.oracle_apply(), call.dtype, what=route)
    assert sg.sgmv_take_device_errors() == 0


def test_noalloc_rejects_problems_beyond_its_scratch():
    lib = sg.load_library()
    p = sg.make_problem("bf16", 200000, 4096, 4096, 64, 16, 16, 20000)
    assert sg.sgmv_workspace_bytes(p) > sg.SGMV_NOALLOC_MAX_WORKSPACE
    fake = ctypes.c_void_p(0x10000)
    assert lib.sgmv_lora_apply_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake,
                                       None) == sg.SGMV_ERR_WORKSPACE


@pytest.mark.parametrize("route", sorted(CASES))
def test_noalloc_call_captured_in_a_graph_replays_exactly(route):
    """The callers this entry point is for capture it in a HIP graph.  A reset of
    Y plus one no-alloc call is captured and replayed several times, with eager
    no-alloc calls in between that use the same static scratch; every replay and
    every eager call must equal the workspace entry point bit for bit."""
    import torch
    from tests.gpu_cases import to_device
    _, small, variant = CASES[route]
    call = _pair(small(), variant)
    ref = to_bits(call.apply()).copy()
    side = _pair(small(), variant)
    Y0d = to_device(call.Y0h, call.dtype)
    call.reset_y()
    sg.sgmv_lora_apply_noalloc(call.problem, call.X, call.A_ptrs, call.B_ptrs, call.Y, call.seg_d, call.lidx_d)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(call.Y), ref)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            call.Y.copy_(Y0d)
            sg.sgmv_lora_apply_noalloc(call.problem, call.X, call.A_ptrs, call.B_ptrs, call.Y, call.seg_d,
                                       call.lidx_d, stream=stream)
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(call.Y), ref), f"{route}: replay {rep} differs"
        side.reset_y()
        sg.sgmv_lora_apply_noalloc(side.problem, side.X, side.A_ptrs, side.B_ptrs, side.Y, side.seg_d,
                                   side.lidx_d)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(side.Y), ref), f"{route}: eager no-alloc call after replay {rep} differs"
    assert sg.sgmv_take_device_errors() == 0
