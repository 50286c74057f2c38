"""Calls captured in a HIP graph and replayed give the eager result on every replay.

The one-launch decode kernel validates its exchanged partials with a tag made
from the dispatch packet id, which differs on every replay; the two-launch
vector route leaves its arrival counters zero after each call.  Each case
captures a reset of Y plus one call, replays it several times with eager calls
of the library in between (which consume their own dispatch ids and reuse the
workspace), and compares every replay bit for bit with the eager result.
"""
import numpy as np
import pytest

import segmented_gather_matvec_amd as sg
import workloads
from tests.gpu_cases import DeviceCall, to_bits, to_device

pytestmark = pytest.mark.gpu


def _case(name):
    if name == "decode":
        w, variant = workloads.decode_distinct(), sg.SGMV_VARIANT_AUTO
    elif name == "skewed_decode":
        w, variant = workloads.popularity("skewed", 64), sg.SGMV_VARIANT_AUTO
    elif name == "mfma":
        w, variant = workloads.mixed(64, seed=464, pairs=((512, 1376),), lo=16, hi=100)[0], sg.SGMV_VARIANT_MFMA
    else:
        w, variant = workloads.decode_distinct(), sg.SGMV_VARIANT_VECTOR
    if w.req_lora is not None:
        perm, seg, lidx, _ = sg.sgmv_build_segments(w.req_lora, w.num_loras)
        X, Y0 = w.X[perm], w.Y0[perm]
    else:
        seg, lidx, X, Y0 = w.seg_indptr, w.lora_idx, w.X, w.Y0
    return DeviceCall(w.dtype, X, w.A, w.B, Y0, seg, lidx, variant=variant)


@pytest.mark.parametrize("name", ["decode", "skewed_decode", "mfma", "vector"])
def test_graph_replays_match_eager(name):
    import torch
    call = _case(name)
    Y0d = to_device(call.Y0h, call.dtype)
    call.apply()
    torch.cuda.synchronize()
    eager = to_bits(call.Y).copy()

    side = DeviceCall(call.dtype, call.Xh, call.Ah, call.Bh, call.Y0h, call.seg, call.lidx,
                      variant=call.problem.variant)
    side.ws = call.ws  # eager calls between replays share the captured call's workspace

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            call.Y.copy_(Y0d)
            sg.sgmv_lora_apply(call.problem, call.X, call.A_ptrs, call.B_ptrs, call.Y, call.seg_d, call.lidx_d,
                               call.ws, stream=stream)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(call.Y), eager), f"{name}: replay {rep} differs from the eager call"
        side.reset_y()
        side.apply()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(side.Y), eager), f"{name}: eager call after replay {rep} differs"


@pytest.mark.parametrize("packed", [False, True])
def test_base_projection_graph_replays_match_eager(packed):
    """sgmv_base_lora_apply, or its packed-W twin (no counters, no tags: two
    launches over plain workspace planes), captured and replayed, with eager
    calls sharing the workspace in between."""
    import torch
    from tests.test_gpu_base import make_case
    from tests.gpu_cases import i32
    dtype = "bf16"
    X, W, A, B, seg, lidx = make_case(31, dtype, 24, 640, 392, 32, 6, "skewed")
    seg, lidx = np.asarray(seg, np.int32), np.asarray(lidx, np.int32)
    prob = sg.make_problem(dtype, 24, 640, 392, 32, 6, len(lidx), int(np.diff(seg).max()))
    Xd, Wd, Ad, Bd = (to_device(a, dtype) for a in (X, W, A, B))
    apply = sg.sgmv_base_lora_apply
    if packed:
        Wd, apply = sg.pack_base_weight(Wd), sg.sgmv_base_lora_apply_packed
        torch.cuda.synchronize()
    At, Bt = sg.pointer_table(Ad), sg.pointer_table(Bd)
    seg_d, lidx_d = i32(seg), i32(lidx)
    ws = sg.new_base_workspace(prob)
    Y = torch.zeros((24, 392), dtype=Xd.dtype, device="cuda")
    apply(prob, Xd, Wd, At, Bt, Y, seg_d, lidx_d, ws)
    torch.cuda.synchronize()
    eager = to_bits(Y).copy()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            Y.zero_()
            apply(prob, Xd, Wd, At, Bt, Y, seg_d, lidx_d, ws, stream=stream)
    torch.cuda.synchronize()
    Y2 = torch.zeros_like(Y)
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(Y), eager), f"replay {rep} differs from the eager call"
        Y2.zero_()
        apply(prob, Xd, Wd, At, Bt, Y2, seg_d, lidx_d, ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(Y2), eager), f"eager call after replay {rep} differs"
