"""GPU tests of the decode route's safety contract, through the C ABI.

* The wait of a decode-route workgroup for its unit's other partial sums is
  bounded; the host's test hook (a wait limit of 0) makes every wait give up
  at once, so the give-up path runs with every kernel exiting normally: Y is
  left untouched and the device error word reports the timeout.  A later call
  with the default limit is correct again.
* The decode route's tagged slots live in a workspace area that no other
  route writes: calls of the matrix-core and two-launch routes on the same
  workspace (their fp32 partials could otherwise pose as tagged words), and a
  workspace holding arbitrary bytes outside its counter area, leave the
  decode route's result equal to the oracle's.
Workload: the decode batch of the Punica README's throughput paragraph
(page "Punica：多 LoRA 模型统一服务框架"), Distinct popularity, H = 4096, r = 16.
"""
import numpy as np
import pytest

import oracle
import segmented_gather_matvec_amd as sg
import workloads
from tests.gpu_cases import DeviceCall, assert_close, to_bits

pytestmark = pytest.mark.gpu

DEFAULT_WAIT_US = 1000000


def decode_call(seed=2, n=32, h=4096):
    w = workloads.decode_distinct(seed=seed, n=n, h=h)
    call = DeviceCall(w.dtype, w.X, w.A, w.B, w.Y0, w.seg_indptr, w.lora_idx)
    assert sg.sgmv_query_plan(call.problem).route == sg.SGMV_ROUTE_DECODE
    return call


def test_decode_wait_gives_up_under_the_test_hook_and_recovers():
    import torch
    call = decode_call()
    assert sg.sgmv_take_device_errors() == 0
    try:
        sg.sgmv_set_wait_limit(0)
        call.apply()
        torch.cuda.synchronize()
        assert sg.sgmv_take_device_errors() == sg.SGMV_DEVICE_ERR_WAIT_TIMEOUT
        # every workgroup gave up before its expand: Y is untouched
        assert np.array_equal(to_bits(call.Y), call.Y0h)
        assert sg.sgmv_take_device_errors() == 0  # the query clears the word
    finally:
        sg.sgmv_set_wait_limit(DEFAULT_WAIT_US)
    call.reset_y()
    assert_close(to_bits(call.apply()), call.oracle_apply(), "f16")
    assert sg.sgmv_take_device_errors() == 0


def test_multi_pass_decode_gives_up_in_every_pass():
    """A batch whose units do not all fit on the device at once runs in passes;
    every pass takes the give-up path."""
    import torch
    call = decode_call(seed=9, n=512)   # more units than the device holds at once: passes
    info = sg.sgmv_query_plan(call.problem)
    assert info.route == sg.SGMV_ROUTE_DECODE and info.launches > 1, info.as_dict()
    try:
        sg.sgmv_set_wait_limit(0)
        call.apply()
        torch.cuda.synchronize()
        assert sg.sgmv_take_device_errors() == sg.SGMV_DEVICE_ERR_WAIT_TIMEOUT
        assert np.array_equal(to_bits(call.Y), call.Y0h)
    finally:
        sg.sgmv_set_wait_limit(DEFAULT_WAIT_US)
    call.reset_y()
    rows = np.r_[0:4, 250:266, 508:512]
    mask = np.zeros(512, np.uint8)
    mask[rows] = 1
    assert_close(to_bits(call.apply()), call.oracle_apply(row_mask=mask), "f16", rows=rows)
    assert sg.sgmv_take_device_errors() == 0


@pytest.mark.parametrize("seg,lidx", [([0, 100, 256], [2, 0]),
                                      (list(range(0, 257, 16)), [i % 3 for i in range(16)])],
                         ids=["full_tiles_flags", "short_tiles_tagged_words"])
def test_matrix_core_lead_wait_gives_up_under_the_test_hook_and_recovers(seg, lidx):
    """The first workgroups of the expand launch sum the shrink's partial
    planes: for full row tiles (12 planes) they flag each row block, for short
    tiles (32 planes) they publish V as tagged words; the others wait under the
    same bound as the decode route.  Under the test hook every such wait gives
    up: Y is untouched and the error word reports it."""
    import torch
    rng = np.random.default_rng(4242)
    X, A, B, Y0 = workloads.integer_exact(rng, 256, 8192, 256, 64, 3, "bf16", 2, 64)
    call = DeviceCall("bf16", X, A, B, Y0, seg, lidx, variant=sg.SGMV_VARIANT_MFMA)
    info = sg.sgmv_query_plan(call.problem)
    assert info.route == sg.SGMV_ROUTE_MFMA and info.splits > 8 and info.launches == 2, info.as_dict()
    assert sg.sgmv_take_device_errors() == 0
    try:
        sg.sgmv_set_wait_limit(0)
        call.apply()
        torch.cuda.synchronize()
        assert sg.sgmv_take_device_errors() == sg.SGMV_DEVICE_ERR_WAIT_TIMEOUT
        assert np.array_equal(to_bits(call.Y), call.Y0h)
    finally:
        sg.sgmv_set_wait_limit(DEFAULT_WAIT_US)
    call.reset_y()
    assert np.array_equal(oracle.decode(to_bits(call.apply()), "bf16"), call.oracle_apply())
    assert sg.sgmv_take_device_errors() == 0


def test_matrix_core_lead_calls_on_two_streams():
    """Two matrix-core calls whose expand launches carry lead workgroups (one
    with short tiles and tagged V words, one with full tiles and flags) run at
    the same time on two streams, each with its own workspace.  Lead workgroups
    wait for nothing and every wait is for lead workgroups of its own launch,
    dispatched ahead of it, so the calls need no device to themselves: both
    give the oracle's bits (integer-exact inputs) and no wait gives up."""
    import torch
    rng = np.random.default_rng(777)
    calls = []
    for seg, lidx in ((list(range(0, 257, 16)), [i % 3 for i in range(16)]), ([0, 100, 256], [2, 0])):
        X, A, B, Y0 = workloads.integer_exact(rng, 256, 8192, 2048, 64, 3, "bf16", 2, 64)
        c = DeviceCall("bf16", X, A, B, Y0, seg, lidx, variant=sg.SGMV_VARIANT_MFMA)
        info = sg.sgmv_query_plan(c.problem)
        assert info.route == sg.SGMV_ROUTE_MFMA and info.splits > 1, info.as_dict()
        calls.append(c)
    refs = [c.oracle_apply() for c in calls]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    assert sg.sgmv_take_device_errors() == 0
    for _ in range(4):
        for c in calls:
            c.reset_y()
        torch.cuda.synchronize()
        for c, st in zip(calls, streams):
            sg.sgmv_lora_apply(c.problem, c.X, c.A_ptrs, c.B_ptrs, c.Y, c.seg_d, c.lidx_d, c.ws, stream=st)
        torch.cuda.synchronize()
        for c, ref in zip(calls, refs):
            assert np.array_equal(oracle.decode(to_bits(c.Y), "bf16"), ref)
    assert sg.sgmv_take_device_errors() == 0


def test_decode_slots_untouched_by_other_routes():
    """One workspace serves the matrix-core route, the two-launch route and the
    decode route in turn; the decode route's result is the oracle's."""
    import torch
    call = decode_call(seed=11)
    mfma = DeviceCall("f16", call.Xh, call.Ah, call.Bh, call.Y0h, call.seg, call.lidx,
                      variant=sg.SGMV_VARIANT_MFMA)
    vec = DeviceCall("f16", call.Xh, call.Ah, call.Bh, call.Y0h, call.seg, call.lidx,
                     variant=sg.SGMV_VARIANT_VECTOR)
    nbytes = max(sg.sgmv_workspace_bytes(c.problem) for c in (call, mfma, vec))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ref = call.oracle_apply()
    for c in (mfma, vec, call, mfma, call):
        c.ws = ws
        c.reset_y()
        assert_close(to_bits(c.apply()), ref, "f16")
    assert sg.sgmv_take_device_errors() == 0


def test_decode_route_accepts_any_bytes_outside_the_counter_area():
    import torch
    call = decode_call(seed=12)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    n = call.ws.numel()
    call.ws[sg.SGMV_WS_COUNTER_BYTES:] = torch.randint(0, 256, (n - sg.SGMV_WS_COUNTER_BYTES,), generator=g,
                                                       device="cuda", dtype=torch.int32).to(torch.uint8)
    ref = call.oracle_apply()
    for _ in range(2):
        call.reset_y()
        assert_close(to_bits(call.apply()), ref, "f16")
    assert sg.sgmv_take_device_errors() == 0
