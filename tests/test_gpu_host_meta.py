"""sgmv_lora_apply_host_meta against sgmv_lora_apply and the fp64 oracle,
through the C ABI.

The call takes the batch's segments and the LoRA pointer tables from host
memory (the segments the host builder forms for a batch; Punica README, page
"Punica：多 LoRA 模型统一服务框架", SGMV paragraph) and carries each segment's
bounds and A_k / B_k in the kernel's arguments.  Its result must equal
sgmv_lora_apply on device copies of the same arrays bit for bit, and the
oracle within the parity bound, on decode batches of every popularity
(throughput paragraph) with one-row and multi-row segments, empty segments and
rows no segment covers.  A call the one-launch route does not take (here: a
variant that names another route) is refused with SGMV_ERR_UNSUPPORTED and
nothing is written; the bounded wait's
give-up path works as in sgmv_lora_apply.
"""
import numpy as np
import pytest

import segmented_gather_matvec_amd as sg
import workloads
from tests.gpu_cases import DeviceCall, assert_close, to_bits

pytestmark = pytest.mark.gpu

DEFAULT_WAIT_US = 1000000


def _sorted_call(w):
    if w.req_lora is not None:
        perm, seg, lidx, _ = sg.sgmv_build_segments(w.req_lora, w.num_loras)
        return DeviceCall(w.dtype, w.X[perm], w.A, w.B, w.Y0[perm], seg, lidx)
    return DeviceCall(w.dtype, w.X, w.A, w.B, w.Y0, w.seg_indptr, w.lora_idx)


def _rand(seed, n, h_in, h_out, rank, P, seg, lidx, dtype="f16"):
    rng = np.random.default_rng(seed)
    X = workloads.to_bits(rng.standard_normal((n, h_in), dtype=np.float32), dtype)
    A = workloads.to_bits(rng.standard_normal((P, h_in, rank), dtype=np.float32) / np.sqrt(h_in), dtype)
    B = workloads.to_bits(rng.standard_normal((P, rank, h_out), dtype=np.float32) / np.sqrt(rank), dtype)
    Y0 = workloads.to_bits(rng.standard_normal((n, h_out), dtype=np.float32), dtype)
    return DeviceCall(dtype, X, A, B, Y0, seg, lidx)


CASES = {
    "distinct_b32_f16_r16": lambda: _sorted_call(workloads.decode_distinct()),
    "distinct_b64_bf16_r64": lambda: _sorted_call(workloads.decode_distinct(seed=3, n=64, h=1024, rank=64,
                                                                            dtype="bf16")),
    "distinct_b8_f16_r8": lambda: _sorted_call(workloads.decode_distinct(seed=4, n=8, h=512, rank=8)),
    "uniform_b32": lambda: _sorted_call(workloads.popularity("uniform", 32, seed=5)),
    "skewed_b32": lambda: _sorted_call(workloads.popularity("skewed", 32, seed=6)),
    "identical_b32": lambda: _sorted_call(workloads.popularity("identical", 32, seed=7)),
    "empty_segments_uncovered_rows": lambda: _rand(8, 20, 256, 128, 16, 5, [0, 0, 3, 3, 4, 9, 9, 15],
                                                   [4, 2, 2, 0, 1, 3, 2]),
    "unsorted_lora_ids_h11008_r32": lambda: _rand(9, 12, 11008, 4096, 32, 6, [0, 2, 3, 7, 12],
                                                  [5, 0, 3, 1]),
}


def _host_meta(call, Y=None):
    sg.sgmv_lora_apply_host_meta(call.problem, call.X, call.A_ptrs.cpu().numpy(), call.B_ptrs.cpu().numpy(),
                                 call.Y if Y is None else Y, call.seg, call.lidx, call.ws)


@pytest.mark.parametrize("case", sorted(CASES))
def test_host_meta_equals_device_metadata_call_and_oracle(case):
    import torch
    call = CASES[case]()
    assert sg.sgmv_query_plan(call.problem).route == sg.SGMV_ROUTE_DECODE, case
    ref = to_bits(call.apply()).copy()
    call.reset_y()
    _host_meta(call)
    torch.cuda.synchronize()
    got = to_bits(call.Y)
    assert np.array_equal(got, ref), f"{case}: host-metadata call differs from sgmv_lora_apply"
    assert_close(got, call.oracle_apply(), call.dtype, what=case)
    assert sg.sgmv_take_device_errors() == 0


def test_host_meta_twice_in_a_row_with_other_tables():
    """Two calls back to back on one workspace, the second with a different batch
    and LoRA pool: the arguments of each launch carry its own metadata."""
    import torch
    first = _sorted_call(workloads.popularity("skewed", 32, seed=11))
    second = _sorted_call(workloads.decode_distinct(seed=12, n=16, h=4096))
    second.ws = first.ws if first.ws.numel() >= second.ws.numel() else second.ws
    _host_meta(first)
    _host_meta(second)
    torch.cuda.synchronize()
    assert_close(to_bits(first.Y), first.oracle_apply(), "f16", what="first")
    assert_close(to_bits(second.Y), second.oracle_apply(), "f16", what="second")


def test_host_meta_refuses_batches_the_one_launch_route_does_not_take():
    """A batch of prefill segments with the matrix-core variant requested, and a
    decode batch with the vector variant requested: both are refused and Y is
    left alone."""
    import torch
    w = workloads.mixed(16, seed=413, pairs=((512, 1376),), lo=40, hi=100, n_decode=4)[0]
    long_call = DeviceCall(w.dtype, w.X, w.A, w.B, w.Y0, w.seg_indptr, w.lora_idx,
                           variant=sg.SGMV_VARIANT_MFMA)
    assert sg.sgmv_query_plan(long_call.problem).route == sg.SGMV_ROUTE_MFMA
    w2 = workloads.decode_distinct(seed=14, n=16, h=1024)
    forced = DeviceCall(w2.dtype, w2.X, w2.A, w2.B, w2.Y0, w2.seg_indptr, w2.lora_idx,
                        variant=sg.SGMV_VARIANT_VECTOR)
    for call in (long_call, forced):
        with pytest.raises(sg.SgmvError) as e:
            _host_meta(call)
        assert e.value.status == sg.SGMV_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(call.Y), call.Y0h)


def test_host_meta_wait_gives_up_under_the_test_hook_and_recovers():
    import torch
    call = CASES["distinct_b32_f16_r16"]()
    assert sg.sgmv_take_device_errors() == 0
    try:
        sg.sgmv_set_wait_limit(0)
        _host_meta(call)
        torch.cuda.synchronize()
        assert sg.sgmv_take_device_errors() == sg.SGMV_DEVICE_ERR_WAIT_TIMEOUT
        assert np.array_equal(to_bits(call.Y), call.Y0h)
    finally:
        sg.sgmv_set_wait_limit(DEFAULT_WAIT_US)
    call.reset_y()
    _host_meta(call)
    torch.cuda.synchronize()
    assert_close(to_bits(call.Y), call.oracle_apply(), "f16")
    assert sg.sgmv_take_device_errors() == 0
