"""GPU parity of per-LoRA ranks and scales (sgmv_lora_apply_batched), through the C ABI.

The Punica discussion page ("Punica: Serving multiple LoRA finetuned LLM as
one", the question on LoRAs with different ranks) serves mixed ranks as if
every LoRA were padded to one rank.  Here each LoRA keeps its own rank r_k and
compact storage (A_k [h_in, r_k], B_k [r_k, h_out], one allocation per LoRA,
null pointers for rank 0), and the result must equal the fp64 oracle with the
same ranks and scales, within |gpu - ref| <= 1e-3 + 1e-2*|ref|, on every route.
"""
import numpy as np
import pytest

import oracle
import segmented_gather_matvec_amd as sg
import workloads
from tests.gpu_cases import assert_close, i32, to_bits, to_device

pytestmark = pytest.mark.gpu


class HetCall:
    """One batch with per-LoRA ranks (compact storage) and scales on the device."""

    def __init__(self, seed, dtype, n, h_in, h_out, R, P, seg, lidx, rank_choices, variant=sg.SGMV_VARIANT_AUTO,
                 splits=0, with_scales=True, rows_total=None):
        import torch
        rng = np.random.default_rng(seed)
        self.dtype, self.seg, self.lidx = dtype, np.asarray(seg, np.int32), np.asarray(lidx, np.int32)
        self.ranks = rng.choice(rank_choices, P).astype(np.int32)
        self.scales = (rng.uniform(0.25, 2.0, P) * rng.choice([-1, 1], P)).astype(np.float32) if with_scales else None
        rows = rows_total or n
        self.Xh = workloads.to_bits(rng.standard_normal((rows, h_in)).astype(np.float32), dtype)
        self.Y0h = workloads.to_bits(rng.standard_normal((rows, h_out)).astype(np.float32), dtype)
        self.Ah, self.Bh, self.A, self.B = [], [], [], []
        for k in range(P):
            r = int(self.ranks[k])
            a = workloads.to_bits((rng.standard_normal((h_in, r)) * h_in ** -0.5).astype(np.float32), dtype)
            b = workloads.to_bits((rng.standard_normal((r, h_out)) * max(r, 1) ** -0.5).astype(np.float32), dtype)
            self.Ah.append(a)
            self.Bh.append(b)
            self.A.append(to_device(a, dtype) if r else None)
            self.B.append(to_device(b, dtype) if r else None)
        lens = np.diff(self.seg)
        self.problem = sg.make_problem(dtype, rows, h_in, h_out, R, P, len(self.lidx), int(lens.max()), variant,
                                       splits)
        self.X = to_device(self.Xh, dtype)
        self.Y = to_device(self.Y0h, dtype)
        self.A_ptrs, self.B_ptrs = sg.pointer_list(self.A), sg.pointer_list(self.B)
        self.ranks_d = i32(self.ranks)
        self.scales_d = None if self.scales is None else torch.from_numpy(self.scales).cuda()
        self.seg_d, self.lidx_d = i32(self.seg), i32(self.lidx)
        self.R = R

    def projection(self):
        return (self.A_ptrs, self.B_ptrs, self.Y, self.ranks_d, self.scales_d)

    def oracle(self, rows=None):
        """fp64 reference on sorted rows `rows` of X / Y0 (default: the first n)."""
        rows = np.arange(self.seg[-1]) if rows is None else rows
        return oracle.sgmv_apply(self.dtype, self.Xh[rows], self.Ah, self.Bh, self.seg, self.lidx,
                                 self.Y0h[rows], scales=self.scales, rank=self.R)


def distinct(n, P):
    return list(range(n + 1)), list(np.random.default_rng(n + P).permutation(P)[:n])


CASES = {
    # name: (seed, dtype, n, h_in, h_out, R, P, segments, rank choices, variant, splits)
    "decode_r16_b32": (1, "f16", 32, 4096, 4096, 16, 32, distinct(32, 32), [0, 8, 16], 0, 0),
    "decode_r64_b32": (2, "bf16", 32, 4096, 4096, 64, 48, distinct(32, 48), [0, 8, 16, 24, 40, 64], 0, 0),
    "decode_r32_pool96": (3, "f16", 24, 2048, 1024, 32, 96, distinct(24, 96), [0, 8, 16, 32], 0, 0),
    "decode_rb4": (4, "f16", 32, 1024, 2048, 16, 8, ([0, 4, 8, 12, 16, 20, 24, 28, 32], list(range(8))),
                   [0, 8, 16], sg.SGMV_VARIANT_FUSED, 64),
    "mfma_r64": (5, "bf16", 300, 1024, 1376, 64, 6, ([0, 120, 121, 250, 251, 300], [3, 0, 5, 1, 2]),
                 [0, 16, 32, 48, 64], sg.SGMV_VARIANT_MFMA, 0),
    # short row tiles and 20 H1 planes: summed by the lead workgroups of the expand launch
    "mfma_r64_lead": (11, "bf16", 200, 5120, 1024, 64, 24, (list(range(0, 201, 10)), [(7 * i) % 24 for i in range(20)]),
                      [0, 16, 32, 64], sg.SGMV_VARIANT_MFMA, 0),
    "mfma_r16": (8, "f16", 160, 2048, 512, 16, 4, ([0, 70, 71, 160], [1, 2, 3]), [0, 8, 16],
                 sg.SGMV_VARIANT_MFMA, 0),
    "vector_r32": (7, "f16", 40, 1024, 1000, 32, 10, ([0, 5, 6, 20, 21, 40], [9, 0, 4, 7, 2]),
                   [0, 8, 24, 32], sg.SGMV_VARIANT_VECTOR, 0),
    "vector_r8": (10, "bf16", 16, 512, 256, 8, 4, ([0, 3, 16], [2, 1]), [0, 8], sg.SGMV_VARIANT_VECTOR, 0),
}


def _run(call, row_idx=None, extra=()):
    import torch
    nproj = 1 + len(extra)
    ws = torch.zeros(sg.batched_workspace_bytes(call.problem, nproj), dtype=torch.uint8, device="cuda")
    sg.sgmv_lora_apply_batched(call.problem, call.X, [call.projection()] + [c.projection() for c in extra],
                               call.seg_d, call.lidx_d, ws, row_idx=row_idx)
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", sorted(CASES))
def test_ranks_and_scales_match_oracle(case):
    seed, dtype, n, h_in, h_out, R, P, (seg, lidx), choices, variant, splits = CASES[case]
    call = HetCall(seed, dtype, n, h_in, h_out, R, P, seg, lidx, choices, variant, splits)
    assert (call.ranks[call.lidx] == 0).any() and (call.ranks[call.lidx] > 0).any(), "case covers rank 0 and > 0"
    _run(call)
    assert_close(to_bits(call.Y), call.oracle(), dtype, what=case)


@pytest.mark.parametrize("case", ["decode_r16_b32", "mfma_r64", "vector_r32"])
def test_ranks_without_scales(case):
    seed, dtype, n, h_in, h_out, R, P, (seg, lidx), choices, variant, splits = CASES[case]
    call = HetCall(seed + 100, dtype, n, h_in, h_out, R, P, seg, lidx, choices, variant, splits, with_scales=False)
    _run(call)
    assert_close(to_bits(call.Y), call.oracle(), dtype, what=case)


@pytest.mark.parametrize("case", ["decode_r64_b32", "mfma_r16", "mfma_r64_lead", "vector_r32"])
def test_ranks_scales_with_row_map(case):
    """Request-order rows (row map) together with ranks and scales."""
    import torch
    seed, dtype, n, h_in, h_out, R, P, (seg, lidx), choices, variant, splits = CASES[case]
    total = n + 5
    call = HetCall(seed + 200, dtype, n, h_in, h_out, R, P, seg, lidx, choices, variant, splits, rows_total=total)
    perm = np.random.default_rng(seed).permutation(total)[:n].astype(np.int32)
    _run(call, row_idx=torch.from_numpy(perm).cuda())
    ref = oracle.decode(call.Y0h, dtype)
    ref[perm] = call.oracle(rows=perm)
    assert_close(to_bits(call.Y), ref, dtype, what=case)


@pytest.mark.parametrize("case", ["decode_r16_b32", "mfma_r64", "mfma_r64_lead"])
def test_batched_projections_with_their_own_ranks(case):
    """Two projections in one call, each with its own rank table and scales."""
    seed, dtype, n, h_in, h_out, R, P, (seg, lidx), choices, variant, splits = CASES[case]
    c0 = HetCall(seed + 300, dtype, n, h_in, h_out, R, P, seg, lidx, choices, variant, splits)
    c1 = HetCall(seed + 301, dtype, n, h_in, h_out, R, P, seg, lidx, choices, variant, splits)
    c1.X, c1.Xh = c0.X, c0.Xh  # projections share the input
    _run(c0, extra=(c1,))
    assert_close(to_bits(c0.Y), c0.oracle(), dtype, what="projection 0")
    assert_close(to_bits(c1.Y), c1.oracle(), dtype, what="projection 1")


@pytest.mark.parametrize("variant", [sg.SGMV_VARIANT_AUTO, sg.SGMV_VARIANT_MFMA, sg.SGMV_VARIANT_VECTOR])
def test_full_rank_table_and_unit_scales_equal_the_plain_call(variant):
    """Every r_k = R and every scale 1 through the extended path gives the same
    bits as the plain call."""
    import torch
    w = workloads.mixed(16, seed=416, pairs=((512, 1376),), lo=16, hi=100)[0] if variant == sg.SGMV_VARIANT_MFMA \
        else workloads.decode_distinct()
    from tests.gpu_cases import DeviceCall
    call = DeviceCall(w.dtype, w.X, w.A, w.B, w.Y0, w.seg_indptr, w.lora_idx, variant=variant)
    call.apply()
    torch.cuda.synchronize()
    plain = to_bits(call.Y).copy()
    call.reset_y()
    P = w.A.shape[0]
    ranks = i32(np.full(P, w.A.shape[2]))
    ones = torch.ones(P, dtype=torch.float32, device="cuda")
    ws = sg.new_workspace(call.problem)
    sg.sgmv_lora_apply_batched(call.problem, call.X, [(call.A_ptrs, call.B_ptrs, call.Y, ranks, ones)],
                               call.seg_d, call.lidx_d, ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(call.Y), plain)
