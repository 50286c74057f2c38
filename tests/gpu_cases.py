"""Helpers shared by the GPU parity tests: move a Workload to the device, run
libsgmv through its C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import oracle
import segmented_gather_matvec_amd as sg

# Per-element acceptance bound against the unrounded fp64 oracle.
ATOL, RTOL = 1e-3, 1e-2


def torch_dtype(dtype: str):
    import torch
    return torch.float16 if dtype == "f16" else torch.bfloat16


def to_device(bits: np.ndarray, dtype: str):
    """uint16 bit patterns -> device tensor of the matching 16-bit float type."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch_dtype(dtype)).cuda()


def to_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(a):
    import torch
    return torch.tensor(np.asarray(a, dtype=np.int32), dtype=torch.int32, device="cuda")


class DeviceCall:
    """Device copies of one call's inputs plus its problem description."""

    def __init__(self, dtype, X, A, B, Y0, seg_indptr, lora_idx, variant=sg.SGMV_VARIANT_AUTO,
                 splits=0, max_seg_len=None):
        self.dtype = dtype
        self.Xh, self.Ah, self.Bh, self.Y0h = X, A, B, Y0
        self.seg = np.asarray(seg_indptr, np.int32)
        self.lidx = np.asarray(lora_idx, np.int32)
        n, h_in = X.shape
        P, _, rank = A.shape
        h_out = B.shape[2]
        lens = np.diff(self.seg) if len(self.seg) > 1 else np.zeros(0, np.int32)
        mx = int(lens.max()) if lens.size else 0
        self.problem = sg.make_problem(dtype, n, h_in, h_out, rank, P, len(self.lidx),
                                       mx if max_seg_len is None else max_seg_len, variant, splits)
        self.X = to_device(X, dtype)
        self.A = to_device(A, dtype)
        self.B = to_device(B, dtype)
        self.Y = to_device(Y0, dtype)
        self.A_ptrs = sg.pointer_table(self.A)
        self.B_ptrs = sg.pointer_table(self.B)
        self.seg_d = i32(self.seg if self.seg.size else [0])
        self.lidx_d = i32(self.lidx if self.lidx.size else [0])
        try:
            self.ws = sg.new_workspace(self.problem)
        except sg.SgmvError:
            # an unsupported problem: the call itself must report the status
            import torch
            self.ws = torch.zeros(sg.SGMV_WS_COUNTER_BYTES, dtype=torch.uint8, device="cuda")

    def reset_y(self):
        self.Y.copy_(to_device(self.Y0h, self.dtype))

    def apply(self):
        sg.sgmv_lora_apply(self.problem, self.X, self.A_ptrs, self.B_ptrs, self.Y, self.seg_d,
                           self.lidx_d, self.ws)
        return self.Y

    def shrink(self, fill=float("nan")):
        import torch
        V = torch.full((self.Xh.shape[0], self.Ah.shape[2]), fill, dtype=torch.float32, device="cuda")
        sg.sgmv_shrink(self.problem, self.X, self.A_ptrs, V, self.seg_d, self.lidx_d, self.ws)
        return V

    def expand(self, V):
        sg.sgmv_expand(self.problem, V, self.B_ptrs, self.Y, self.seg_d, self.lidx_d)
        return self.Y

    def oracle_apply(self, row_mask=None):
        return oracle.sgmv_apply(self.dtype, self.Xh, self.Ah, self.Bh, self.seg, self.lidx,
                                 self.Y0h, row_mask=row_mask)

    def counters_clear(self) -> bool:
        import torch
        return bool((self.ws[: sg.SGMV_WS_COUNTER_BYTES] == 0).all().item())


def assert_close(gpu_bits: np.ndarray, ref: np.ndarray, dtype: str, rows=None, what="Y"):
    got = oracle.decode(gpu_bits, dtype)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of bound; first at "
                             f"{tuple(idx)}: got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}; "
                             f"max err/bound {float((err / bound).max()):.3f}")
    return float((err / bound).max())


def assert_close_f32(got: np.ndarray, ref: np.ndarray, what="V"):
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    assert (err <= bound).all(), f"{what}: max err/bound {float((err / bound).max()):.3f}"
