"""Python binding of libsgmv (SGMV LoRA kernels for MI355X / gfx950).

A thin ctypes layer over the C ABI in ``include/sgmv.h``: each function here
has the name of the C entry point it calls and only marshals arguments
(torch tensors -> device pointers, the current HIP stream, status codes ->
exceptions).  Every step of the computation runs in the library's HIP
kernels; there is no fallback path.  PyTorch is used for device memory and
streams only.

What is computed is the LoRA term of the Punica README (page "Punica：多 LoRA
模型统一服务框架", LoRA and multi-LoRA paragraphs): for rows grouped into
segments that share a LoRA pair (A_k [H1, r], B_k [r, H2]),
``Y[i] += (X[i] @ A_k) @ B_k`` on top of the base output already in Y.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsgmv.so")

SGMV_OK, SGMV_ERR_INVALID_ARG, SGMV_ERR_UNSUPPORTED, SGMV_ERR_WORKSPACE, SGMV_ERR_HIP = range(5)
SGMV_F16, SGMV_BF16 = 0, 1
SGMV_VARIANT_AUTO, SGMV_VARIANT_VECTOR, SGMV_VARIANT_FUSED, SGMV_VARIANT_MFMA = range(4)
SGMV_ROUTE_NONE, SGMV_ROUTE_DECODE, SGMV_ROUTE_MFMA, SGMV_ROUTE_VECTOR = range(4)
SGMV_WS_COUNTER_BYTES = 1 << 20
SGMV_MAX_PROJECTIONS = 4

ENTRY_POINTS = ("sgmv_status_str", "sgmv_build_segments", "sgmv_check_problem",
                "sgmv_check_segments", "sgmv_workspace_bytes", "sgmv_query_plan", "sgmv_shrink",
                "sgmv_expand", "sgmv_lora_apply", "sgmv_lora_apply_batched", "sgmv_base_workspace_bytes",
                "sgmv_base_lora_apply", "sgmv_base_packed_weight_bytes", "sgmv_base_pack_weight",
                "sgmv_base_lora_apply_packed", "sgmv_set_wait_limit", "sgmv_take_device_errors",
                "sgmv_lora_apply_noalloc", "sgmv_base_lora_apply_partial", "sgmv_lora_apply_host_meta")
SGMV_DEVICE_ERR_WAIT_TIMEOUT = 1
SGMV_NOALLOC_MAX_WORKSPACE = 16 << 20
SGMV_BASE_MAX_ROWS = 128
SGMV_HOST_META_MAX_SEGS = 64


class SgmvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sgmv_status_str(status)}")


class sgmv_problem_t(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_rows", ctypes.c_int32), ("h_in", ctypes.c_int32),
                ("h_out", ctypes.c_int32), ("rank", ctypes.c_int32), ("num_loras", ctypes.c_int32),
                ("num_segs", ctypes.c_int32), ("max_seg_len", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("splits", ctypes.c_int32)]

    def __repr__(self):
        return "sgmv_problem_t(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class sgmv_plan_info_t(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int32), ("launches", ctypes.c_int32), ("rows_per_unit", ctypes.c_int32),
                ("units", ctypes.c_int32), ("splits", ctypes.c_int32), ("grid", ctypes.c_int32)]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class sgmv_projection_t(ctypes.Structure):
    _fields_ = [("A_ptrs", ctypes.c_void_p), ("B_ptrs", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("ranks", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsgmv.so (built in-tree by ``python -m segmented_gather_matvec_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libsgmv is not built ({path} missing); run "
                          "`python -m segmented_gather_matvec_amd.build` with ROCm's hipcc")
    # PyTorch ships its own HIP runtime.  Load it first so that libsgmv binds to
    # that same runtime (one process, one HIP runtime); loading libsgmv first
    # would bring in the system runtime beside torch's, and launches on torch's
    # memory and streams would then fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    prob = ctypes.POINTER(sgmv_problem_t)
    lib.sgmv_status_str.argtypes = [ctypes.c_int]
    lib.sgmv_status_str.restype = ctypes.c_char_p
    lib.sgmv_build_segments.argtypes = [P, I32, I32, P, P, P, P, P]
    lib.sgmv_check_problem.argtypes = [prob]
    lib.sgmv_check_segments.argtypes = [prob, P, P]
    lib.sgmv_workspace_bytes.argtypes = [prob, ctypes.POINTER(SZ)]
    lib.sgmv_query_plan.argtypes = [prob, ctypes.POINTER(sgmv_plan_info_t)]
    lib.sgmv_shrink.argtypes = [prob, P, P, P, P, P, P, SZ, P]
    lib.sgmv_expand.argtypes = [prob, P, P, P, P, P, P]
    lib.sgmv_lora_apply.argtypes = [prob, P, P, P, P, P, P, P, SZ, P]
    lib.sgmv_lora_apply_batched.argtypes = [prob, P, ctypes.POINTER(sgmv_projection_t), I32, P, P, P, P, SZ, P]
    lib.sgmv_base_workspace_bytes.argtypes = [prob, ctypes.POINTER(SZ)]
    lib.sgmv_base_lora_apply.argtypes = [prob, P, P, P, P, P, P, P, P, SZ, P]
    lib.sgmv_base_packed_weight_bytes.argtypes = [I32, I32, ctypes.POINTER(SZ)]
    lib.sgmv_base_pack_weight.argtypes = [P, I32, I32, P, SZ, P]
    lib.sgmv_base_lora_apply_packed.argtypes = [prob, P, P, P, P, P, P, P, P, SZ, P]
    lib.sgmv_set_wait_limit.argtypes = [ctypes.c_int64]
    lib.sgmv_take_device_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    lib.sgmv_lora_apply_noalloc.argtypes = [prob, P, P, P, P, P, P, P]
    lib.sgmv_base_lora_apply_partial.argtypes = [prob, P, P, I32, P, P, P, P, P, P, SZ, P]
    lib.sgmv_lora_apply_host_meta.argtypes = [prob, P, P, P, P, P, P, P, SZ, P]
    for name in ENTRY_POINTS[1:]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def sgmv_status_str(status: int) -> str:
    return load_library().sgmv_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != SGMV_OK:
        raise SgmvError(status, where)


def make_problem(dtype, n_rows, h_in, h_out, rank, num_loras, num_segs, max_seg_len,
                 variant=SGMV_VARIANT_AUTO, splits=0) -> sgmv_problem_t:
    """Fill an sgmv_problem_t; ``dtype`` is 'f16' / 'bf16', a torch dtype, or an SGMV_* code."""
    return sgmv_problem_t(_dtype_code(dtype), int(n_rows), int(h_in), int(h_out), int(rank),
                          int(num_loras), int(num_segs), int(max_seg_len), int(variant), int(splits))


def _dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    if isinstance(dtype, str):
        return {"f16": SGMV_F16, "bf16": SGMV_BF16}[dtype]
    import torch
    return {torch.float16: SGMV_F16, torch.bfloat16: SGMV_BF16}[dtype]


# ----------------------------------------------------------------- host-only

def sgmv_build_segments(req_lora, num_loras: int):
    """Host segment builder.  Returns numpy int32 ``(perm, seg_indptr, lora_idx)`` and the
    int ``max_seg_len``; ``perm[j]`` is the request placed at sorted row j."""
    ids = np.ascontiguousarray(np.asarray(req_lora, dtype=np.int32).reshape(-1))
    n = ids.size
    perm = np.empty(max(n, 1), np.int32)
    seg = np.empty(n + 1, np.int32)
    lidx = np.empty(max(n, 1), np.int32)
    S, mx = ctypes.c_int32(0), ctypes.c_int32(0)
    st = load_library().sgmv_build_segments(ids.ctypes.data, n, int(num_loras), perm.ctypes.data,
                                            seg.ctypes.data, lidx.ctypes.data,
                                            ctypes.byref(S), ctypes.byref(mx))
    _check(st, "sgmv_build_segments")
    return perm[:n], seg[: S.value + 1], lidx[: S.value], int(mx.value)


def sgmv_check_problem(problem: sgmv_problem_t) -> int:
    return load_library().sgmv_check_problem(ctypes.byref(problem))


def sgmv_check_segments(problem: sgmv_problem_t, seg_indptr, lora_idx) -> int:
    sp = np.ascontiguousarray(np.asarray(seg_indptr, dtype=np.int32))
    li = np.ascontiguousarray(np.asarray(lora_idx, dtype=np.int32))
    return load_library().sgmv_check_segments(ctypes.byref(problem), sp.ctypes.data,
                                              li.ctypes.data if li.size else None)


def sgmv_workspace_bytes(problem: sgmv_problem_t) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().sgmv_workspace_bytes(ctypes.byref(problem), ctypes.byref(out)),
           "sgmv_workspace_bytes")
    return int(out.value)


def sgmv_query_plan(problem: sgmv_problem_t) -> sgmv_plan_info_t:
    """Route, row block, split and grid that sgmv_lora_apply takes on the current device."""
    info = sgmv_plan_info_t()
    _check(load_library().sgmv_query_plan(ctypes.byref(problem), ctypes.byref(info)), "sgmv_query_plan")
    return info


def sgmv_set_wait_limit(microseconds: int):
    """Bound (us) on a decode-route workgroup's wait for its unit's partials; 0 gives up at once."""
    _check(load_library().sgmv_set_wait_limit(int(microseconds)), "sgmv_set_wait_limit")


def sgmv_take_device_errors() -> int:
    """Synchronise the current device, then read and clear its SGMV_DEVICE_ERR_* bits."""
    out = ctypes.c_uint32(0)
    _check(load_library().sgmv_take_device_errors(ctypes.byref(out)), "sgmv_take_device_errors")
    return int(out.value)


# ----------------------------------------------------------------- device calls

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _torch_dtype(problem):
    import torch
    return torch.bfloat16 if problem.dtype == SGMV_BF16 else torch.float16


def sgmv_shrink(problem, X, A_ptrs, V, seg_indptr, lora_idx, ws, stream=None):
    """V[i] = X[i] @ A_{lora_idx[s]} (fp32 V) on the device; asynchronous."""
    import torch
    _need(X, "X", _torch_dtype(problem)); _need(V, "V", torch.float32)
    _need(A_ptrs, "A_ptrs", torch.int64); _need(seg_indptr, "seg_indptr", torch.int32)
    _need(lora_idx, "lora_idx", torch.int32); _need(ws, "ws")
    st = load_library().sgmv_shrink(ctypes.byref(problem), _ptr(X), _ptr(A_ptrs), _ptr(V),
                                    _ptr(seg_indptr), _ptr(lora_idx), _ptr(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0,
                                    _stream(stream))
    _check(st, "sgmv_shrink")


def sgmv_expand(problem, V, B_ptrs, Y, seg_indptr, lora_idx, stream=None):
    """Y[i] += V[i] @ B_{lora_idx[s]} on the device; asynchronous."""
    import torch
    _need(V, "V", torch.float32); _need(Y, "Y", _torch_dtype(problem))
    _need(B_ptrs, "B_ptrs", torch.int64); _need(seg_indptr, "seg_indptr", torch.int32)
    _need(lora_idx, "lora_idx", torch.int32)
    st = load_library().sgmv_expand(ctypes.byref(problem), _ptr(V), _ptr(B_ptrs), _ptr(Y),
                                    _ptr(seg_indptr), _ptr(lora_idx), _stream(stream))
    _check(st, "sgmv_expand")


def sgmv_lora_apply(problem, X, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, stream=None):
    """Y[i] += (X[i] @ A_k) @ B_k on the device; asynchronous."""
    import torch
    dt = _torch_dtype(problem)
    _need(X, "X", dt); _need(Y, "Y", dt)
    _need(A_ptrs, "A_ptrs", torch.int64); _need(B_ptrs, "B_ptrs", torch.int64)
    _need(seg_indptr, "seg_indptr", torch.int32); _need(lora_idx, "lora_idx", torch.int32)
    _need(ws, "ws")
    st = load_library().sgmv_lora_apply(ctypes.byref(problem), _ptr(X), _ptr(A_ptrs), _ptr(B_ptrs),
                                        _ptr(Y), _ptr(seg_indptr), _ptr(lora_idx), _ptr(ws),
                                        ws.numel() * ws.element_size() if ws is not None else 0,
                                        _stream(stream))
    _check(st, "sgmv_lora_apply")


def sgmv_lora_apply_host_meta(problem, X, A_ptrs_host, B_ptrs_host, Y, seg_indptr_host, lora_idx_host, ws,
                              stream=None):
    """sgmv_lora_apply with the segment metadata and the LoRA pointer tables on the host
    (numpy int32 seg_indptr / lora_idx, uint64 or int64 arrays of device pointers),
    carried in the kernel's arguments; decode-shaped calls of at most
    SGMV_HOST_META_MAX_SEGS segments only.  Asynchronous."""
    import numpy as np
    dt = _torch_dtype(problem)
    _need(X, "X", dt); _need(Y, "Y", dt)
    _need(ws, "ws")
    a = np.ascontiguousarray(A_ptrs_host, dtype=np.uint64)
    b = np.ascontiguousarray(B_ptrs_host, dtype=np.uint64)
    seg = np.ascontiguousarray(seg_indptr_host, dtype=np.int32)
    lidx = np.ascontiguousarray(lora_idx_host, dtype=np.int32)
    if lidx.size == 0:
        lidx = np.zeros(1, np.int32)
    st = load_library().sgmv_lora_apply_host_meta(ctypes.byref(problem), _ptr(X), a.ctypes.data, b.ctypes.data,
                                                  _ptr(Y), seg.ctypes.data, lidx.ctypes.data, _ptr(ws),
                                                  ws.numel() * ws.element_size() if ws is not None else 0,
                                                  _stream(stream))
    _check(st, "sgmv_lora_apply_host_meta")


def sgmv_lora_apply_noalloc(problem, X, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, stream=None):
    """sgmv_lora_apply on the library's static device scratch (no workspace argument,
    nothing allocated); calls that overlap on one GPU race.  Asynchronous."""
    import torch
    dt = _torch_dtype(problem)
    _need(X, "X", dt); _need(Y, "Y", dt)
    _need(A_ptrs, "A_ptrs", torch.int64); _need(B_ptrs, "B_ptrs", torch.int64)
    _need(seg_indptr, "seg_indptr", torch.int32); _need(lora_idx, "lora_idx", torch.int32)
    st = load_library().sgmv_lora_apply_noalloc(ctypes.byref(problem), _ptr(X), _ptr(A_ptrs), _ptr(B_ptrs),
                                                _ptr(Y), _ptr(seg_indptr), _ptr(lora_idx), _stream(stream))
    _check(st, "sgmv_lora_apply_noalloc")


def sgmv_lora_apply_batched(problem, X, projections, seg_indptr, lora_idx, ws, row_idx=None, stream=None):
    """Y_p[row(i)] += s_{p,k} * (X[row(i)] @ A_{p,k}) @ B_{p,k} for each projection in
    `projections` (up to SGMV_MAX_PROJECTIONS), one call; asynchronous.  A projection
    is (A_ptrs, B_ptrs, Y) or (A_ptrs, B_ptrs, Y, ranks, scales): `ranks` (device
    int32 [num_loras] or None) gives each LoRA's own rank (compact A_k [h_in, r_k],
    B_k [r_k, h_out]; problem.rank is the largest), `scales` (device float32
    [num_loras] or None) the factor of each LoRA's term.  `row_idx` (optional device
    int32 [n_rows], e.g. the builder's perm) maps sorted row i to row row_idx[i] of
    X and Y.  `ws` must hold batched_workspace_bytes(problem, len(projections)) bytes."""
    import torch
    dt = _torch_dtype(problem)
    _need(X, "X", dt)
    _need(seg_indptr, "seg_indptr", torch.int32); _need(lora_idx, "lora_idx", torch.int32)
    _need(row_idx, "row_idx", torch.int32)
    _need(ws, "ws")
    arr = (sgmv_projection_t * max(1, len(projections)))()
    for i, pj in enumerate(projections):
        A_ptrs, B_ptrs, Y = pj[:3]
        ranks, scales = (tuple(pj[3:]) + (None, None))[:2]
        _need(Y, f"Y[{i}]", dt)
        _need(A_ptrs, f"A_ptrs[{i}]", torch.int64); _need(B_ptrs, f"B_ptrs[{i}]", torch.int64)
        _need(ranks, f"ranks[{i}]", torch.int32); _need(scales, f"scales[{i}]", torch.float32)
        arr[i] = sgmv_projection_t(_ptr(A_ptrs), _ptr(B_ptrs), _ptr(Y), _ptr(ranks), _ptr(scales))
    st = load_library().sgmv_lora_apply_batched(ctypes.byref(problem), _ptr(X), arr, len(projections),
                                                _ptr(seg_indptr), _ptr(lora_idx), _ptr(row_idx), _ptr(ws),
                                                ws.numel() * ws.element_size() if ws is not None else 0,
                                                _stream(stream))
    _check(st, "sgmv_lora_apply_batched")


# ----------------------------------------------------------------- helpers

def sgmv_base_workspace_bytes(problem: sgmv_problem_t) -> int:
    """Workspace bytes of sgmv_base_lora_apply (n_rows <= SGMV_BASE_MAX_ROWS)."""
    out = ctypes.c_size_t(0)
    _check(load_library().sgmv_base_workspace_bytes(ctypes.byref(problem), ctypes.byref(out)),
           "sgmv_base_workspace_bytes")
    return int(out.value)


def new_base_workspace(problem: sgmv_problem_t, device="cuda"):
    """Zero-filled device workspace of sgmv_base_workspace_bytes(problem) bytes."""
    import torch
    return torch.zeros(sgmv_base_workspace_bytes(problem), dtype=torch.uint8, device=device)


def _base_apply(name, problem, X, W, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, stream):
    import torch
    dt = _torch_dtype(problem)
    _need(X, "X", dt); _need(W, "W", dt); _need(Y, "Y", dt)
    _need(A_ptrs, "A_ptrs", torch.int64); _need(B_ptrs, "B_ptrs", torch.int64)
    _need(seg_indptr, "seg_indptr", torch.int32); _need(lora_idx, "lora_idx", torch.int32)
    _need(ws, "ws")
    st = getattr(load_library(), name)(ctypes.byref(problem), _ptr(X), _ptr(W), _ptr(A_ptrs),
                                       _ptr(B_ptrs), _ptr(Y), _ptr(seg_indptr), _ptr(lora_idx),
                                       _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                       _stream(stream))
    _check(st, name)


def sgmv_base_lora_apply(problem, X, W, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, stream=None):
    """Y[i] = X[i] @ W + (X[i] @ A_k) @ B_k on the device (Y written, rounded once); asynchronous.
    Rows no segment covers get X[i] @ W.  At most SGMV_BASE_MAX_ROWS rows."""
    _base_apply("sgmv_base_lora_apply", problem, X, W, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, stream)


def sgmv_base_lora_apply_partial(problem, X, W, A_ptrs, B_ptrs, Yp, seg_indptr, lora_idx, ws, w_packed=False,
                                 stream=None):
    """One shard of a row-parallel base layer: Yp[i] = X_g[i] @ W_g + (X_g[i] @ A_{k,g}) @ B_k in
    fp32, unrounded (Yp float32 [n_rows, h_out]); W_g row-major or packed (w_packed)."""
    import torch
    dt = _torch_dtype(problem)
    _need(X, "X", dt); _need(W, "W", dt); _need(Yp, "Yp", torch.float32)
    _need(A_ptrs, "A_ptrs", torch.int64); _need(B_ptrs, "B_ptrs", torch.int64)
    _need(seg_indptr, "seg_indptr", torch.int32); _need(lora_idx, "lora_idx", torch.int32)
    _need(ws, "ws")
    st = load_library().sgmv_base_lora_apply_partial(
        ctypes.byref(problem), _ptr(X), _ptr(W), 1 if w_packed else 0, _ptr(A_ptrs), _ptr(B_ptrs), _ptr(Yp),
        _ptr(seg_indptr), _ptr(lora_idx), _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream))
    _check(st, "sgmv_base_lora_apply_partial")


def sgmv_base_packed_weight_bytes(h_in: int, h_out: int) -> int:
    """Bytes of the packed copy of a [h_in, h_out] base weight."""
    out = ctypes.c_size_t(0)
    _check(load_library().sgmv_base_packed_weight_bytes(int(h_in), int(h_out), ctypes.byref(out)),
           "sgmv_base_packed_weight_bytes")
    return int(out.value)


def sgmv_base_pack_weight(W, Wp, stream=None):
    """Write the packed copy of the 2-D device weight W into Wp (asynchronous)."""
    _need(W, "W"); _need(Wp, "Wp")
    if W.dim() != 2 or W.element_size() != 2:
        raise ValueError("W must be a 2-D tensor of a 16-bit format")
    h_in, h_out = W.shape
    st = load_library().sgmv_base_pack_weight(_ptr(W), int(h_in), int(h_out), _ptr(Wp),
                                              Wp.numel() * Wp.element_size(), _stream(stream))
    _check(st, "sgmv_base_pack_weight")


def pack_base_weight(W, stream=None):
    """New device tensor (same format as W, flat) holding the packed copy of W."""
    import torch
    n = sgmv_base_packed_weight_bytes(*W.shape) // W.element_size()
    Wp = torch.empty(n, dtype=W.dtype, device=W.device)
    sgmv_base_pack_weight(W, Wp, stream)
    return Wp


def sgmv_base_lora_apply_packed(problem, X, Wp, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws, stream=None):
    """sgmv_base_lora_apply with Wp, the packed copy of W, in place of W."""
    _base_apply("sgmv_base_lora_apply_packed", problem, X, Wp, A_ptrs, B_ptrs, Y, seg_indptr, lora_idx, ws,
                stream)


def batched_workspace_bytes(problem: sgmv_problem_t, num_projections: int) -> int:
    """Workspace bytes of sgmv_lora_apply_batched: one 256-byte aligned slice per projection."""
    w = sgmv_workspace_bytes(problem)
    return (num_projections - 1) * ((w + 255) // 256 * 256) + w


def pointer_table(stacked) -> "torch.Tensor":
    """Device int64 table of per-LoRA pointers into a stacked [P, ...] tensor."""
    import torch
    _need(stacked, "stacked weights")
    P = stacked.shape[0]
    stride = stacked[0].numel() * stacked.element_size() if P else 0
    return (torch.arange(P, device=stacked.device, dtype=torch.int64) * stride
            + stacked.data_ptr()).contiguous()


def pointer_list(tensors, device="cuda") -> "torch.Tensor":
    """Device int64 table of the data pointers of separately allocated per-LoRA
    tensors (None: a null entry, allowed for a LoRA of rank 0)."""
    import torch
    return torch.tensor([0 if t is None else t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def new_workspace(problem: sgmv_problem_t, device="cuda"):
    """Zero-filled device workspace of sgmv_workspace_bytes(problem) bytes."""
    import torch
    nbytes = sgmv_workspace_bytes(problem)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)
