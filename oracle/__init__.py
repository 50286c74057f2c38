"""Oracle for the SGMV LoRA term: plain, slow, obviously correct, CPU only.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The library's compute
path (``segmented_gather_matvec_amd``) never imports it, and it imports
nothing from that package: the two share no code.

Contents
--------
* ``sgmv_oracle.c`` (built here with gcc into ``liboracle_sgmv.so``): fp64
  loops over rows that decode fp16/bf16 inputs exactly and evaluate
  ``Y0[i] + (x_i @ A_k) @ B_k`` as the Punica README states it (page
  "Punica：多 LoRA 模型统一服务框架", LoRA and multi-LoRA paragraphs).
* ``sgmv_base_apply``: the base projection with the LoRA term,
  ``x_i @ W + (x_i @ A_k) @ B_k`` (same page, LoRA paragraph), for rows with
  and without a segment.
* ``build_segments``: the segment builder written as a plain stable sort in
  Python (same page, multi-LoRA and SGMV paragraphs: every request is bound
  to its LoRA, and requests sharing a LoRA form one segment).

Readings taken where the pages are silent: segment metadata is CSR
(``seg_indptr`` [S+1], ``lora_idx`` [S]); segments may come in any order and
repeat ids; empty segments are no-ops; rows past ``seg_indptr[S]`` keep
``Y0`` (and get ``X @ W`` alone in the base projection); the LoRA scale is 1
unless a per-LoRA scale is given, which multiplies the LoRA term only; a
LoRA of smaller rank is its pair zero-padded; the builder sorts by ascending
LoRA id with ties kept in request order and emits only non-empty segments.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgmv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_sgmv.so")

DTYPES = {"f16": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.oracle_decode.argtypes = [ctypes.c_int, p, p, i64]
    lib.oracle_decode.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_sgmv_shrink.argtypes = [ctypes.c_int, i32, i32, i32, p, p, i32, p, p, i32, p, p,
                                       ctypes.c_int]
    lib.oracle_sgmv_shrink.restype = ctypes.c_int
    lib.oracle_sgmv_expand.argtypes = [ctypes.c_int, i32, i32, i32, p, p, i32, p, p, i32, p, p,
                                       p, ctypes.c_int]
    lib.oracle_sgmv_expand.restype = ctypes.c_int
    lib.oracle_sgmv_apply.argtypes = [ctypes.c_int, i32, i32, i32, i32, p, p, p, p, p, i32, p, p, i32,
                                      p, p, p, p, ctypes.c_int]
    lib.oracle_sgmv_apply.restype = ctypes.c_int
    lib.oracle_sgmv_base_apply.argtypes = [ctypes.c_int, i32, i32, i32, i32, p, p, p, p, i32, p, p, i32, p,
                                           p, ctypes.c_int]
    lib.oracle_sgmv_base_apply.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every oracle call to another build of sgmv_oracle.c
    (the mutation tests use it to show that the pins reject planted mistakes)."""
    global _lib
    saved = _lib
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns or float16, got {a.dtype}")
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _table(mats: Sequence[np.ndarray]):
    """ctypes array of host pointers, one per LoRA matrix (keeps the arrays alive)."""
    arrs = [_u16(m) for m in mats]
    table = (ctypes.c_void_p * max(len(arrs), 1))(*[_ptr(a) for a in arrs])
    return table, arrs


def _mask(row_mask, n_rows):
    if row_mask is None:
        return None, 0
    m = np.ascontiguousarray(np.asarray(row_mask, dtype=np.uint8))
    if m.shape != (n_rows,):
        raise ValueError("row_mask must have one entry per row")
    return m, _ptr(m)


def decode(bits, dtype: str) -> np.ndarray:
    """Exact fp64 value of every fp16/bf16 bit pattern in ``bits``."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode(DTYPES[dtype], _ptr(b), _ptr(out), b.size)
    return out


def sgmv_shrink(dtype, X, A, seg_indptr, lora_idx, *, row_mask=None, nthreads=0, out=None):
    """fp64 V[i] = x_i @ A_{lora_idx[s]} for covered rows (others stay NaN or ``out``)."""
    X = _u16(X)
    n, h_in = X.shape
    rank = _u16(A[0]).shape[1]
    sp, li = _i32(seg_indptr), _i32(lora_idx)
    table, keep = _table(A)
    V = np.full((n, rank), np.nan) if out is None else out
    m, mp = _mask(row_mask, n)
    rc = _load().oracle_sgmv_shrink(DTYPES[dtype], n, h_in, rank, _ptr(X), ctypes.addressof(table),
                                    len(keep), _ptr(sp), _ptr(li), len(li), mp, _ptr(V), nthreads)
    if rc != 0:
        raise ValueError("oracle: invalid segment metadata")
    return V


def sgmv_expand(dtype, V, B, seg_indptr, lora_idx, Y0, *, row_mask=None, nthreads=0):
    """fp64 Y[i] = Y0[i] + V[i] @ B_{lora_idx[s]} (uncovered rows: Y0 exactly)."""
    V = np.ascontiguousarray(V, dtype=np.float64)
    Y0 = _u16(Y0)
    n, h_out = Y0.shape
    rank = V.shape[1]
    sp, li = _i32(seg_indptr), _i32(lora_idx)
    table, keep = _table(B)
    Y = np.full((n, h_out), np.nan)
    m, mp = _mask(row_mask, n)
    rc = _load().oracle_sgmv_expand(DTYPES[dtype], n, h_out, rank, _ptr(V), ctypes.addressof(table),
                                    len(keep), _ptr(sp), _ptr(li), len(li), _ptr(Y0), mp, _ptr(Y),
                                    nthreads)
    if rc != 0:
        raise ValueError("oracle: invalid segment metadata")
    return Y


def sgmv_apply(dtype, X, A, B, seg_indptr, lora_idx, Y0, *, scales=None, rank=None, row_mask=None,
               nthreads=0, want_v=False):
    """fp64 Y = Y0 + per-row s_k * (x_i @ A_k) @ B_k.  Returns Y, or (Y, V) with ``want_v``.

    Each A[k] is [h_in, r_k] and B[k] is [r_k, h_out]; the ranks may differ
    (rank 0: the LoRA adds nothing).  ``rank`` is the width of V (default: the
    largest r_k); ``scales`` (default all 1) gives s_k per LoRA."""
    X, Y0 = _u16(X), _u16(Y0)
    n, h_in = X.shape
    h_out = Y0.shape[1]
    # Ranks of the LoRAs that a non-empty segment uses (the others are never
    # read and may be placeholders).
    sp0, li0 = _i32(seg_indptr), _i32(lora_idx)
    # (Ids out of range and malformed segments are left for the C side to reject.)
    used = sorted({int(li0[s]) for s in range(min(len(li0), len(sp0) - 1))
                   if sp0[s + 1] > sp0[s] and 0 <= li0[s] < len(A)})
    rk = np.zeros(len(A), dtype=np.int32)
    for k in used:
        a, b = _u16(A[k]), _u16(B[k])
        if a.ndim != 2 or b.ndim != 2 or a.shape[0] != h_in or b.shape[1] != h_out or a.shape[1] != b.shape[0]:
            raise ValueError(f"LoRA {k}: A {a.shape} and B {b.shape} are not [{h_in}, r] and [r, {h_out}]")
        rk[k] = a.shape[1]
    rank = int(rank if rank is not None else max(int(rk.max(initial=0)), 1))
    uniform = all(rk[k] == rank for k in used)
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float64)
    if sc is not None and sc.shape != (len(A),):
        raise ValueError("scales must hold one value per LoRA")
    sp, li = _i32(seg_indptr), _i32(lora_idx)
    ta, ka = _table(A)
    tb, kb = _table(B)
    if len(ka) != len(kb):
        raise ValueError("A and B must list the same number of LoRAs")
    Y = np.full((n, h_out), np.nan)
    V = np.full((n, rank), np.nan) if want_v else None
    m, mp = _mask(row_mask, n)
    rc = _load().oracle_sgmv_apply(DTYPES[dtype], n, h_in, h_out, rank, 0 if uniform else _ptr(rk),
                                   0 if sc is None else _ptr(sc), _ptr(X),
                                   ctypes.addressof(ta), ctypes.addressof(tb), len(ka), _ptr(sp),
                                   _ptr(li), len(li), _ptr(Y0), mp, _ptr(Y),
                                   _ptr(V) if want_v else 0, nthreads)
    if rc != 0:
        raise ValueError("oracle: invalid segment metadata")
    return (Y, V) if want_v else Y


def sgmv_base_apply(dtype, X, W, A, B, seg_indptr, lora_idx, *, row_mask=None, nthreads=0):
    """fp64 Y = X @ W + per-row (x_i @ A_k) @ B_k (rows no segment covers: X @ W only).

    W is [h_in, h_out]; every A[k] is [h_in, r] and B[k] is [r, h_out] with one r.
    Rows outside ``row_mask`` (when given) are left NaN."""
    X, W = _u16(X), _u16(W)
    n, h_in = X.shape
    if W.ndim != 2 or W.shape[0] != h_in:
        raise ValueError(f"W {W.shape} is not [{h_in}, h_out]")
    h_out = W.shape[1]
    ta, ka = _table(A)
    tb, kb = _table(B)
    if len(ka) != len(kb):
        raise ValueError("A and B must list the same number of LoRAs")
    a0 = _u16(A[0])
    rank = int(a0.shape[1])
    for k in range(len(ka)):
        a, b = _u16(A[k]), _u16(B[k])
        if a.shape != (h_in, rank) or b.shape != (rank, h_out):
            raise ValueError(f"LoRA {k}: A {a.shape} and B {b.shape} are not [{h_in}, {rank}] and [{rank}, {h_out}]")
    sp, li = _i32(seg_indptr), _i32(lora_idx)
    Y = np.full((n, h_out), np.nan)
    m, mp = _mask(row_mask, n)
    rc = _load().oracle_sgmv_base_apply(DTYPES[dtype], n, h_in, h_out, rank, _ptr(X), _ptr(W),
                                        ctypes.addressof(ta), ctypes.addressof(tb), len(ka), _ptr(sp),
                                        _ptr(li), len(li), mp, _ptr(Y), nthreads)
    if rc != 0:
        raise ValueError("oracle: invalid segment metadata")
    return Y


def build_segments(req_lora: Sequence[int], num_loras: int):
    """Segment builder as a plain stable sort (pure Python).

    Returns ``(perm, seg_indptr, lora_idx, max_seg_len)`` where ``perm[j]`` is
    the request placed at sorted row j, segments are the runs of equal LoRA id
    in ascending id order, and ties keep request order.
    """
    ids = [int(v) for v in req_lora]
    for v in ids:
        if not 0 <= v < num_loras:
            raise ValueError(f"LoRA id {v} outside [0, {num_loras})")
    perm = sorted(range(len(ids)), key=lambda i: (ids[i], i))
    seg_indptr = [0]
    lora_idx = []
    for j, i in enumerate(perm):
        if j > 0 and ids[i] != ids[perm[j - 1]]:
            seg_indptr.append(j)
        if j == 0 or ids[i] != ids[perm[j - 1]]:
            lora_idx.append(ids[i])
    if ids:
        seg_indptr.append(len(ids))
    lengths = [seg_indptr[s + 1] - seg_indptr[s] for s in range(len(lora_idx))]
    return perm, seg_indptr, lora_idx, max(lengths, default=0)
