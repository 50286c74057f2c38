"""Seeded synthetic SGMV workloads, shared by the tests, the smoke check and the benchmark.

This module holds no part of the method's arithmetic: it only draws random
numbers, casts them to fp16 / bf16 bit patterns (round to nearest even) and
lays out the segment structures each workload states.  Segment metadata that
must come from the segment builder is NOT made here: such workloads return the
per-request LoRA ids (``req_lora``) with X / Y0 in request order, and the
caller runs a builder and permutes rows.

Value distributions (shared by every workload unless stated): X ~ N(0, 1),
A_k ~ N(0, 1/H1), B_k ~ N(0, 1/r), Y0 ~ N(0, 1) (standing in for the base
projection X@W).  Host draws use ``numpy.random.default_rng(seed)`` (PCG64)
in the fixed order: ids -> segment lengths -> X -> A_k (k ascending) -> B_k
-> Y0.  LoRA popularity follows the four cases of the Punica README's
throughput paragraph (page "Punica：多 LoRA 模型统一服务框架"): Distinct (every
request its own LoRA), Identical (one LoRA), Uniform and Skewed in between.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

F16, BF16 = "f16", "bf16"


def to_bits(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16 / bf16 (nearest even); return uint16 bit patterns."""
    v = np.ascontiguousarray(values_f32, dtype=np.float32)
    if dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        t = torch.from_numpy(v).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


@dataclass
class Workload:
    """One SGMV call's inputs as uint16 bit patterns (row-major)."""
    name: str
    dtype: str
    h_in: int
    h_out: int
    rank: int
    num_loras: int
    X: np.ndarray                      # [n, h_in]
    A: np.ndarray                      # [P, h_in, rank]
    B: np.ndarray                      # [P, rank, h_out]
    Y0: np.ndarray                     # [n, h_out]
    seg_indptr: Optional[np.ndarray] = None   # int32 [S+1] when the workload fixes segments
    lora_idx: Optional[np.ndarray] = None     # int32 [S]
    req_lora: Optional[np.ndarray] = None     # int32 [n] when a builder must make the segments
    meta: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.X.shape[0])


def _normal_bits(rng, shape, std, dtype):
    return to_bits(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std), dtype)


def _values(rng, n, h_in, h_out, rank, num_loras, dtype, y0="normal"):
    X = _normal_bits(rng, (n, h_in), 1.0, dtype)
    A = np.stack([_normal_bits(rng, (h_in, rank), 1.0 / np.sqrt(h_in), dtype)
                  for _ in range(num_loras)]) if num_loras else np.zeros((0, h_in, rank), np.uint16)
    B = np.stack([_normal_bits(rng, (rank, h_out), 1.0 / np.sqrt(rank), dtype)
                  for _ in range(num_loras)]) if num_loras else np.zeros((0, rank, h_out), np.uint16)
    if y0 == "zero":
        Y0 = np.zeros((n, h_out), np.uint16)
    else:
        Y0 = _normal_bits(rng, (n, h_out), 1.0, dtype)
    return X, A, B, Y0


def tiny(seed: int = 1) -> Workload:
    """H1=H2=256, r=8, 4 LoRAs, 8 fp16 rows in segments of lengths [3,1,2,2] bound to
    LoRA ids [2,0,3,1] (unsorted on purpose), Y0 = 0."""
    rng = np.random.default_rng(seed)
    lengths = [3, 1, 2, 2]
    ids = [2, 0, 3, 1]
    X, A, B, Y0 = _values(rng, 8, 256, 256, 8, 4, F16, y0="zero")
    seg = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return Workload("tiny", F16, 256, 256, 8, 4, X, A, B, Y0, seg, np.array(ids, np.int32))


def decode_distinct(seed: int = 2, n: int = 32, h: int = 4096, rank: int = 16,
                    dtype: str = F16) -> Workload:
    """Decode batch, Distinct popularity: one row per segment, row i uses LoRA i
    (Llama-7B q_proj shape by default)."""
    rng = np.random.default_rng(seed)
    X, A, B, Y0 = _values(rng, n, h, h, rank, n, dtype)
    seg = np.arange(n + 1, dtype=np.int32)
    return Workload(f"decode_distinct_b{n}", dtype, h, h, rank, n, X, A, B, Y0, seg,
                    np.arange(n, dtype=np.int32))


def zipf_probs(pool: int, s: float = 1.5) -> np.ndarray:
    """Truncated Zipf over ids 0..pool-1: P(id = k-1) proportional to k^-s."""
    w = np.arange(1, pool + 1, dtype=np.float64) ** (-s)
    return w / w.sum()


def draw_ids(rng, kind: str, n: int) -> (np.ndarray, int):
    """Per-request LoRA ids for a popularity case; returns (ids, pool size)."""
    if kind == "identical":
        return np.zeros(n, np.int32), 1
    if kind == "distinct":
        return np.arange(n, dtype=np.int32), n
    if kind == "uniform":
        return rng.integers(0, 32, size=n).astype(np.int32), 32
    if kind == "skewed":
        return rng.choice(50, size=n, p=zipf_probs(50)).astype(np.int32), 50
    raise ValueError(kind)


POPULARITY_SEEDS = {("identical", 32): 31, ("identical", 64): 32, ("uniform", 32): 33,
                    ("uniform", 64): 34, ("skewed", 32): 35, ("skewed", 64): 36}


def popularity(kind: str, n: int, seed: Optional[int] = None, h: int = 4096, rank: int = 16,
               dtype: str = F16) -> Workload:
    """Decode batch with LoRA ids drawn Identical / Uniform (pool 32) / Skewed
    (Zipf s=1.5 over a pool of 50).  X and Y0 are in request order; a segment
    builder must sort them (``req_lora`` holds the ids)."""
    if seed is None:
        seed = POPULARITY_SEEDS.get((kind, n), 30)
    rng = np.random.default_rng(seed)
    ids, pool = draw_ids(rng, kind, n)
    X, A, B, Y0 = _values(rng, n, h, h, rank, pool, dtype)
    return Workload(f"{kind}_b{n}", dtype, h, h, rank, pool, X, A, B, Y0, req_lora=ids)


def mixed_layout(rng, num_loras: int = 16, n_prefill: int = 8, n_decode: int = 24,
                 lo: int = 128, hi: int = 1024):
    """Mixed prefill+decode segments: n_prefill segments of length U{lo..hi} first, then
    n_decode one-row segments; ids are two seeded permutations of 0..num_loras-1 back to
    back, so every LoRA serves exactly two segments."""
    ids = np.concatenate([rng.permutation(num_loras), rng.permutation(num_loras)]).astype(np.int32)
    ids = ids[: n_prefill + n_decode]
    lengths = np.concatenate([rng.integers(lo, hi + 1, size=n_prefill), np.ones(n_decode, np.int64)])
    seg = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return seg, ids


def mixed(rank: int, seed: Optional[int] = None, pairs=((4096, 11008), (11008, 4096)),
          num_loras: int = 16, lo: int = 128, hi: int = 1024, n_prefill: int = 8,
          n_decode: int = 24) -> List[Workload]:
    """Mixed prefill+decode batch on Llama-7B MLP shapes, bf16: one Workload per
    (h_in, h_out) pair, all sharing the segment layout."""
    if seed is None:
        seed = 41 if rank == 16 else 42
    rng = np.random.default_rng(seed)
    seg, ids = mixed_layout(rng, num_loras, n_prefill, n_decode, lo, hi)
    n = int(seg[-1])
    out = []
    for h_in, h_out in pairs:
        X, A, B, Y0 = _values(rng, n, h_in, h_out, rank, num_loras, BF16)
        out.append(Workload(f"mixed_r{rank}_{h_in}to{h_out}", BF16, h_in, h_out, rank, num_loras,
                            X, A, B, Y0, seg.copy(), ids.copy()))
    return out


def base_weight(rng, h_in: int, h_out: int, dtype: str) -> np.ndarray:
    """Base projection weight W [h_in, h_out] ~ N(0, 1/h_in), so that X @ W ~ N(0, 1)."""
    return _normal_bits(rng, (h_in, h_out), 1.0 / np.sqrt(h_in), dtype)


def integer_exact(rng, n, h_in, h_out, rank, num_loras, dtype, nnz_per_col, y0_bound):
    """Inputs whose every product and partial sum is an integer well inside fp32's exact
    range and whose final Y is exact in fp16 / bf16: X, B in {-1, 0, 1}; each column of
    A_k has exactly ``nnz_per_col`` entries in {-1, +1}; Y0 integer in [-y0_bound, y0_bound].
    With rank*nnz_per_col + y0_bound <= 2048 (fp16) or <= 256 (bf16) every result is
    representable, so any summation order gives the same bits."""
    X = rng.integers(-1, 2, size=(n, h_in)).astype(np.float32)
    A = np.zeros((num_loras, h_in, rank), np.float32)
    for k in range(num_loras):
        for j in range(rank):
            rows = rng.choice(h_in, size=nnz_per_col, replace=False)
            A[k, rows, j] = rng.choice([-1.0, 1.0], size=nnz_per_col)
    B = rng.integers(-1, 2, size=(num_loras, rank, h_out)).astype(np.float32)
    Y0 = rng.integers(-y0_bound, y0_bound + 1, size=(n, h_out)).astype(np.float32)
    return to_bits(X, dtype), to_bits(A, dtype), to_bits(B, dtype), to_bits(Y0, dtype)


# ---------------------------------------------------------------------------
# Device-side generation for workloads too large to draw on the host.
# ---------------------------------------------------------------------------

def device_normal(shape, std, dtype: str, seed: int, device="cuda"):
    """Seeded N(0, std^2) tensor drawn by torch's generator on ``device``, cast
    (nearest even) to float16 / bfloat16."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(torch.float16 if dtype == F16 else torch.bfloat16)


# 13B full-model LoRA sweep: 40 layers x 7 projections, r=64, bf16, 64 LoRAs.
LLAMA13B_PROJ = (("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
                 ("gate", 5120, 13824), ("up", 5120, 13824), ("down", 13824, 5120))
LLAMA13B_LAYERS = 40


def full_model_ids(seed: int = 5, n: int = 256, pool: int = 64) -> np.ndarray:
    """Per-request LoRA ids for the 13B sweep: truncated Zipf s=1.5 over 64 LoRAs,
    drawn once (a request keeps its LoRA in every layer)."""
    rng = np.random.default_rng(seed)
    return rng.choice(pool, size=n, p=zipf_probs(pool)).astype(np.int32)


def full_model_weight_seed(layer: int, proj: int) -> int:
    return 5000 + 7 * layer + proj
