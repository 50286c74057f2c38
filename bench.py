#!/usr/bin/env python3
"""Benchmark of libsgmv's SGMV LoRA term on one MI355X.

Default workload (the headline): decode batch, Distinct LoRA popularity
(Punica README, page "Punica：多 LoRA 模型统一服务框架", throughput paragraph):
H1 = H2 = 4096 (Llama-7B q_proj), r = 16, 32 fp16 rows, one row per segment,
each on its own LoRA.  One step is one sgmv_lora_apply call (shrink + expand
of the whole batch) with the segment metadata already built.  To measure HBM
rather than the 256 MB Infinity Cache, each call's LoRAs come from a physical
pool of >= 1 GiB (the logical ids are shifted by a multiple of the logical
pool per call, which keeps the popularity structure) and X / Y rotate over
several copies.

Other workloads (--workload): the popularity sweep (Identical / Uniform /
Skewed, batch 32 and 64, segments made by the library's builder), the mixed
prefill+decode batch on Llama-7B MLP shapes (r = 16 or 64, bf16), and one
forward of all 280 LoRA calls of a 13B model (r = 64, bf16, batch 256, Zipf
LoRA assignment), where one step is the whole forward.

Prints one JSON line.  The timed region is K back-to-back steps on one stream,
with HIP events recorded on that stream at both ends and a device
synchronisation before and after.  A bounded sleep kernel (about 200 us, timed
and reported as preroll_us) is queued ahead of the first event, so the host has
already enqueued the first steps when the device clock starts and the events
time the K steps running back to back, not the host-to-device latency of the
first launch (about 15 us, a sixth of a 20-step region of 5 us calls).  value =
whole-job algorithmic GB/s over the device time between the two events
(ms_per_step and tokens_per_s come from the same device time); the host wall
clock around the region less the pre-roll, which adds the fixed cost of the
synchronisations and of the first launch, is reported beside it
(wall_ms_per_step, wall_value).  roofline.achieved = algorithmic bytes per
launch / mean launch duration from the same events; roofline.traffic = HBM
bytes per launch from the committed counter runs (FETCH_SIZE + WRITE_SIZE
scaled by a copy kernel of known size; roofline_traffic_from names the file),
reported only while the kernel sources still match the ones the counters were
taken on; cpu_baseline = the fp64 oracle timed on the host cores on a bounded
sample of the same workload (default workload only).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SGMV shrink+expand achieved HBM GB/s (% peak) and tokens/s, H=4096 r=16 batch 32"
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ("segmented_gather_matvec_amd/csrc/sgmv_decode.hip",
                  "segmented_gather_matvec_amd/csrc/sgmv_device.h",
                  "segmented_gather_matvec_amd/csrc/sgmv_units.h",
                  "segmented_gather_matvec_amd/csrc/sgmv_plan.h",
                  "segmented_gather_matvec_amd/csrc/sgmv_api.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sgmv_decode_kernel_decode_distinct_h4096_r16_b32_traffic.json")
COPY_CALIBRATION_BYTES = 512 << 20
DEFAULT_WORKLOAD = "decode_distinct_h4096_r16_b32"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(elem, n_rows_covered, h_in, h_out, rank, distinct_loras):
    """Minimum HBM bytes of one call: each distinct LoRA's A and B once, X once,
    Y read and written once."""
    return elem * (distinct_loras * (h_in * rank + rank * h_out) + n_rows_covered * h_in
                   + 2 * n_rows_covered * h_out)


def recorded_traffic(src_hash, workload):
    """HBM bytes per launch measured by the committed counter runs, if they were
    taken on the current kernel sources and this workload."""
    if workload != DEFAULT_WORKLOAD:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def traffic_applies(args) -> bool:
    """The committed counter run was taken on the headline workload's default
    launch (automatic variant and split count, device metadata, rows in segment
    order); other launches run other kernels or plans.  Graph replay launches
    the same kernel."""
    return (args.workload == DEFAULT_WORKLOAD and args.variant == "auto" and args.splits == 0
            and not args.host_meta and args.row_map == "none")


def _bits(t):
    import numpy as np
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# --------------------------------------------------------------------------- layouts

def workload_layout(name):
    """(dtype, h_in, h_out, rank, n_rows, seg_indptr, lora_idx, logical_pool, seed) of a
    single-call workload; segment metadata comes from the workload's definition or from
    the library's segment builder."""
    import numpy as np
    import segmented_gather_matvec_amd as sg
    import workloads as wl
    parts = name.split("_")
    if name.startswith("decode_distinct"):
        # decode_distinct[_qkv]_h{H}_r{r}_b{n}
        if parts[2] == "qkv":
            parts = parts[:2] + parts[3:]
        h, r, n = int(parts[2][1:]), int(parts[3][1:]), int(parts[4][1:])
        return "f16", h, h, r, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32), n, 2
    if parts[0] in ("identical", "uniform", "skewed"):
        # {kind}_b{n}: H=4096, r=16, fp16
        kind, n = parts[0], int(parts[1][1:])
        seed = wl.POPULARITY_SEEDS[(kind, n)]
        ids, pool = wl.draw_ids(np.random.default_rng(seed), kind, n)
        _, seg, lidx, _ = sg.sgmv_build_segments(ids, pool)
        return "f16", 4096, 4096, 16, n, seg, lidx, pool, seed
    if parts[0] == "mixed":
        # mixed_r{r}_{h_in}to{h_out}
        r = int(parts[1][1:])
        h_in, h_out = (int(x) for x in parts[2].split("to"))
        seed = 41 if r == 16 else 42
        seg, ids = wl.mixed_layout(np.random.default_rng(seed))
        return "bf16", h_in, h_out, r, int(seg[-1]), seg, ids, 16, seed
    raise SystemExit(f"unknown workload {name}")


SINGLE_WORKLOADS = (["decode_distinct_h4096_r16_b32", "decode_distinct_h4096_r16_b64"]
                    + [f"decode_distinct_h4096_r16_b{n}" for n in (1, 8, 16, 128, 256, 512)]
                    + ["decode_distinct_h4096_r32_b32", "decode_distinct_h4096_r64_b8",
                       "decode_distinct_h4096_r64_b32", "decode_distinct_h11008_r16_b32"]
                    + ["decode_distinct_qkv_h4096_r16_b32", "decode_distinct_qkv_h4096_r16_b64"]
                    + [f"{k}_b{n}" for k in ("identical", "uniform", "skewed") for n in (32, 64)]
                    + [f"mixed_r{r}_{a}" for r in (16, 64) for a in ("4096to11008", "11008to4096")])
MODEL_WORKLOADS = ["llama13b_r64_b256_forward"]
# Mixed ranks: Distinct decode batch whose LoRAs have ranks 8..64 (compact
# storage, per-LoRA rank table and scales), against the same batch padded to
# rank 64 (decode_distinct_h4096_r64_b32).
HET_WORKLOADS = ["decode_mixedrank_h4096_r64_b32"]
# Base projection with the LoRA term (sgmv_base_lora_apply): Y = X @ W + the
# per-row LoRA term, Distinct decode batches.
# The base_packed_ lines run sgmv_base_lora_apply_packed on W packed once
# beforehand (the packing is not timed: a server packs its weights at load).
BASE_WORKLOADS = ["base_decode_distinct_h4096_r16_b32", "base_decode_distinct_h4096_r16_b8",
                  "base_decode_distinct_h4096_r16_b64", "base_decode_distinct_h11008to4096_r16_b32",
                  "base_decode_distinct_h4096_r16_b128"]
BASE_WORKLOADS += [w.replace("base_", "base_packed_", 1) for w in BASE_WORKLOADS]
# One GPU's shard of a tensor-parallel layer over 8 GPUs (H = 4096): the
# column-parallel shard (W[:, slice], B_k[:, slice]: 4096 -> 512, the ordinary
# call) and the row-parallel shard (W[slice, :], A_k[slice, :]: 512 -> 4096,
# sgmv_base_lora_apply_partial, fp32 partial output for the layer's all-reduce).
BASE_WORKLOADS += ["base_decode_distinct_h4096to512_r16_b32", "base_partial_decode_distinct_h512to4096_r16_b32",
                   "base_packed_decode_distinct_h4096to512_r16_b32"]


class SingleCallBench:
    """One sgmv_lora_apply call per step, weights rotated through a >= 1 GiB pool.
    A "_qkv" workload runs three projections that share X (a layer's query, key and
    value projections, each with its own LoRA pool and output) as one
    sgmv_lora_apply_batched call per step."""

    def __init__(self, name, variant=0, splits=0, row_map="none", host_meta=False):
        import numpy as np
        import torch
        import segmented_gather_matvec_amd as sg
        import workloads as wl

        self.name, self.sg, self.torch = name, sg, torch
        self.row_map = row_map
        self.host_meta = host_meta
        self.nproj = 3 if "_qkv_" in name else 1
        if self.nproj > 1 and row_map != "none":
            raise SystemExit("the projection-batched workloads take rows in segment order only")
        if host_meta and (self.nproj > 1 or row_map != "none"):
            raise SystemExit("--host-meta runs one projection with rows in segment order")
        (self.dtype, self.h_in, self.h_out, self.rank, self.n, seg, lidx, self.lpool,
         seed) = workload_layout(name)
        seg, lidx = np.asarray(seg, np.int32), np.asarray(lidx, np.int32)
        lens = np.diff(seg)
        used = sorted(set(int(k) for k, L in zip(lidx, lens) if L > 0))
        self.seg_h, self.lidx_h = seg, lidx
        self.distinct = len(used)
        self.rows_covered = int(seg[-1])
        e = 2
        lora_bytes = e * (self.h_in * self.rank + self.rank * self.h_out)
        # Physical pool: >= 1 GiB of weights, a multiple of the logical pool.
        self.tables = max(1, min(4096 // self.lpool, math.ceil((1 << 30) / (lora_bytes * self.lpool))))
        self.ppool = self.tables * self.lpool
        xy_bytes = e * self.n * (self.h_in + self.h_out)
        self.copies = max(2, min(64, math.ceil((256 << 20) / xy_bytes)))
        s0 = seed * 1000
        self.X = wl.device_normal((self.copies, self.n, self.h_in), 1.0, self.dtype, s0 + 3)
        dev = "cuda"
        phys = (torch.arange(self.tables, device=dev)[:, None] * self.lpool
                + torch.arange(self.lpool, device=dev)[None, :]).to(torch.int64)
        # one LoRA pool, pointer tables and output per projection
        self.As, self.Bs, self.Ys, self.A_tabs, self.B_tabs = [], [], [], [], []
        for j in range(self.nproj):
            sj = s0 + 10 * j
            A = wl.device_normal((self.ppool, self.h_in, self.rank), self.h_in ** -0.5, self.dtype, sj + 1)
            B = wl.device_normal((self.ppool, self.rank, self.h_out), self.rank ** -0.5, self.dtype, sj + 2)
            Y = wl.device_normal((self.copies, self.n, self.h_out), 1.0, self.dtype, sj + 4)
            self.As.append(A)
            self.Bs.append(B)
            self.Ys.append(Y)
            self.A_tabs.append((A.data_ptr() + phys * (self.h_in * self.rank * e)).contiguous())
            self.B_tabs.append((B.data_ptr() + phys * (self.rank * self.h_out * e)).contiguous())
        self.A, self.B, self.Y = self.As[0], self.Bs[0], self.Ys[0]
        self.A_tab, self.B_tab = self.A_tabs[0], self.B_tabs[0]
        self.seg = torch.from_numpy(seg).to(dev)
        self.lidx = torch.from_numpy(lidx if lidx.size else np.zeros(1, np.int32)).to(dev)
        self.problem = sg.make_problem(self.dtype, self.n, self.h_in, self.h_out, self.rank, self.lpool,
                                       len(lidx), int(lens.max()) if lens.size else 0, variant, splits)
        self.ws = torch.zeros(sg.batched_workspace_bytes(self.problem, self.nproj), dtype=torch.uint8,
                              device=dev)
        # X is read once for all projections; each projection streams its own
        # LoRAs and reads and writes its own Y.
        self.bytes = (algorithmic_bytes(e, self.rows_covered, self.h_in, self.h_out, self.rank, self.distinct)
                      + (self.nproj - 1) * (algorithmic_bytes(e, self.rows_covered, self.h_in, self.h_out,
                                                              self.rank, self.distinct)
                                            - e * self.rows_covered * self.h_in))
        self.rows_per_step = self.rows_covered
        self.calls_per_step = 1
        # Row layout of X and Y.  "none": rows in segment order.  Otherwise rows
        # are in request order, with request perm[j] at sorted row j (a seeded
        # shuffle), and either the kernels gather / scatter them through the row
        # map ("kernel") or the caller permutes around the call ("torch").
        self.perm_h = (np.random.default_rng(seed + 7).permutation(self.n).astype(np.int32)
                       if row_map != "none" else np.arange(self.n, dtype=np.int32))
        self.perm = torch.from_numpy(self.perm_h).to(dev)
        self.perm64 = self.perm.to(torch.int64)
        lib = sg.load_library()
        self.fn, self.fn_batched = lib.sgmv_lora_apply, lib.sgmv_lora_apply_batched
        if host_meta:
            # sgmv_lora_apply_host_meta: metadata and pointer tables from host memory
            self.fn = lib.sgmv_lora_apply_host_meta
            self.A_tab_h = [np.ascontiguousarray(tab.cpu().numpy().astype(np.uint64)) for tab in self.A_tab]
            self.B_tab_h = [np.ascontiguousarray(tab.cpu().numpy().astype(np.uint64)) for tab in self.B_tab]
            self.seg_hc = np.ascontiguousarray(seg, np.int32)
            self.lidx_hc = np.ascontiguousarray(lidx if lidx.size else np.zeros(1, np.int32), np.int32)
        if row_map == "torch":
            # X and Y gathered into segment order around each call
            self.X_sorted = torch.empty_like(self.X[0])
            self.Y_sorted = torch.empty_like(self.Y[0])
        self.marshal()
        torch.cuda.synchronize()

    def marshal(self):
        pb = ctypes.byref(self.problem)
        wsn = self.ws.numel()
        self.args, self.keep = [], []
        for c in range(max(self.tables, self.copies)):
            t, x = c % self.tables, c % self.copies
            if self.nproj > 1:
                pj = (self.sg.sgmv_projection_t * self.nproj)(
                    *[self.sg.sgmv_projection_t(self.A_tabs[j][t].data_ptr(), self.B_tabs[j][t].data_ptr(),
                                                self.Ys[j][x].data_ptr()) for j in range(self.nproj)])
                self.keep.append(pj)
                self.args.append((pb, self.X[x].data_ptr(), pj, self.nproj, self.seg.data_ptr(),
                                  self.lidx.data_ptr(), None, self.ws.data_ptr(), wsn))
            elif self.row_map == "kernel":
                pj = (self.sg.sgmv_projection_t * 1)(
                    self.sg.sgmv_projection_t(self.A_tab[t].data_ptr(), self.B_tab[t].data_ptr(),
                                              self.Y[x].data_ptr()))
                self.keep.append(pj)
                self.args.append((pb, self.X[x].data_ptr(), pj, 1, self.seg.data_ptr(), self.lidx.data_ptr(),
                                  self.perm.data_ptr(), self.ws.data_ptr(), wsn))
            elif self.row_map == "torch":
                self.args.append((pb, self.X_sorted.data_ptr(), self.A_tab[t].data_ptr(), self.B_tab[t].data_ptr(),
                                  self.Y_sorted.data_ptr(), self.seg.data_ptr(), self.lidx.data_ptr(),
                                  self.ws.data_ptr(), wsn))
            elif self.host_meta:
                self.args.append((pb, self.X[x].data_ptr(), self.A_tab_h[t].ctypes.data,
                                  self.B_tab_h[t].ctypes.data, self.Y[x].data_ptr(), self.seg_hc.ctypes.data,
                                  self.lidx_hc.ctypes.data, self.ws.data_ptr(), wsn))
            else:
                self.args.append((pb, self.X[x].data_ptr(), self.A_tab[t].data_ptr(), self.B_tab[t].data_ptr(),
                                  self.Y[x].data_ptr(), self.seg.data_ptr(), self.lidx.data_ptr(),
                                  self.ws.data_ptr(), wsn))

    def step(self, c, stream):
        i = c % len(self.args)
        if self.row_map == "kernel" or self.nproj > 1:
            st = self.fn_batched(*self.args[i], stream)
        elif self.row_map == "torch":
            # The caller's alternative to the row map: gather X and Y into
            # segment order, apply, scatter Y back (torch ops on the same stream).
            x = i % self.copies
            torch = self.torch
            torch.index_select(self.X[x], 0, self.perm64, out=self.X_sorted)
            torch.index_select(self.Y[x], 0, self.perm64, out=self.Y_sorted)
            st = self.fn(*self.args[i], stream)
            self.Y[x].index_copy_(0, self.perm64, self.Y_sorted)
        else:
            st = self.fn(*self.args[i], stream)
        if st != 0:
            raise RuntimeError(self.sg.sgmv_status_str(st))

    def check_sample(self, calls=2, max_rows=64):
        """Parity of the timed launch configuration on sampled calls (oracle, fp64)."""
        import numpy as np
        import oracle
        torch = self.torch
        worst = 0.0
        sid = torch.cuda.current_stream().cuda_stream
        for c in range(calls):
            t, x = c % self.tables, c % self.copies
            Xh = _bits(self.X[x])[self.perm_h]
            Y0 = [_bits(Y[x])[self.perm_h] for Y in self.Ys]
            A = [[_bits(As[t * self.lpool + k]) for k in range(self.lpool)] for As in self.As]
            B = [[_bits(Bs[t * self.lpool + k]) for k in range(self.lpool)] for Bs in self.Bs]
            mask = None
            if self.n > max_rows:
                rows = set(np.random.default_rng(c).choice(self.n, 16, replace=False).tolist())
                for s in range(len(self.seg_h) - 1):
                    if self.seg_h[s + 1] > self.seg_h[s]:
                        rows.update((int(self.seg_h[s]), int(self.seg_h[s + 1]) - 1))
                mask = np.zeros(self.n, np.uint8)
                mask[sorted(rows)] = 1
            self.step(c, sid)
            torch.cuda.synchronize()
            for j in range(self.nproj):
                got = oracle.decode(_bits(self.Ys[j][x])[self.perm_h], self.dtype)
                ref = oracle.sgmv_apply(self.dtype, Xh, A[j], B[j], self.seg_h, self.lidx_h, Y0[j],
                                        row_mask=mask)
                sel = slice(None) if mask is None else mask.astype(bool)
                ratio = np.abs(got[sel] - ref[sel]) / (1e-3 + 1e-2 * np.abs(ref[sel]))
                worst = max(worst, float(ratio.max()))
        if worst > 1.0:
            raise AssertionError(f"bench parity check failed: max err/bound {worst:.3f}")
        return worst

    def config(self):
        return {"workload": self.name, "h_in": self.h_in, "h_out": self.h_out, "rank": self.rank,
                "projections": self.nproj,
                "batch_rows": self.n, "segments": int(len(self.lidx_h)), "distinct_loras": self.distinct,
                "lora_pool": self.lpool, "physical_lora_pool": self.ppool, "xy_copies": self.copies,
                "row_layout": {"none": "segment order", "kernel": "request order, kernel row map",
                               "torch": "request order, torch gather/scatter"}[self.row_map],
                "algorithmic_bytes_per_step": self.bytes,
                "entry_point": "sgmv_lora_apply_host_meta" if self.host_meta else
                               ("sgmv_lora_apply_batched" if self.nproj > 1 or self.row_map == "kernel"
                                else "sgmv_lora_apply"),
                "plan": self.sg.sgmv_query_plan(self.problem).as_dict()}


class MixedRankBench:
    """One sgmv_lora_apply_batched call per step over a Distinct decode batch
    (H1 = H2 = 4096, 32 fp16 rows, 32 LoRAs) whose LoRAs keep their own ranks,
    drawn from {8, 16, 32, 64} (compact storage: A_k [4096, r_k], B_k [r_k, 4096]),
    each with its own scale.  The largest rank (64) sets the compiled tile; the
    kernels read only r_k ranks of each LoRA.  Weights rotate through a >= 1 GiB
    pool and X / Y through copies, as in the other workloads."""

    def __init__(self, name, variant=0, splits=0):
        import numpy as np
        import torch
        import segmented_gather_matvec_amd as sg
        import workloads as wl

        self.name, self.sg, self.torch = name, sg, torch
        self.dtype, self.h_in, self.h_out, self.R, self.n = "f16", 4096, 4096, 64, 32
        rng = np.random.default_rng(61)
        self.ranks_h = rng.choice([8, 16, 32, 64], self.n).astype(np.int32)
        self.scales_h = rng.uniform(0.5, 2.0, self.n).astype(np.float32)
        e = 2
        lora_elems = (self.h_in + self.h_out) * self.ranks_h.astype(np.int64)
        per_table = int(lora_elems.sum()) * e
        self.tables = max(1, math.ceil((1 << 30) / per_table))
        self.copies = 64
        # one flat buffer per table: LoRA k's A_k then B_k, compact
        offs = np.concatenate([[0], np.cumsum(lora_elems)])[:-1]
        self.W = wl.device_normal((self.tables, int(lora_elems.sum())), 1.0, self.dtype, 6100)
        # scale each LoRA's values to a unit-variance term: A by h_in^-1/2, B by r^-1/2
        for k in range(self.n):
            r, o = int(self.ranks_h[k]), int(offs[k])
            self.W[:, o: o + self.h_in * r].mul_(self.h_in ** -0.5)
            self.W[:, o + self.h_in * r: o + (self.h_in + self.h_out) * r].mul_(r ** -0.5)
        base = self.W.data_ptr() + torch.arange(self.tables, dtype=torch.int64, device="cuda")[:, None] \
            * (int(lora_elems.sum()) * e)
        a_off = torch.from_numpy(offs * e).cuda()
        b_off = torch.from_numpy((offs + self.h_in * self.ranks_h.astype(np.int64)) * e).cuda()
        self.A_tab = (base + a_off[None, :]).contiguous()
        self.B_tab = (base + b_off[None, :]).contiguous()
        self.offs = offs
        self.X = wl.device_normal((self.copies, self.n, self.h_in), 1.0, self.dtype, 6101)
        self.Y = wl.device_normal((self.copies, self.n, self.h_out), 1.0, self.dtype, 6102)
        self.seg_h = np.arange(self.n + 1, dtype=np.int32)
        self.lidx_h = np.arange(self.n, dtype=np.int32)
        self.seg = torch.from_numpy(self.seg_h).cuda()
        self.lidx = torch.from_numpy(self.lidx_h).cuda()
        self.ranks = torch.from_numpy(self.ranks_h).cuda()
        self.scales = torch.from_numpy(self.scales_h).cuda()
        self.problem = sg.make_problem(self.dtype, self.n, self.h_in, self.h_out, self.R, self.n, self.n, 1,
                                       variant, splits)
        self.ws = sg.new_workspace(self.problem)
        self.bytes = e * (int(lora_elems.sum()) + self.n * self.h_in + 2 * self.n * self.h_out)
        self.rows_per_step = self.n
        self.calls_per_step = 1
        self.fn = sg.load_library().sgmv_lora_apply_batched
        pb = ctypes.byref(self.problem)
        self.args, self.keep = [], []
        for c in range(max(self.tables, self.copies)):
            t, x = c % self.tables, c % self.copies
            pj = (sg.sgmv_projection_t * 1)(sg.sgmv_projection_t(
                self.A_tab[t].data_ptr(), self.B_tab[t].data_ptr(), self.Y[x].data_ptr(),
                self.ranks.data_ptr(), self.scales.data_ptr()))
            self.keep.append(pj)
            self.args.append((pb, self.X[x].data_ptr(), pj, 1, self.seg.data_ptr(), self.lidx.data_ptr(), None,
                              self.ws.data_ptr(), self.ws.numel()))
        torch.cuda.synchronize()

    def step(self, c, stream):
        st = self.fn(*self.args[c % len(self.args)], stream)
        if st != 0:
            raise RuntimeError(self.sg.sgmv_status_str(st))

    def check_sample(self, calls=2):
        import numpy as np
        import oracle
        torch = self.torch
        worst = 0.0
        sid = torch.cuda.current_stream().cuda_stream
        for c in range(calls):
            t, x = c % self.tables, c % self.copies
            Xh, Y0 = _bits(self.X[x]), _bits(self.Y[x])
            Wt = _bits(self.W[t])
            A, B = [], []
            for k in range(self.n):
                r, o = int(self.ranks_h[k]), int(self.offs[k])
                A.append(Wt[o: o + self.h_in * r].reshape(self.h_in, r))
                B.append(Wt[o + self.h_in * r: o + (self.h_in + self.h_out) * r].reshape(r, self.h_out))
            self.step(c, sid)
            torch.cuda.synchronize()
            got = oracle.decode(_bits(self.Y[x]), self.dtype)
            ref = oracle.sgmv_apply(self.dtype, Xh, A, B, self.seg_h, self.lidx_h, Y0, scales=self.scales_h,
                                    rank=self.R)
            worst = max(worst, float((np.abs(got - ref) / (1e-3 + 1e-2 * np.abs(ref))).max()))
        if worst > 1.0:
            raise AssertionError(f"bench parity check failed: max err/bound {worst:.3f}")
        return worst

    def config(self):
        return {"workload": self.name, "h_in": self.h_in, "h_out": self.h_out, "max_rank": self.R,
                "ranks": self.ranks_h.tolist(), "scaled": True, "batch_rows": self.n, "segments": self.n,
                "distinct_loras": self.n, "physical_tables": self.tables, "xy_copies": self.copies,
                "algorithmic_bytes_per_step": self.bytes}


class ModelForwardBench:
    """All 280 LoRA calls of one 13B forward (40 layers x q,k,v,o,gate,up,down), r=64,
    bf16, 64 LoRAs per projection, batch 256 with Zipf(1.5) LoRA assignment."""

    dtype = "bf16"

    def __init__(self, name, variant=0, splits=0, layers=None, batch_projections=True, row_map="none"):
        import numpy as np
        import torch
        import segmented_gather_matvec_amd as sg
        import workloads as wl

        self.name, self.sg, self.torch = name, sg, torch
        self.n, self.rank, self.P = 256, 64, 64
        self.layers = layers or wl.LLAMA13B_LAYERS
        ids = wl.full_model_ids(seed=5, n=self.n, pool=self.P)
        perm, seg, lidx, mx = sg.sgmv_build_segments(ids, self.P)
        self.seg_h, self.lidx_h = seg, lidx
        # "none": activations in segment order.  "kernel" / "torch": in request
        # order (request perm[j] at sorted row j, the builder's output), gathered
        # and scattered by the kernels' row map or by torch around each call.
        self.row_map = row_map
        self.perm_h = perm if row_map != "none" else np.arange(self.n, dtype=np.int32)
        self.perm = torch.from_numpy(np.ascontiguousarray(self.perm_h)).to("cuda")
        self.perm64 = self.perm.to(torch.int64)
        self.distinct = len(lidx)
        self.seg = torch.from_numpy(seg).to("cuda")
        self.lidx = torch.from_numpy(lidx).to("cuda")
        lib = sg.load_library()
        self.fn = lib.sgmv_lora_apply
        self.fn_batched = lib.sgmv_lora_apply_batched
        self.batch_projections = batch_projections
        self.calls, self.keep, total = [], [], 0
        self.launch_groups = []  # per layer: lists of projection indices issued as one call
        probs = {}
        for (_, h_in, h_out) in wl.LLAMA13B_PROJ:
            if (h_in, h_out) not in probs:
                probs[(h_in, h_out)] = sg.make_problem("bf16", self.n, h_in, h_out, self.rank, self.P,
                                                        len(lidx), mx, variant, splits)
        self.probs = probs
        ws_bytes = max(sg.batched_workspace_bytes(p, 3) for p in probs.values())
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        for layer in range(self.layers):
            xs = {"qkv": wl.device_normal((self.n, 5120), 1.0, "bf16", 900000 + 4 * layer),
                  "o": wl.device_normal((self.n, 5120), 1.0, "bf16", 900001 + 4 * layer),
                  "gu": wl.device_normal((self.n, 5120), 1.0, "bf16", 900002 + 4 * layer),
                  "down": wl.device_normal((self.n, 13824), 1.0, "bf16", 900003 + 4 * layer)}
            for proj, (pname, h_in, h_out) in enumerate(wl.LLAMA13B_PROJ):
                seed = wl.full_model_weight_seed(layer, proj)
                A = wl.device_normal((self.P, h_in, self.rank), h_in ** -0.5, "bf16", seed * 2)
                B = wl.device_normal((self.P, self.rank, h_out), self.rank ** -0.5, "bf16", seed * 2 + 1)
                Y = wl.device_normal((self.n, h_out), 1.0, "bf16", 950000 + 7 * layer + proj)
                group = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gu", "up": "gu",
                         "down": "down"}[pname]
                X = xs[group]
                At, Bt = sg.pointer_table(A), sg.pointer_table(B)
                self.keep.append((A, B, Y, X, At, Bt))
                pb = probs[(h_in, h_out)]
                self.calls.append((ctypes.byref(pb), X.data_ptr(), At.data_ptr(), Bt.data_ptr(), Y.data_ptr(),
                                   self.seg.data_ptr(), self.lidx.data_ptr(), self.ws.data_ptr(),
                                   self.ws.numel()))
                total += algorithmic_bytes(2, self.n, h_in, h_out, self.rank, self.distinct)
        # Projections that read the same input (q, k, v; gate, up) run as one
        # batched call unless asked otherwise.
        names = [pn for (pn, _, _) in wl.LLAMA13B_PROJ]
        groups = ([[names.index(g) for g in grp] for grp in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))]
                  if batch_projections else [[i] for i in range(len(names))])
        self.batched, self.group_idx = [], []
        self.group_names = ",".join("".join(names[j] for j in grp) for grp in groups)
        for layer in range(self.layers):
            for grp in groups:
                idx = [layer * len(names) + j for j in grp]
                self.group_idx.append(idx)
                if len(idx) == 1 and row_map != "kernel":
                    self.batched.append(("single", self.calls[idx[0]]))
                else:
                    first = self.calls[idx[0]]
                    arr = (sg.sgmv_projection_t * len(idx))(
                        *[sg.sgmv_projection_t(self.calls[c][2], self.calls[c][3], self.calls[c][4]) for c in idx])
                    self.keep.append(arr)
                    self.batched.append(("batched", (first[0], first[1], arr, len(idx), first[5], first[6],
                                                     self.perm.data_ptr() if row_map == "kernel" else None,
                                                     first[7], first[8])))
        if row_map == "torch":
            # Segment-order staging buffers: one X per input group and one Y
            # per projection of the largest group, reused by every call.
            self.stage_x = {w: torch.empty((self.n, w), dtype=torch.bfloat16, device="cuda")
                            for w in (5120, 13824)}
            maxh = max(h for (_, _, h) in wl.LLAMA13B_PROJ)
            self.stage_y = [torch.empty(self.n * maxh, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
            self.torch_calls = []
            for g, (kind, args) in enumerate(self.batched):
                idx = self.group_idx[g]
                X = self.keep[idx[0]][3]
                xs = self.stage_x[X.shape[1]]
                ys = [self.stage_y[j][: self.n * self.keep[c][2].shape[1]].view(self.n, -1)
                      for j, c in enumerate(idx)]
                pj = (sg.sgmv_projection_t * len(idx))(
                    *[sg.sgmv_projection_t(self.calls[c][2], self.calls[c][3], ys[j].data_ptr())
                      for j, c in enumerate(idx)])
                self.keep.append(pj)
                first = self.calls[idx[0]]
                self.torch_calls.append((X, xs, [self.keep[c][2] for c in idx], ys,
                                         (first[0], xs.data_ptr(), pj, len(idx), first[5], first[6], None,
                                          first[7], first[8])))
        self.bytes = total
        self.rows_per_step = self.n
        self.calls_per_step = len(self.batched)
        torch.cuda.synchronize()

    def run_group(self, g, stream):
        if self.row_map == "torch":
            torch = self.torch
            X, xs, Ys, ys, args = self.torch_calls[g]
            torch.index_select(X, 0, self.perm64, out=xs)
            for Y, y in zip(Ys, ys):
                torch.index_select(Y, 0, self.perm64, out=y)
            st = self.fn_batched(*args, stream)
            for Y, y in zip(Ys, ys):
                Y.index_copy_(0, self.perm64, y)
        else:
            kind, args = self.batched[g]
            st = self.fn(*args, stream) if kind == "single" else self.fn_batched(*args, stream)
        if st != 0:
            raise RuntimeError(self.sg.sgmv_status_str(st))

    def step(self, c, stream):
        for g in range(len(self.batched)):
            self.run_group(g, stream)

    def check_sample(self, rows=16):
        """The first and the last call of a forward (layer 0's first projection group,
        the last layer's down projection), every projection in them against the
        oracle on sampled rows."""
        import numpy as np
        import oracle
        torch = self.torch
        sid = torch.cuda.current_stream().cuda_stream
        used = set(int(k) for k in self.lidx_h)
        worst = 0.0
        for g in (0, len(self.batched) - 1):
            snaps = []
            for idx in self.group_idx[g]:
                A, B, Y, X, _, _ = self.keep[idx]
                snaps.append((Y, _bits(X)[self.perm_h], _bits(Y)[self.perm_h],
                              [_bits(A[k]) if k in used else np.zeros((1, 1), np.uint16) for k in range(self.P)],
                              [_bits(B[k]) if k in used else np.zeros((1, 1), np.uint16) for k in range(self.P)]))
            self.run_group(g, sid)
            torch.cuda.synchronize()
            mask = np.zeros(self.n, np.uint8)
            mask[np.random.default_rng(g).choice(self.n, rows, replace=False)] = 1
            mask[[0, self.n - 1]] = 1
            sel = mask.astype(bool)
            for Y, Xh, Y0, Ah, Bh in snaps:
                got = oracle.decode(_bits(Y)[self.perm_h], "bf16")
                ref = oracle.sgmv_apply("bf16", Xh, Ah, Bh, self.seg_h, self.lidx_h, Y0, row_mask=mask)
                worst = max(worst, float((np.abs(got[sel] - ref[sel]) / (1e-3 + 1e-2 * np.abs(ref[sel]))).max()))
        if worst > 1.0:
            raise AssertionError(f"bench parity check failed: max err/bound {worst:.3f}")
        return worst

    def config(self):
        return {"workload": self.name, "layers": self.layers, "projections": "q,k,v,o,gate,up,down",
                "rank": self.rank, "batch_rows": self.n, "segments": self.distinct,
                "distinct_loras": self.distinct, "lora_pool": self.P, "projection_calls": len(self.calls),
                "calls_per_step": len(self.batched), "calls_per_layer": self.group_names,
                "row_layout": {"none": "segment order", "kernel": "request order, kernel row map",
                               "torch": "request order, torch gather/scatter"}[self.row_map],
                "algorithmic_bytes_per_step": self.bytes,
                "plans": {f"{h_in}to{h_out}": self.sg.sgmv_query_plan(prob).as_dict()
                          for (h_in, h_out), prob in self.probs.items()}}


def latency_curve(batches=(1, 2, 4, 8, 16, 32, 64), steps=200, warmup=20):
    """Latency of the LoRA addend against batch size, the micro-benchmark of the
    Punica README (page "Punica：多 LoRA 模型统一服务框架", micro-benchmark
    paragraph): the base projection X@W keeps its batching effect, a naive LoRA
    implementation does not, SGMV does.  Shape of the headline workload
    (H1 = H2 = 4096, r = 16, fp16, Distinct: every row its own LoRA).

    Per batch size n, one call of each:
      base_gemm   torch.matmul(X, W), W [4096, 4096] (context: the base layer)
      sgmv        sgmv_lora_apply (this library)
      loop        naive LoRA, one (x_i @ A_k) @ B_k pair of torch matmuls per segment
      gather_bmm  naive LoRA, A_k / B_k gathered per row, then two torch.bmm
    Each is timed eagerly (<name>_us: wall time per call, host launch costs
    included) and as 16 calls replayed from a captured HIP graph
    (<name>_graph_us: device time per call).
    Weights come from a 1 GiB pool (W from 16 copies) rotated per call, as in
    the other workloads.  Every method's output is checked against the fp64
    oracle on the first call (max |err| / (1e-3 + 1e-2 |ref|), reported; the
    torch baselines round V to fp16 and may exceed 1)."""
    import numpy as np
    import torch
    import oracle
    import segmented_gather_matvec_amd as sg
    import workloads as wl

    H, r, P, dt = 4096, 16, 4096, torch.float16
    A = wl.device_normal((P, H, r), H ** -0.5, "f16", 7001)
    B = wl.device_normal((P, r, H), r ** -0.5, "f16", 7002)
    Ws = wl.device_normal((16, H, H), H ** -0.5, "f16", 7003)
    lib = sg.load_library()
    curve = []
    for n in batches:
        X = wl.device_normal((16, n, H), 1.0, "f16", 7100 + n)
        Y = wl.device_normal((16, n, H), 1.0, "f16", 7200 + n)
        out = torch.empty((n, H), dtype=dt, device="cuda")
        tables = P // n
        phys = torch.arange(tables * n, device="cuda", dtype=torch.int64).view(tables, n)
        A_tab = (A.data_ptr() + phys * (H * r * 2)).contiguous()
        B_tab = (B.data_ptr() + phys * (r * H * 2)).contiguous()
        seg = torch.arange(n + 1, dtype=torch.int32, device="cuda")
        lidx = torch.arange(n, dtype=torch.int32, device="cuda")
        prob = sg.make_problem("f16", n, H, H, r, n, n, 1)
        ws = sg.new_workspace(prob)
        pb = ctypes.byref(prob)

        def base_gemm(c):
            torch.matmul(X[c % 16], Ws[c % 16], out=out)

        sgmv_args = [(pb, X[c % 16].data_ptr(), A_tab[c % tables].data_ptr(), B_tab[c % tables].data_ptr(),
                      Y[c % 16].data_ptr(), seg.data_ptr(), lidx.data_ptr(), ws.data_ptr(), ws.numel())
                     for c in range(max(tables, 16))]

        def sgmv(c):
            st = lib.sgmv_lora_apply(*sgmv_args[c % len(sgmv_args)], torch.cuda.current_stream().cuda_stream)
            if st != 0:
                raise RuntimeError(sg.sgmv_status_str(st))

        def loop(c):
            t, x, y = c % tables, X[c % 16], Y[c % 16]
            for i in range(n):
                k = t * n + i
                y[i:i + 1].addmm_(torch.mm(x[i:i + 1], A[k]), B[k])

        def gather_bmm(c):
            t, x, y = c % tables, X[c % 16], Y[c % 16]
            idx = phys[t]
            v = torch.bmm(x[:, None, :], A.index_select(0, idx))
            y += torch.bmm(v, B.index_select(0, idx))[:, 0, :]

        methods = {"base_gemm": base_gemm, "sgmv": sgmv, "loop": loop, "gather_bmm": gather_bmm}
        row = {"batch": n}
        # Parity of each LoRA method on call 0 against the oracle (host copies
        # taken before the call; Y restored afterwards).
        Xh = _bits(X[0])
        Ah = [_bits(A[k]) for k in range(n)]
        Bh = [_bits(B[k]) for k in range(n)]
        for name in ("sgmv", "loop", "gather_bmm"):
            y0 = Y[0].clone()
            ref = oracle.sgmv_apply("f16", Xh, Ah, Bh, np.arange(n + 1, dtype=np.int32),
                                    np.arange(n, dtype=np.int32), _bits(y0))
            methods[name](0)
            torch.cuda.synchronize()
            got = oracle.decode(_bits(Y[0]), "f16")
            row[name + "_err_over_bound"] = round(float((np.abs(got - ref) / (1e-3 + 1e-2 * np.abs(ref))).max()), 4)
            Y[0].copy_(y0)
        if row["sgmv_err_over_bound"] > 1.0:
            raise AssertionError(f"sgmv parity failed at batch {n}: {row['sgmv_err_over_bound']}")
        for name, fn in methods.items():
            # Eager: what a Python caller sees, host launch costs included.
            for c in range(warmup):
                fn(c)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for c in range(steps):
                fn(c)
            torch.cuda.synchronize()
            row[name + "_us"] = round((time.perf_counter() - t0) / steps * 1e6, 3)
            # Device time: 16 calls (distinct weights) captured in a HIP graph
            # and replayed, which takes the host out.
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(16):
                    fn(c)
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, steps // 16)
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            row[name + "_graph_us"] = round((time.perf_counter() - t0) / (reps * 16) * 1e6, 3)
            del g
        curve.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del X, Y, out, A_tab, B_tab, ws
    return {"metric": "LoRA addend latency vs batch size: SGMV against naive LoRA (base X@W for context)",
            "unit": "us", "higher_is_better": False, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "latency_curve_h4096_r16_distinct", "h_in": H, "h_out": H, "rank": r,
                       "lora_pool": P, "steps": steps, "warmup": warmup},
            "curve": curve}


def base_rows_curve(batches=(8, 16, 32, 64, 128, 256, 512, 1024), steps=160):
    """The base projection with the LoRA term, Y = X @ W + (X @ A_k) @ B_k, against
    the number of rows (Punica README, page "Punica：多 LoRA 模型统一服务框架",
    LoRA and multi-LoRA paragraphs).  H1 = H2 = 4096, r = 16, fp16, Distinct
    LoRAs (every row its own).  Per batch size n, device time per call from 16
    calls replayed out of a captured HIP graph (weights rotate through >= 1 GiB):
      torch_gemm_us            torch.matmul(X, W) written to Y (the base layer alone)
      torch_gemm_plus_sgmv_us  that GEMM, then sgmv_lora_apply adding the LoRA term
      fused_us                 sgmv_base_lora_apply (n <= SGMV_BASE_MAX_ROWS only), one rounding
      fused_packed_us          sgmv_base_lora_apply_packed on W packed beforehand
    with the HBM floor of streaming W once (w_floor_us, 8 TB/s) and the matrix-core
    floor of the GEMM's flops (gemm_flop_floor_us, 2.5 PFLOP/s fp16)."""
    import torch
    import segmented_gather_matvec_amd as sg
    import workloads as wl

    H, r = 4096, 16
    Ws = wl.device_normal((16, H, H), H ** -0.5, "f16", 7301)
    Wps = [sg.pack_base_weight(Ws[i]) for i in range(16)]
    lib = sg.load_library()
    sid = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    curve = []
    for n in batches:
        P = max(n, 64) * 4
        A = wl.device_normal((P, H, r), H ** -0.5, "f16", 7400 + n)
        B = wl.device_normal((P, r, H), r ** -0.5, "f16", 7500 + n)
        X = wl.device_normal((16, n, H), 1.0, "f16", 7600 + n)
        Y = torch.zeros((16, n, H), dtype=torch.float16, device="cuda")
        tables = P // n
        phys = torch.arange(tables * n, device="cuda", dtype=torch.int64).view(tables, n)
        A_tab = (A.data_ptr() + phys * (H * r * 2)).contiguous()
        B_tab = (B.data_ptr() + phys * (r * H * 2)).contiguous()
        seg = torch.arange(n + 1, dtype=torch.int32, device="cuda")
        lidx = torch.arange(n, dtype=torch.int32, device="cuda")
        prob = sg.make_problem("f16", n, H, H, r, n, n, 1)
        ws = sg.new_workspace(prob)
        bws = sg.new_base_workspace(prob) if n <= sg.SGMV_BASE_MAX_ROWS else None
        pb = ctypes.byref(prob)

        def gemm(c):
            torch.matmul(X[c % 16], Ws[c % 16], out=Y[c % 16])

        def gemm_sgmv(c):
            gemm(c)
            st = lib.sgmv_lora_apply(pb, X[c % 16].data_ptr(), A_tab[c % tables].data_ptr(),
                                     B_tab[c % tables].data_ptr(), Y[c % 16].data_ptr(), seg.data_ptr(),
                                     lidx.data_ptr(), ws.data_ptr(), ws.numel(), sid())
            if st != 0:
                raise RuntimeError(sg.sgmv_status_str(st))

        def fused_with(fn, W):
            def run(c):
                st = fn(pb, X[c % 16].data_ptr(), W[c % 16].data_ptr(), A_tab[c % tables].data_ptr(),
                        B_tab[c % tables].data_ptr(), Y[c % 16].data_ptr(), seg.data_ptr(), lidx.data_ptr(),
                        bws.data_ptr(), bws.numel(), sid())
                if st != 0:
                    raise RuntimeError(sg.sgmv_status_str(st))
            return run

        methods = {"torch_gemm": gemm, "torch_gemm_plus_sgmv": gemm_sgmv}
        if n <= sg.SGMV_BASE_MAX_ROWS:
            methods["fused"] = fused_with(lib.sgmv_base_lora_apply, Ws)
            methods["fused_packed"] = fused_with(lib.sgmv_base_lora_apply_packed, Wps)
        row = {"rows": n, "w_floor_us": round(2 * H * H / 8e12 * 1e6, 3),
               "gemm_flop_floor_us": round(2 * n * H * H / 2.5e15 * 1e6, 3)}
        for name, fn in methods.items():
            for c in range(16):
                fn(c)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(16):
                    fn(c)
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, steps // 16)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            row[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / (reps * 16), 3)
            del g
        for name in ("fused", "fused_packed"):
            row.setdefault(name + "_us", None)
        curve.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del A, B, X, Y, A_tab, B_tab, ws, bws
    return {"metric": "base projection with the LoRA term: fused call vs torch GEMM + SGMV, device time per call",
            "unit": "us", "higher_is_better": False, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "base_rows_curve_h4096_r16_distinct", "h_in": H, "h_out": H, "rank": r,
                       "steps": steps},
            "curve": curve}


def preroll_cycles(stream, target_us=200.0):
    """Cycle count for torch's sleep kernel that keeps the stream busy for
    about target_us, from one timed calibration launch after an untimed one
    (the first launch also loads the kernel's code, about 1 ms); bounded so a
    clock that reads slower than expected still gives a finite pre-roll."""
    import torch
    probe = 100000
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(probe)
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(probe)
    b.record(stream)
    torch.cuda.synchronize()
    us = max(a.elapsed_time(b) * 1e3, 1.0)
    return int(min(probe * target_us / us, 20 * probe))


def cpu_baseline(seconds=10.0, threads=0):
    """The oracle as it stands, on a host copy of the headline workload's shape
    (threads: 0 = every host core OpenMP offers)."""
    import oracle
    import workloads
    w = workloads.decode_distinct()
    threads = threads if threads > 0 else oracle.max_threads()
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.sgmv_apply("f16", w.X, w.A, w.B, w.seg_indptr, w.lora_idx, w.Y0, nthreads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds or calls >= 10000:
            break
    per_call = el / calls
    nbytes = algorithmic_bytes(2, w.n_rows, w.h_in, w.h_out, w.rank, w.num_loras)
    return {"value": round(nbytes / per_call / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{calls} oracle calls on one decode batch (32 rows, H1=H2=4096, r=16, "
                       f"32 LoRAs, fp16 inputs, fp64 arithmetic) in {el:.1f} s; "
                       f"{per_call * 1e3:.2f} ms/call, {w.n_rows / per_call:.0f} rows/s")}


class BaseBench:
    """One sgmv_base_lora_apply call per step: Y = X @ W + (X @ A_k) @ B_k for a
    Distinct decode batch (row i -> LoRA i), fp16.  "base_partial_" workloads
    run sgmv_base_lora_apply_partial instead: the same product written as an
    unrounded fp32 partial, one shard of a row-parallel layer.  W rotates through >= 1 GiB of
    copies, the LoRAs through a >= 1 GiB pool and X / Y through 64 copies, so no
    step finds its weights in the 256 MB Infinity Cache.  For context the config
    also carries the unfused composition on the same buffers: torch's X @ W
    (written to Y), then sgmv_lora_apply adding the LoRA term (two roundings)."""

    def __init__(self, name):
        import re
        import torch
        import numpy as np
        import segmented_gather_matvec_amd as sg
        import workloads as wl

        m = re.fullmatch(r"base_(packed_|partial_)?decode_distinct_h(\d+)(?:to(\d+))?_r(\d+)_b(\d+)", name)
        if not m:
            raise SystemExit(f"unknown workload {name}")
        self.packed = m.group(1) == "packed_"
        self.partial = m.group(1) == "partial_"
        self.name, self.sg, self.torch = name, sg, torch
        self.dtype = "f16"
        self.h_in = int(m.group(2))
        self.h_out = int(m.group(3) or m.group(2))
        self.rank, self.n = int(m.group(4)), int(m.group(5))
        e = 2
        w_bytes = e * self.h_in * self.h_out
        self.wcopies = max(2, math.ceil((1 << 30) / w_bytes))
        lora_bytes = e * (self.h_in + self.h_out) * self.rank
        self.tables = max(2, math.ceil((1 << 30) / (lora_bytes * self.n)))
        self.copies = 64
        s0 = 7000 + self.n
        self.W = wl.device_normal((self.wcopies, self.h_in, self.h_out), self.h_in ** -0.5, self.dtype, s0)
        self.A = wl.device_normal((self.tables * self.n, self.h_in, self.rank), self.h_in ** -0.5, self.dtype,
                                  s0 + 1)
        self.B = wl.device_normal((self.tables * self.n, self.rank, self.h_out), self.rank ** -0.5, self.dtype,
                                  s0 + 2)
        self.X = wl.device_normal((self.copies, self.n, self.h_in), 1.0, self.dtype, s0 + 3)
        self.Y = torch.zeros((self.copies, self.n, self.h_out), dtype=torch.float32 if self.partial else self.X.dtype,
                             device="cuda")
        idx = torch.arange(self.tables * self.n, dtype=torch.int64, device="cuda").view(self.tables, self.n)
        self.A_tab = (self.A.data_ptr() + idx * (self.h_in * self.rank * e)).contiguous()
        self.B_tab = (self.B.data_ptr() + idx * (self.rank * self.h_out * e)).contiguous()
        self.seg_h = np.arange(self.n + 1, dtype=np.int32)
        self.lidx_h = np.arange(self.n, dtype=np.int32)
        self.seg = torch.from_numpy(self.seg_h).cuda()
        self.lidx = torch.from_numpy(self.lidx_h).cuda()
        self.problem = sg.make_problem(self.dtype, self.n, self.h_in, self.h_out, self.rank, self.n, self.n, 1)
        self.ws = sg.new_base_workspace(self.problem)
        self.bytes = (e * (self.h_in * self.h_out + self.n * (self.h_in + self.h_out) * self.rank + self.n * self.h_in)
                      + (4 if self.partial else e) * self.n * self.h_out)
        self.rows_per_step = self.n
        self.calls_per_step = 1
        self.fn = sg.load_library().sgmv_base_lora_apply
        Wsrc = self.W
        if self.partial:
            self.fn = sg.load_library().sgmv_base_lora_apply_partial
        if self.packed:
            self.fn = sg.load_library().sgmv_base_lora_apply_packed
            Wsrc = torch.stack([sg.pack_base_weight(self.W[w]) for w in range(self.wcopies)])
            self.Wp = Wsrc
        pb = ctypes.byref(self.problem)
        self.args = []
        for c in range(max(self.wcopies, self.tables, self.copies)):
            w, t, x = c % self.wcopies, c % self.tables, c % self.copies
            head = (pb, self.X[x].data_ptr(), Wsrc[w].data_ptr()) + ((0,) if self.partial else ())
            self.args.append(head + (self.A_tab[t].data_ptr(), self.B_tab[t].data_ptr(), self.Y[x].data_ptr(),
                                     self.seg.data_ptr(), self.lidx.data_ptr(), self.ws.data_ptr(), self.ws.numel()))
        # (a shard's fp32 partial has no torch counterpart of the same semantics)
        self.unfused = None if self.partial else self.time_unfused()
        torch.cuda.synchronize()

    def step(self, c, stream):
        st = self.fn(*self.args[c % len(self.args)], stream)
        if st != 0:
            raise RuntimeError(self.sg.sgmv_status_str(st))

    def time_unfused(self, iters=200):
        """Per-call time of torch's X @ W followed by sgmv_lora_apply (same rotation)."""
        torch, sg = self.torch, self.sg
        prob = sg.make_problem(self.dtype, self.n, self.h_in, self.h_out, self.rank, self.n, self.n, 1)
        ws = sg.new_workspace(prob)
        fn = sg.load_library().sgmv_lora_apply
        sid = torch.cuda.current_stream().cuda_stream

        def one(c):
            w, t, x = c % self.wcopies, c % self.tables, c % self.copies
            torch.matmul(self.X[x], self.W[w], out=self.Y[x])
            st = fn(ctypes.byref(prob), self.X[x].data_ptr(), self.A_tab[t].data_ptr(), self.B_tab[t].data_ptr(),
                    self.Y[x].data_ptr(), self.seg.data_ptr(), self.lidx.data_ptr(), ws.data_ptr(), ws.numel(),
                    sid)
            if st != 0:
                raise RuntimeError(sg.sgmv_status_str(st))

        for c in range(20):
            one(c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for c in range(iters):
            one(c)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    def check_sample(self, calls=2):
        import numpy as np
        import oracle
        torch = self.torch
        worst = 0.0
        sid = torch.cuda.current_stream().cuda_stream
        for c in range(calls):
            w, t, x = c % self.wcopies, c % self.tables, c % self.copies
            A = [_bits(self.A[t * self.n + k]) for k in range(self.n)]
            B = [_bits(self.B[t * self.n + k]) for k in range(self.n)]
            self.Y[x].fill_(float("nan"))
            self.step(c, sid)
            torch.cuda.synchronize()
            got = (self.Y[x].cpu().numpy().astype(np.float64) if self.partial
                   else oracle.decode(_bits(self.Y[x]), self.dtype))
            ref = oracle.sgmv_base_apply(self.dtype, _bits(self.X[x]), _bits(self.W[w]), A, B, self.seg_h,
                                         self.lidx_h)
            worst = max(worst, float((np.abs(got - ref) / (1e-3 + 1e-2 * np.abs(ref))).max()))
        if not worst <= 1.0:
            raise AssertionError(f"bench parity check failed: max err/bound {worst:.3f}")
        return worst

    def config(self):
        return {"workload": self.name, "h_in": self.h_in, "h_out": self.h_out, "rank": self.rank,
                "batch_rows": self.n, "segments": self.n, "distinct_loras": self.n, "w_copies": self.wcopies,
                "lora_tables": self.tables, "xy_copies": self.copies, "algorithmic_bytes_per_step": self.bytes,
                "output": ("fp32 partial X_g @ W_g + LoRA term of one row-parallel shard (written, unrounded)"
                           if self.partial else "Y = X @ W + LoRA term (written, one rounding)"),
                "weight_layout": "packed once before timing" if self.packed else "row-major",
                "unfused_torch_matmul_plus_sgmv_us_per_call": None if self.unfused is None else round(self.unfused, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 2000; 20 for a forward)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 200; 3 for a forward)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=SINGLE_WORKLOADS + MODEL_WORKLOADS + HET_WORKLOADS + BASE_WORKLOADS)
    ap.add_argument("--variant", choices=["auto", "vector", "fused", "mfma"], default="auto")
    ap.add_argument("--splits", type=int, default=0, help="workgroups per segment block (0 = automatic)")
    ap.add_argument("--no-batch", action="store_true",
                    help="forward workload: one call per projection instead of batching the "
                         "projections that share an input (q,k,v and gate,up)")
    ap.add_argument("--row-map", choices=["none", "kernel", "torch"], default="none",
                    help="rows of X and Y in segment order (none), or in request order gathered and "
                         "scattered by the kernels' row map (kernel) or by torch around each call (torch)")
    ap.add_argument("--host-meta", action="store_true",
                    help="single-projection workloads: call sgmv_lora_apply_host_meta (segment bounds and "
                         "LoRA pointer tables from host memory, passed in the kernel's arguments)")
    ap.add_argument("--curve", action="store_true",
                    help="instead of one workload: the LoRA addend's latency against batch size for "
                         "SGMV and two naive LoRA implementations (one JSON line)")
    ap.add_argument("--base-rows-curve", action="store_true",
                    help="instead of one workload: the base projection with the LoRA term against the "
                         "number of rows, fused call vs torch GEMM + SGMV (one JSON line)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from a captured HIP graph instead of eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads of the oracle baseline (0 = all cores)")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 8 plain device copies of 512 MiB (reference for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the SGMV path runs on a single MI355X and has no "
              "multi-GPU mode (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda").normal_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    if args.curve:
        print(json.dumps(latency_curve()), flush=True)
        return
    if args.base_rows_curve:
        print(json.dumps(base_rows_curve()), flush=True)
        return
    variant = {"auto": 0, "vector": 1, "fused": 2, "mfma": 3}[args.variant]
    model = args.workload in MODEL_WORKLOADS
    K = args.steps if args.steps is not None else (20 if model else 2000)
    W = args.warmup if args.warmup is not None else (3 if model else 200)
    if args.workload in HET_WORKLOADS:
        bench = MixedRankBench(args.workload, variant=variant, splits=args.splits)
    elif args.workload in BASE_WORKLOADS:
        bench = BaseBench(args.workload)
    elif model:
        bench = ModelForwardBench(args.workload, variant=variant, splits=args.splits,
                                  batch_projections=not args.no_batch, row_map=args.row_map)
    else:
        bench = SingleCallBench(args.workload, variant=variant, splits=args.splits, row_map=args.row_map,
                                host_meta=args.host_meta)
    worst = None if args.no_check else bench.check_sample()

    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    for c in range(W):
        bench.step(c, sid)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for c in range(K):
                bench.step(c, cap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    # Timed region: K steps between two device synchronisations, with HIP
    # events recorded on the launch stream at both ends, behind the pre-roll.
    sleep = getattr(torch.cuda, "_sleep", None)  # torch's internal spin kernel; absent: no pre-roll
    cycles = preroll_cycles(stream) if sleep is not None else 0
    ep, e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ep.record(stream)
    if cycles:
        sleep(cycles)
    e0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for c in range(K):
            bench.step(c, sid)
    e1.record(stream)
    torch.cuda.synchronize()
    preroll_s = ep.elapsed_time(e0) * 1e-3
    wall = time.perf_counter() - t0 - preroll_s
    ev_s = e0.elapsed_time(e1) * 1e-3
    ms_per_step = ev_s / K * 1e3
    launch_s = ev_s / (K * bench.calls_per_step)

    value = bench.bytes * K / ev_s / 1e9
    achieved = bench.bytes / bench.calls_per_step / launch_s / 1e9
    src_hash = kernel_source_hash()
    traffic = recorded_traffic(src_hash, args.workload) if traffic_applies(args) else None
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": bench.dtype,
        "data": "synthetic",
        "config": dict(bench.config(), variant=args.variant,
                       launch="graph" if graph is not None else "eager"),
        "pct_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(bench.rows_per_step * K / ev_s, 1),
        "us_per_call": round(ms_per_step * 1e3 / bench.calls_per_step, 3),
        "launch_us_mean_events": round(launch_s * 1e6, 3),
        "wall_ms_per_step": round(wall / K * 1e3, 6),
        "wall_value": round(bench.bytes * K / wall / 1e9, 2),
        "preroll_us": round(preroll_s * 1e6, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "roofline_traffic_from": (None if traffic is None else
                                  "committed counter run " + os.path.relpath(TRAFFIC_FILE, ROOT)
                                  + " (FETCH_SIZE + WRITE_SIZE per launch, scaled by a 512 MiB copy; "
                                  "kernel sources " + src_hash + ")"),
        "kernel_source_hash": src_hash,
        "parity_max_err_over_bound": None if worst is None else round(worst, 4),
    }
    if not args.no_cpu_baseline and args.workload == DEFAULT_WORKLOAD:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds, args.cpu_threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
