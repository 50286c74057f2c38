#!/usr/bin/env python3
"""Benchmark of libsgmv's SGMV LoRA term on one MI355X.

Default workload: decode batch, Distinct LoRA popularity (Punica README, page
"Punica：多 LoRA 模型统一服务框架", throughput paragraph): H1 = H2 = 4096 (Llama-7B
q_proj), r = 16, 32 fp16 rows, one row per segment, each on its own LoRA.
One step is one sgmv_lora_apply call (shrink + expand of the whole batch)
with the segment metadata already built.  To measure HBM and not the 256 MB
Infinity Cache, the 32 LoRAs of call c are drawn from a pool of 4096
(1 GiB of A and B) shifted by 32*c, and X / Y rotate over 64 copies.

Prints one JSON line: value = whole-job algorithmic GB/s over the timed steps
(K back-to-back launches, wall time between two device synchronisations);
roofline.achieved = algorithmic bytes per launch / mean launch duration from
HIP events recorded on the launch stream around the same timed region;
roofline.traffic = HBM bytes per launch from the committed counter runs
(FETCH_SIZE + WRITE_SIZE scaled by a copy kernel of known size), reported only
while the kernel sources still match the ones the counters were taken on;
cpu_baseline = the fp64 oracle timed on the host cores on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
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


def recorded_traffic(src_hash):
    """HBM bytes per launch measured by the committed counter runs, if they were
    taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


class DecodeBench:
    """Config: H1 = H2 = h, rank r, n rows, one segment per row, LoRA pool rotation."""

    def __init__(self, h=4096, rank=16, n=32, pool=4096, copies=64, variant=0, seed=2, splits=0):
        import torch
        import segmented_gather_matvec_amd as sg
        import workloads

        self.sg, self.torch = sg, torch
        self.h, self.rank, self.n, self.pool, self.copies = h, rank, n, pool, copies
        dev = "cuda"
        # Weights: pool of `pool` LoRAs, drawn on the device (seeded), fp16.
        self.A = workloads.device_normal((pool, h, rank), 1.0 / h ** 0.5, "f16", seed * 1000 + 1)
        self.B = workloads.device_normal((pool, rank, h), 1.0 / rank ** 0.5, "f16", seed * 1000 + 2)
        self.X = workloads.device_normal((copies, n, h), 1.0, "f16", seed * 1000 + 3)
        self.Y = workloads.device_normal((copies, n, h), 1.0, "f16", seed * 1000 + 4)
        self.tables = pool // n if pool >= n else 1
        a0, b0 = self.A.data_ptr(), self.B.data_ptr()
        sa, sb = h * rank * 2, rank * h * 2
        ids = (torch.arange(self.tables, device=dev)[:, None] * n
               + torch.arange(n, device=dev)[None, :]) % pool
        self.A_tab = (a0 + ids.to(torch.int64) * sa).contiguous()
        self.B_tab = (b0 + ids.to(torch.int64) * sb).contiguous()
        self.seg = torch.arange(n + 1, dtype=torch.int32, device=dev)
        self.lidx = torch.arange(n, dtype=torch.int32, device=dev)
        self.problem = sg.make_problem("f16", n, h, h, rank, n, n, 1, variant, splits)
        self.ws = sg.new_workspace(self.problem)
        self.bytes = algorithmic_bytes(2, n, h, h, rank, n)
        # Raw C entry point and per-call argument tuples (marshalled once).
        self.fn = sg.load_library().sgmv_lora_apply
        self.marshal()
        torch.cuda.synchronize()

    def marshal(self):
        pb = ctypes.byref(self.problem)
        wsn = self.ws.numel()
        self.args = []
        for c in range(max(self.tables, self.copies)):
            t, x = c % self.tables, c % self.copies
            self.args.append((pb, self.X[x].data_ptr(), self.A_tab[t].data_ptr(),
                              self.B_tab[t].data_ptr(), self.Y[x].data_ptr(), self.seg.data_ptr(),
                              self.lidx.data_ptr(), self.ws.data_ptr(), wsn))

    def step(self, c, stream=None):
        """Launch call c on `stream` (a raw hipStream_t; None = torch's current stream)."""
        if stream is None:
            stream = self.torch.cuda.current_stream().cuda_stream
        st = self.fn(*self.args[c % len(self.args)], stream)
        if st != 0:
            raise RuntimeError(self.sg.sgmv_status_str(st))

    def check_sample(self, calls=2):
        """Parity of the timed launch configuration on sampled calls (oracle, fp64)."""
        import numpy as np
        import oracle
        torch = self.torch
        worst = 0.0
        for c in range(calls):
            t, x = c % self.tables, c % self.copies
            ids = [(t * self.n + i) % self.pool for i in range(self.n)]
            Xh = self.X[x].view(torch.int16).cpu().numpy().view(np.uint16)
            Y0 = self.Y[x].view(torch.int16).cpu().numpy().view(np.uint16).copy()
            A = [self.A[k].view(torch.int16).cpu().numpy().view(np.uint16) for k in ids]
            B = [self.B[k].view(torch.int16).cpu().numpy().view(np.uint16) for k in ids]
            self.step(c)
            torch.cuda.synchronize()
            got = oracle.decode(self.Y[x].view(torch.int16).cpu().numpy().view(np.uint16), "f16")
            ref = oracle.sgmv_apply("f16", Xh, A, B, list(range(self.n + 1)), list(range(self.n)), Y0)
            ratio = np.abs(got - ref) / (1e-3 + 1e-2 * np.abs(ref))
            worst = max(worst, float(ratio.max()))
        if worst > 1.0:
            raise AssertionError(f"bench parity check failed: max err/bound {worst:.3f}")
        return worst


def cpu_baseline(seconds=10.0):
    """The oracle as it stands, on a host copy of the same workload shape."""
    import numpy as np
    import oracle
    import workloads
    w = workloads.decode_distinct()
    threads = oracle.max_threads()
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--variant", choices=["auto", "vector", "fused"], default="auto")
    ap.add_argument("--splits", type=int, default=0, help="workgroups per segment (0 = automatic)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from a captured HIP graph instead of eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 8 plain device copies of 512 MiB (reference for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only; the SGMV path runs on a single "
              "MI355X and has no multi-GPU mode (run with --gpus 1).", file=sys.stderr)
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
    variant = {"auto": 0, "vector": 1, "fused": 2}[args.variant]
    bench = DecodeBench(variant=variant, splits=args.splits)
    worst = None if args.no_check else bench.check_sample()

    K, W = args.steps, args.warmup
    for c in range(W):
        bench.step(c)
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
    # events recorded on the launch stream at both ends.
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for c in range(K):
            bench.step(c, sid)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / K * 1e3
    mean_kernel_s = e0.elapsed_time(e1) * 1e-3 / K

    value = bench.bytes * K / wall / 1e9
    achieved = bench.bytes / mean_kernel_s / 1e9
    src_hash = kernel_source_hash()
    traffic = recorded_traffic(src_hash)
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
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode_distinct_h4096_r16_b32", "h_in": 4096, "h_out": 4096,
                   "rank": 16, "batch_rows": 32, "segments": 32, "distinct_loras": 32,
                   "lora_pool": bench.pool, "xy_copies": bench.copies, "variant": args.variant,
                   "launch": "graph" if graph is not None else "eager",
                   "algorithmic_bytes_per_step": bench.bytes},
        "pct_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(bench.n * K / wall, 1),
        "us_per_call": round(ms_per_step * 1e3, 3),
        "launch_us_mean_events": round(mean_kernel_s * 1e6, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "kernel_source_hash": src_hash,
        "parity_max_err_over_bound": None if worst is None else round(worst, 4),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
