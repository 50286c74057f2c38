"""Summaries of rocprofv3 output for libsgmv kernels.

    python -m segmented_gather_matvec_amd.profiling stats --trace DIR --out FILE.txt --command "..."
    python -m segmented_gather_matvec_amd.profiling traffic --fetch DIR --write DIR --kernel REGEX \
        --copy REGEX --copy-bytes N --algorithmic-bytes B --source-hash H --out FILE.json \
        --summary FILE.txt --command-fetch "..." --command-write "..."
    python -m segmented_gather_matvec_amd.profiling counters --pmc DIR [DIR ...] --kernel REGEX \
        --simds N --out FILE.txt --command "..." [--command "..."]

`stats` reads the kernel-trace CSVs of a `rocprofv3 --kernel-trace -f csv` run
and writes per-kernel launch counts and durations.  `counters` reads
`rocprofv3 --pmc ... -f csv` runs and writes, per matched kernel, the mean of
every counter per dispatch (summed over the device's XCDs / SEs) and the ratios
derived from them: matrix-core busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
SIMDs x GPU-busy cycles per XCD), LDS bank-conflict fraction of active LDS
cycles, L2 hit rate, mean L1->L2 read latency and reads in flight, the share of
L1 cycles stalled with its table of pending L2 reads full, and the share of
wave time spent waiting.  `traffic` reads two
`rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs (KiB per dispatch),
scales each counter by what it reads for a plain device copy of known size in
the same run, and writes the HBM bytes per launch of the matched kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import statistics as st
from typing import Dict, List


def _rows(directory: str, suffix: str) -> List[dict]:
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def short_name(name: str) -> str:
    """Kernel name without its parameter list, return type and anonymous
    namespaces; template arguments kept."""
    n = name.strip().replace("(anonymous namespace)::", "")
    if n.endswith(")"):
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += n[i] == ")"
            depth -= n[i] == "("
            if depth == 0:
                n = n[:i]
                break
    return re.sub(r"^void ", "", n)


def kernel_stats(trace_dir: str) -> Dict[str, dict]:
    out: Dict[str, List[float]] = {}
    for r in _rows(trace_dir, "kernel_trace.csv"):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
        out.setdefault(short_name(r["Kernel_Name"]), []).append(d)
    res = {}
    for k, ds in out.items():
        res[k] = {"calls": len(ds), "total_us": sum(ds), "mean_us": st.mean(ds),
                  "median_us": st.median(ds), "min_us": min(ds), "max_us": max(ds)}
    return res


def counter_means(pmc_dir: str, counter: str) -> Dict[str, dict]:
    vals: Dict[str, List[float]] = {}
    for r in _rows(pmc_dir, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        vals.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: {"dispatches": len(v), "mean": st.mean(v), "median": st.median(v)} for k, v in vals.items()}


def copy_reference(pmc_dir: str, counter: str, regex: str) -> dict:
    """Counter of the calibration copies: among the dispatches whose kernel
    matches `regex`, those with the largest grid (other, smaller copies made
    by the program are left out)."""
    rows = [r for r in _rows(pmc_dir, "counter_collection.csv")
            if r.get("Counter_Name") == counter and re.search(regex, short_name(r["Kernel_Name"]))]
    if not rows:
        raise SystemExit(f"no copy dispatch matches {regex!r}")
    grid = max(int(r["Grid_Size"]) for r in rows)
    v = [float(r["Counter_Value"]) for r in rows if int(r["Grid_Size"]) == grid]
    return {"dispatches": len(v), "mean": st.mean(v), "median": st.median(v), "grid": grid}


def _match(table: Dict[str, dict], regex: str) -> dict:
    keys = [k for k in table if re.search(regex, k)]
    if not keys:
        raise SystemExit(f"no kernel matches {regex!r}; kernels: {sorted(table)}")
    if len(keys) > 1:
        # several template instances: pool them by dispatch-weighted mean
        n = sum(table[k].get("dispatches", table[k].get("calls", 0)) for k in keys)
        m = sum(table[k]["mean"] * table[k]["dispatches"] for k in keys) / n
        return {"dispatches": n, "mean": m, "kernels": keys}
    return dict(table[keys[0]], kernels=keys)


def cmd_stats(a):
    stats = kernel_stats(a.trace)
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {a.command}", "",
             f"{'kernel':100s} {'calls':>7s} {'mean_us':>9s} {'median_us':>9s} {'min_us':>8s} {'max_us':>8s} {'total_us':>10s}"]
    for k, v in sorted(stats.items(), key=lambda kv: -kv[1]["total_us"]):
        lines.append(f"{k[:100]:100s} {v['calls']:7d} {v['mean_us']:9.3f} {v['median_us']:9.3f} "
                     f"{v['min_us']:8.3f} {v['max_us']:8.3f} {v['total_us']:10.1f}")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def pmc_dispatch_totals(dirs: List[str]) -> Dict[str, Dict[str, List[float]]]:
    """kernel -> counter -> per-dispatch totals (summed over the rows a
    dispatch has per XCD / SE / instance)."""
    acc: Dict[str, Dict[str, Dict[str, float]]] = {}
    for d in dirs:
        for r in _rows(d, "counter_collection.csv"):
            k = short_name(r["Kernel_Name"])
            c = acc.setdefault(k, {}).setdefault(r["Counter_Name"], {})
            key = f"{d}:{r['Dispatch_Id']}"
            c[key] = c.get(key, 0.0) + float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in acc.items()}


def cmd_counters(a):
    tot = pmc_dispatch_totals(a.pmc)
    keys = sorted(k for k in tot if re.search(a.kernel, k))
    if not keys:
        raise SystemExit(f"no kernel matches {a.kernel!r}; kernels: {sorted(tot)}")
    lines = ["# rocprofv3 counters per dispatch (mean over dispatches; each summed over the device)"]
    lines += [f"# command: {c}" for c in a.command]
    lines += [f"# derived ratios assume {a.simds} SIMDs, {a.cus} CUs and {a.xcds} XCDs", ""]
    for k in keys:
        m = {c: st.mean(v) for c, v in tot[k].items()}
        n = max(len(v) for v in tot[k].values())
        lines.append(f"kernel: {k}  ({n} dispatches)")
        for c in sorted(m):
            lines.append(f"  {c:36s} {m[c]:18,.1f}")
        der = []
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "GRBM_GUI_ACTIVE" in m:
            der.append(("matrix-core busy fraction",
                        m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / a.xcds * a.simds)))
        if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_LDS_IDX_ACTIVE"):
            der.append(("LDS bank-conflict share of active LDS cycles", m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"]))
        if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m and m["TCC_HIT_sum"] + m["TCC_MISS_sum"] > 0:
            der.append(("L2 hit rate", m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"])))
        if m.get("TCP_TCC_READ_REQ_sum"):
            der.append(("mean L1->L2 read latency (cycles)", m["TCP_TCC_READ_REQ_LATENCY_sum"] / m["TCP_TCC_READ_REQ_sum"]))
        if m.get("TCP_TCC_READ_REQ_LATENCY_sum") and m.get("GRBM_GUI_ACTIVE"):
            der.append(("mean L1->L2 reads in flight (device)",
                        m["TCP_TCC_READ_REQ_LATENCY_sum"] / (m["GRBM_GUI_ACTIVE"] / a.xcds)))
        if "TCP_PENDING_STALL_CYCLES" in m and m.get("GRBM_GUI_ACTIVE"):
            der.append(("share of L1 cycles stalled on pending L2 data",
                        m["TCP_PENDING_STALL_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / a.xcds * a.cus)))
        if m.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in m:
            der.append(("share of wave cycles waiting on a dependency", m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]))
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m or "SQ_INSTS_VALU_MFMA_MOPS_F16" in m:
            mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + m.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
            der.append(("matrix-core flops per dispatch (MOPS x 512)", mops * 512))
        for name, v in der:
            lines.append(f"  = {name:46s} {v:14.4f}" if v < 1e6 else f"  = {name:46s} {v:14,.0f}")
        lines.append("")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


def cmd_traffic(a):
    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    kf, kw = _match(fetch, a.kernel), _match(write, a.kernel)
    cf, cw = copy_reference(a.fetch, "FETCH_SIZE", a.copy), copy_reference(a.write, "WRITE_SIZE", a.copy)
    # Scale: a copy of N bytes reads N and writes N bytes of HBM.
    f_scale = a.copy_bytes / (cf["mean"] * 1024.0)
    w_scale = a.copy_bytes / (cw["mean"] * 1024.0)
    fb = kf["mean"] * 1024.0 * f_scale
    wb = kw["mean"] * 1024.0 * w_scale
    rec = {"kernel": a.kernel, "bytes_per_launch": round(fb + wb), "fetch_bytes_per_launch": round(fb),
           "write_bytes_per_launch": round(wb), "fetch_kib_raw": kf["mean"], "write_kib_raw": kw["mean"],
           "copy_bytes": a.copy_bytes, "copy_fetch_kib_raw": cf["mean"], "copy_write_kib_raw": cw["mean"],
           "fetch_scale": f_scale, "write_scale": w_scale, "dispatches": [kf["dispatches"], kw["dispatches"]],
           "algorithmic_bytes_per_launch": a.algorithmic_bytes,
           "traffic_over_algorithmic": (fb + wb) / a.algorithmic_bytes if a.algorithmic_bytes else None,
           "kernel_source_hash": a.source_hash, "command_fetch": a.command_fetch,
           "command_write": a.command_write}
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
    lines = ["# HBM traffic per launch from rocprofv3 counters",
             f"# fetch run: {a.command_fetch}", f"# write run: {a.command_write}", "",
             f"kernel                      : {a.kernel} ({kf['dispatches']} / {kw['dispatches']} dispatches)",
             f"FETCH_SIZE raw (KiB/launch) : {kf['mean']:.1f}   copy reference {cf['mean']:.1f} for {a.copy_bytes} B -> scale {f_scale:.4f}",
             f"WRITE_SIZE raw (KiB/launch) : {kw['mean']:.1f}   copy reference {cw['mean']:.1f} for {a.copy_bytes} B -> scale {w_scale:.4f}",
             f"HBM bytes per launch        : fetch {fb:,.0f} + write {wb:,.0f} = {fb + wb:,.0f}",
             f"algorithmic bytes / launch  : {a.algorithmic_bytes:,}",
             f"traffic / algorithmic       : {(fb + wb) / a.algorithmic_bytes:.3f}" if a.algorithmic_bytes else "",
             f"kernel source hash          : {a.source_hash}"]
    text = "\n".join(lines) + "\n"
    with open(a.summary, "w") as f:
        f.write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, default=0)
    t.add_argument("--source-hash", default="")
    t.add_argument("--out", required=True)
    t.add_argument("--summary", required=True)
    t.add_argument("--command-fetch", default="")
    t.add_argument("--command-write", default="")
    c = sub.add_parser("counters")
    c.add_argument("--pmc", nargs="+", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--out", required=True)
    c.add_argument("--command", action="append", default=[])
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
