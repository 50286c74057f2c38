"""bench.py's contract, checked on the CPU.

- A run that asks for more than one GPU exits with a message before it touches a device.
- The roofline's traffic figure comes from the committed counter record only while the
  kernel sources hash as they did when the counters were taken, and only for the
  workload they were taken on.
- The algorithmic byte count of the headline decode call (the Punica README page
  "Punica：多 LoRA 模型统一服务框架", SGMV and micro-benchmark paragraphs: each
  distinct LoRA's A and B, X once, Y read and written once) equals the closed form
  written out below.
- The CPU baseline leg times the oracle and reports the fields the bench line carries.
"""
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8", "--steps", "3"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_headline_algorithmic_bytes_closed_form():
    # 32 distinct LoRAs of A [4096, 16] and B [16, 4096], 32 rows of X [4096],
    # 32 rows of Y [4096] read and written, 2-byte elements.
    lora = 32 * (4096 * 16 + 16 * 4096)
    rows = 32 * 4096 + 2 * 32 * 4096
    assert bench.algorithmic_bytes(2, 32, 4096, 4096, 16, 32) == 2 * (lora + rows) == 9_175_040


def test_traffic_record_is_gated_by_source_hash_and_workload(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_source_hash": "0123456789abcdef", "bytes_per_launch": 9_370_882}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("0123456789abcdef", bench.DEFAULT_WORKLOAD) == 9_370_882
    assert bench.recorded_traffic("0123456789abcdee", bench.DEFAULT_WORKLOAD) is None
    assert bench.recorded_traffic("0123456789abcdef", "mixed_r64_4096to11008") is None
    f.write_text("{not json")
    assert bench.recorded_traffic("0123456789abcdef", bench.DEFAULT_WORKLOAD) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.recorded_traffic("0123456789abcdef", bench.DEFAULT_WORKLOAD) is None


def test_source_hash_changes_with_every_listed_kernel_source(tmp_path, monkeypatch):
    for rel in bench.KERNEL_SOURCES:
        os.makedirs(tmp_path / os.path.dirname(rel), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), tmp_path / rel)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_hash()
    seen = {base}
    for rel in bench.KERNEL_SOURCES:
        p = tmp_path / rel
        original = p.read_bytes()
        p.write_bytes(original + b"\n")
        h = bench.kernel_source_hash()
        assert h not in seen, f"editing {rel} left the hash unchanged"
        seen.add(h)
        p.write_bytes(original)
    assert bench.kernel_source_hash() == base


def test_committed_traffic_record_describes_the_headline_kernel():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert rec["kernel"] == "sgmv_decode_kernel"
    assert rec["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(2, 32, 4096, 4096, 16, 32)
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert 1.0 <= rec["traffic_over_algorithmic"] < 1.5
    assert "FETCH_SIZE" in rec["command_fetch"] and "WRITE_SIZE" in rec["command_write"]


def test_cpu_baseline_times_the_oracle():
    cb = bench.cpu_baseline(seconds=0.2, threads=1)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] == 1
    assert cb["value"] > 0
    assert "oracle calls on one decode batch" in cb["sample"]


def test_traffic_record_only_for_the_default_launch():
    """The counter run behind roofline.traffic was taken on the headline's
    default launch; a forced variant, split count, host metadata or row layout
    runs other kernels and reports no traffic."""
    import argparse
    base = dict(workload=bench.DEFAULT_WORKLOAD, variant="auto", splits=0, host_meta=False, row_map="none")
    assert bench.traffic_applies(argparse.Namespace(**base))
    for k, v in (("variant", "vector"), ("variant", "mfma"), ("splits", 16), ("host_meta", True),
                 ("row_map", "kernel"), ("workload", "skewed_b32")):
        assert not bench.traffic_applies(argparse.Namespace(**dict(base, **{k: v}))), (k, v)
