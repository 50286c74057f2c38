"""Host code under the address and undefined-behaviour sanitizers (CPU only).

Builds, with g++ / gcc and -fsanitize=address,undefined (no device code, no
HIP), two drivers:
* tests/sanitize/host_checks.cpp with the library's host-only part
  (segmented_gather_matvec_amd/csrc/sgmv_host.cpp: the segment builder, the
  problem and metadata checks, the kernel plans and the workspace layout),
  run over seeded random, extreme and malformed inputs;
* tests/sanitize/oracle_checks.c with the C oracle (oracle/sgmv_oracle.c),
  run over random and malformed segment metadata.
A sanitizer report or a failed check makes the driver exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _tool(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not found")
    return path


def _build_and_run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower() and "cannot find" in r.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, f"build failed:\n{r.stderr[-4000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300, cwd=str(tmp_path))
    assert run.returncode == 0, f"{os.path.basename(exe)} failed:\n{run.stdout[-2000:]}\n{run.stderr[-6000:]}"
    return run.stdout


def test_host_planning_and_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = [_tool("g++"), "-std=c++17"] + SAN + [
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "segmented_gather_matvec_amd", "csrc"),
        os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
        os.path.join(ROOT, "segmented_gather_matvec_amd", "csrc", "sgmv_host.cpp"), "-o", exe]
    assert "host checks ok" in _build_and_run(cmd, exe, tmp_path)


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    cmd = [_tool("gcc"), "-std=c11"] + SAN + ["-fopenmp",
        os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), os.path.join(ROOT, "oracle", "sgmv_oracle.c"),
        "-lm", "-o", exe]
    assert "oracle checks ok" in _build_and_run(cmd, exe, tmp_path)
