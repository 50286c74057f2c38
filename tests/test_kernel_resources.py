"""CPU test of the compiled kernels' resources (no GPU).

Every kernel of the library is compiled for gfx950 with the build's own flags
(device code only, to assembly), and the code-object metadata of each kernel
must show no private (scratch) segment and no VGPR spills (a few SGPR spills
are allowed: with no private segment they go to VGPR lanes, not memory).  Scratch use
appears without any diagnostic when the compiler cannot keep a local array or
struct copy in registers (for instance a conditional copy of a kernel-argument
struct selected by blockIdx.y), and it puts a memory round trip on the
kernel's critical path.
"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from segmented_gather_matvec_amd import build

KERNEL_FILES = sorted(f for f in os.listdir(build.CSRC) if f.endswith(".hip"))


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in build.COMMON if f != "-fPIC"]
    cmd = [build.hipcc()] + flags + ["--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, f"device compile failed: {src}\n{res.stderr[-4000:]}"
    with open(out) as f:
        return f.read()


def _kernel_resources(asm: str):
    """(name, private segment bytes, vgpr spills, sgpr spills) of every kernel
    in the AMDGPU metadata of one assembly file."""
    out = []
    for block in re.split(r"\n\s+- \.agpr_count:", asm):
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        vsp = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
        ssp = re.search(r"\.sgpr_spill_count:\s+(\d+)", block)
        if name and priv and vsp and ssp:
            out.append((name.group(1), int(priv.group(1)), int(vsp.group(1)), int(ssp.group(1))))
    return out


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    srcs = [os.path.join(build.CSRC, f) for f in KERNEL_FILES]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        asms = list(ex.map(lambda s: _device_asm(s, d), srcs))
    return {f: _kernel_resources(a) for f, a in zip(KERNEL_FILES, asms)}


@pytest.mark.parametrize("src", KERNEL_FILES)
def test_no_scratch_and_no_spills(resources, src):
    kernels = resources[src]
    assert kernels, f"no kernel metadata parsed from {src}"
    bad = [k for k in kernels if k[1] or k[2]]
    assert not bad, f"{len(bad)} kernel(s) of {src} use scratch or spill VGPRs (name, private bytes, vgpr, sgpr): {bad[:4]}"
