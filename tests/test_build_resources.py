"""Every kernel compiles for gfx950 without spilling to memory (CPU only).

A VGPR spill sends registers to scratch memory, which costs the matrix
phases far more than the spilled registers are worth; it has happened when a
change pushed one instance of a kernel template past 256 VGPRs.  This test
compiles each HIP source with the compiler's resource report and checks
every kernel instance: no VGPR spills, no scratch memory at all, and two
waves per SIMD for the forward and backward kernels.  SGPR spills are
allowed: they go to lanes of a VGPR (v_writelane / v_readlane), not to
memory, and the scratch check would catch any that did not.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_tiled_04_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_bwd_bf16.hip", "fa_fwd_kvouter.hip"]


def _report(src, tmp_path):
    from io_aware_tiled_04_amd import build
    cmd = [HIPCC, *build.FLAGS, "--cuda-device-only", "-c",
           os.path.join(CSRC, src), "-o", str(tmp_path / (src + ".o")),
           "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    kernels = {}
    name = None
    for line in out.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(.+?): (\d+) \[-Rpass", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("src", SOURCES)
def test_no_spills_and_occupancy(src, tmp_path):
    kernels = _report(src, tmp_path)
    assert kernels, f"no kernel resource report for {src}"
    for name, r in kernels.items():
        assert r.get("VGPRs Spill", 0) == 0, (name, r)
        assert r.get("ScratchSize [bytes/lane]", 0) == 0, (name, r)
        if "fwd_bf16_kernel" in name or "bwd_dq_kernel" in name or "bwd_dkv_kernel" in name:
            assert r.get("Occupancy [waves/SIMD]", 0) >= 2, (name, r)
