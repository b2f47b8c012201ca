"""Every kernel compiles for gfx950 without spilling to memory (CPU only).

A VGPR spill sends registers to scratch memory, which costs the matrix
phases far more than the spilled registers are worth; it has happened when a
change pushed one instance of a kernel template past 256 VGPRs.  This test
compiles each HIP source with the compiler's resource report and checks
every kernel instance: no VGPR spills, no scratch memory at all, and two
waves per SIMD for the forward and backward kernels.  SGPR spills are
allowed: they go to lanes of a VGPR (v_writelane / v_readlane), not to
memory, and the scratch check would catch any that did not.

The direct global-to-LDS copies are inline assembly that sets M0 (the LDS
address of the copy) and declares it clobbered.  M0 is a register the
compiler reserves, and it warns that such a clobber may not be preserved.
The copies are only safe if no compiler-generated instruction uses M0, so
the same compile's assembly is checked for that too.
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


_ASM = {}


def _report(src, tmp_path):
    from io_aware_tiled_04_amd import build
    asm = tmp_path / (src + ".s")
    cmd = [HIPCC, *build.FLAGS, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(asm),
           "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    _ASM[src] = asm.read_text()
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


def _instructions(text):
    for line in text.splitlines():
        line = line.split(";")[0].strip()
        if line and not line.startswith(".") and not line.endswith(":"):
            yield line


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("src", ["fa_fwd_bf16.hip", "fa_bwd_bf16.hip"])
def test_m0_is_only_the_direct_copy_address(src, tmp_path):
    if src not in _ASM:
        _report(src, tmp_path)
    ins = list(_instructions(_ASM[src]))
    copies = 0
    for i, line in enumerate(ins):
        if not re.search(r"\bm0\b", line):
            continue
        # the only instruction naming M0 is the copy's own set-up, followed by
        # the copy itself
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", line), line
        assert ins[i + 1] == "s_nop 0", ins[i + 1]
        assert ins[i + 2].startswith("buffer_load_dwordx4") and ins[i + 2].endswith("offen lds"), ins[i + 2]
        copies += 1
    assert copies > 0
