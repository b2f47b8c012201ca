"""Build the attention forward library (libfa.so) for gfx950 with hipcc.

``python -m io_aware_tiled_04_amd.build`` (or ``build()``) compiles every HIP
source under ``csrc/`` and links ``libfa.so`` next to this file (and the
bench's shader-clock probe into ``libfa_clock.so``).  It always recompiles.  The library is loaded in-tree by ``io_aware_tiled_04_amd.fa``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fa_api.cpp", "fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_bwd_bf16.hip", "fa_fwd_kvouter.hip",
           "fa_noalloc.hip"]

# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-x", "hip",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _run_all(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        # hipcc's host pass does not know the device-only feature flag above
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln
                 and "warning: unknown" not in ln]
        if p.returncode != 0:
            failed.append((cmd, out))
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        msg = "\n\n".join(" ".join(c) + "\n" + o for c, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")


# The bench's shader-clock probe: a separate library, not part of the ABI.
CLOCK_SRC = "clock_probe.hip"
CLOCK_LIB = os.path.join(PKG, "libfa_clock.so")


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    ctmp = CLOCK_LIB + ".tmp"
    _run_all([[HIPCC, *FLAGS, "-shared", os.path.join(CSRC, CLOCK_SRC), "-o", ctmp]], verbose)
    os.replace(ctmp, CLOCK_LIB)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    _run_all(cmds, verbose)
    tmp = LIB + ".tmp"
    _run_all([[HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
