"""Build libmamba_mi355x.so in-tree with hipcc for gfx950.

    python -m selective_state_space_22_amd.build

All HIP code is compiled without packed-fp32 instructions (the
``-packed-fp32-ops`` target feature): the scan is written in ordinary fp32.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmamba_mi355x.so")
SOURCES = ["api.cpp", "scan_kernels.hip", "scan_wg.hip", "scan_wp.hip", "scan_bwd.hip", "selection.hip", "scan_complex.hip", "noalloc.hip", "calibrate.hip"]
ARCH = os.environ.get("MAMBA_MI355X_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def command(out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"),
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmamba_mi355x.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
