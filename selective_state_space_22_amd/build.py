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
from concurrent.futures import ThreadPoolExecutor

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


FLAGS = ["-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]
OBJ_DIR = os.path.join(ROOT, "_build")


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}"] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed: {' '.join(cmd[-3:])}")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library.
    Every call compiles every source."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(lambda so: _run(compile_command(os.path.join(CSRC, so[0]), so[1]), verbose),
                      zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
