"""The fp64 oracle and the library's host-side argument handling under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

- The oracle (oracle/s6_oracle.c) is built with gcc and the sanitizers into a
  small driver (tests/sanitize/oracle_driver.c) that calls every entry point on
  seeded inputs and edge cases (one token, an empty sequence, no channels, every
  N, with and without h0 and the gate, rejected arguments); leak checking on.
- The library is built with the sanitizers on its host code only (each
  -fsanitize= behind -Xarch_host; the device code is the ordinary build) and
  linked into a driver (tests/sanitize/abi_driver.c) that exercises validation,
  workspace sizing, the options, the no-allocation scan's refusal and the
  calibration utility's checks.  Every call there returns before the HIP runtime
  is asked to do anything, so no GPU is needed.

Either driver exits non-zero on a failed check, and any sanitizer report aborts
it (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_22_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    rc, log = _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fopenmp", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "s6_oracle.c"), "-lm"])
    assert rc == 0, log
    rc, log = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4"))
    assert rc == 0 and "all checks passed" in log, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log


def test_host_validation_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    from selective_state_space_22_amd import build as lib_build

    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument",
             "-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        return obj, _run([HIPCC] + flags + ["-c", "-o", obj, os.path.join(CSRC, src)])

    with ThreadPoolExecutor(8) as ex:
        results = list(ex.map(compile_one, lib_build.SOURCES))
    for obj, (rc, log) in results:
        assert rc == 0, log
    lib = str(tmp_path / "libmamba_san.so")
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + [o for o, _ in results])
    assert rc == 0, log
    exe = str(tmp_path / "abi_driver")
    rc, log = _run([CLANG, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(HERE, "abi_driver.c"), lib, f"-Wl,-rpath,{tmp_path}", "-lstdc++"])
    assert rc == 0, log
    rc, log = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert rc == 0 and "all checks passed" in log, log
    assert "runtime error" not in log and "AddressSanitizer" not in log, log
