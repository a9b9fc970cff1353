"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.cpp (validation, sizing, the monomial-table export) is compiled again with both sanitizers on its host
code only (`-Xarch_host` before each `-fsanitize=`; the device objects are the ones the library build
left in `_build/`, unchanged), linked into an instrumented copy of the library in a temporary folder,
and driven by `tests/abi_host_checks.cpp`: exact-size buffers for the table export, size queries at
the edges of their ranges, and every entry point with arguments it must reject.  No call reaches the
device, so this runs without a GPU.
"""

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "recurrent_state_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["--offload-arch=gfx950", "-std=c++20", "-fPIC", "-O1", "-g", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_abi_host_logic_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    kernels = sorted(o for o in glob.glob(os.path.join(BUILD, "*.o")) if not o.endswith("api.cpp.o"))
    if len(kernels) < 7:
        pytest.skip("kernel objects not built (run the library build first)")
    d = str(tmp_path)
    _run([HIPCC, "-x", "hip"] + COMMON + HOST_SAN + ["-c", os.path.join(CSRC, "api.cpp"), "-o", "api_san.o"], d)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", "libtaylor_attn_san.so", "api_san.o"] + kernels
         + HOST_SAN[:4] + ["-Wl,-rpath,/opt/rocm/lib"], d)
    _run([HIPCC, "-x", "hip"] + COMMON + HOST_SAN
         + ["-c", os.path.join(ROOT, "tests", "abi_host_checks.cpp"), "-o", "checks.o"], d)
    _run([HIPCC, "--offload-arch=gfx950", "checks.o", "libtaylor_attn_san.so", "-o", "abi_host_checks"]
         + HOST_SAN[:4] + [f"-Wl,-rpath,{d}"], d)
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([os.path.join(d, "abi_host_checks")], cwd=d, capture_output=True, text=True, timeout=300,
                       env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "host ABI checks passed" in out
    assert "Sanitizer" not in out and "runtime error" not in out, out[-6000:]
    shutil.rmtree(d, ignore_errors=True)
