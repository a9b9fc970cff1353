"""Build the HIP library in-tree: recurrent_state_amd/_lib/libtaylor_attn.so (gfx950).

Every source is compiled with hipcc for gfx950 only, in parallel, then linked
into one shared library with an rpath to the ROCm runtime.  Packed-fp32
instruction selection is turned off for all device code.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libtaylor_attn.so")

SOURCES = ["api.cpp", "decode.hip", "prefill_generic.hip", "prefill_mfma.hip", "prefill_wide.hip", "centered.hip", "backward.hip", "backward_wide.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-Wall", "-Wno-unused-function",
    ]


def _compile(src):
    out = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{errs}")
    return out, errs


def build(verbose=True, jobs=None):
    """Compile every source and link the library. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (_, errs), src in zip(results, SOURCES):
        if errs.strip() and verbose:
            print(f"[{src}]\n{errs}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results] + [
        "-Wl,-rpath,/opt/rocm/lib", "-Wl,-soname,libtaylor_attn.so"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
