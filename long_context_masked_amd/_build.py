"""Build libattn.so in-tree: hipcc for the gfx950 kernels, g++ for the host
mask compiler, one shared library next to this file."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")

HIP_SOURCES = ["api.hip", "fwd.hip", "bwd.hip", "dyn.hip"]
CXX_SOURCES = ["plan.cpp", "desc_cache.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
# Packed fp32 VALU forms are disabled for all device code.
# NaNs never arise on the path (masked scores are -inf, never NaN), which
# lets max chains fold into v_max3_f32 without canonicalisation.
HIP_FLAGS = COMMON + [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                      "-packed-fp32-ops", "-fno-honor-nans", "-Wno-unused-command-line-argument"]
CXX_FLAGS = COMMON + ["-Wall", "-Wextra", "-Wno-unused-parameter"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, extra_hip_flags=()) -> str:
    """Compile every source and link libattn.so; returns the library path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(OUT_DIR, s + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *extra_hip_flags, "-c", os.path.join(CSRC, s), "-o", o])
    cxx = shutil.which("g++") or "g++"
    for s in CXX_SOURCES:
        o = os.path.join(OUT_DIR, s + ".o")
        jobs.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(OUT_DIR, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
