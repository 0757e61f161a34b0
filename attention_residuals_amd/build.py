"""Builds the gfx950 HIP library ``libattnres.so`` in-tree with hipcc.

Every ``csrc/*.hip`` file (kernel instantiations) and ``csrc/attnres_host.cpp`` (the C ABI) is
compiled to an object in ``_build/`` in parallel, then linked into
``attention_residuals_amd/libattnres.so``. All device code is built with packed-FP32 instructions
disabled (``-packed-fp32-ops``); hipcc's host pass warns that it does not know that feature.

Usage: ``python -m attention_residuals_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattnres.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -amdgpu-atomic-optimizer-strategy=None: the backward takes its token ticket with a single-lane
# atomic whose result is consumed after a whole pass of math; the optimizer's wave-reduced form
# reads the result back immediately, which waits for every outstanding memory operation.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compiles every source and links the library. Always rebuilds. Returns the library path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "attnres_host.cpp")]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
