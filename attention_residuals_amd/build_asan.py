"""CPU-only checking build: the C ABI's host code (``csrc/attnres_host.cpp``: argument checks,
planning, launches) compiled with AddressSanitizer on the host pass only, linked with the kernel
objects of the last ``build()`` into ``_build/libattnres_asan.so``. The device code is the
ordinary build's; nothing here is meant for a GPU run. ``tests/test_abi_asan.py`` loads it with
the sanitizer runtime preloaded and runs the host-only ABI tests against it.

Usage: ``python -m attention_residuals_amd.build_asan`` (after ``python -m
attention_residuals_amd.build``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from .build import ARCH, CSRC, FLAGS, HIPCC, OUT_DIR

ASAN_LIB = os.path.join(OUT_DIR, "libattnres_asan.so")
# the sanitizer for the host pass only (each -fsanitize= right after -Xarch_host)
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload into Python)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("no shared AddressSanitizer runtime found next to hipcc")
    return path


def build_asan() -> str:
    objs = sorted(o for o in glob.glob(os.path.join(OUT_DIR, "*.hip.o")))
    if not objs:
        raise RuntimeError("no kernel objects in _build/: run attention_residuals_amd.build first")
    host = os.path.join(CSRC, "attnres_host.cpp")
    obj = os.path.join(OUT_DIR, "attnres_host_asan.o")
    r = subprocess.run([HIPCC] + FLAGS + HOST_SAN + ["-c", host, "-o", obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {host}:\n{r.stderr}")
    tmp = ASAN_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + HOST_SAN +
                       ["-o", tmp, obj] + objs, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build_asan())
    sys.exit(0)
