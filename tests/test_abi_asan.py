"""The host-only ABI tests (tests/test_abi.py) once more against the host-side AddressSanitizer
build of the library (attention_residuals_amd/build_asan.py): the argument checks, plans and error
paths must not read or write out of bounds or use freed memory. CPU only: the test runs them in a
child Python with the sanitizer runtime preloaded and fails on any sanitizer report."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only check (no GPU runs)")
def test_host_abi_checks_under_address_sanitizer():
    from attention_residuals_amd import build_asan
    try:
        lib = build_asan.build_asan()
        rt = build_asan.runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "ATTNRES_LIB": lib,
                "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0:"
                                "halt_on_error=1:exitcode=86"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
