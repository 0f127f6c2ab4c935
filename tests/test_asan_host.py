"""The C ABI's host code under AddressSanitizer (no GPU).

tests/asan/build_asan.py builds the library with AddressSanitizer on its host
code only, and tests/asan/abi_check.cpp, linked against it, drives every host
path of the ABI: workspace sizes and launch plans over a sweep of valid and
invalid layers, token counts and workspace sizes; compute calls with one
invalid argument each, which must be rejected before any launch; the chunk
selector against its definition on random inputs; settings, status strings,
graph and flag calls with invalid handles.  Any out-of-bounds or
use-after-free access in that host code aborts the checker.
"""

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_host_code_under_address_sanitizer():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("the ROCm toolchain is needed to build the checker")
    sys.path.insert(0, os.path.join(HERE, "asan"))
    try:
        import build_asan  # the build script sits beside the checker's source
    finally:
        sys.path.pop(0)
    check = build_asan.build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    res = subprocess.run([check], capture_output=True, text=True, timeout=600, env=env)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert "0 failed expectations" in res.stdout
