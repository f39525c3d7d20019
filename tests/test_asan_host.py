"""The library's host code under AddressSanitizer (CPU only).

libq4dec_asan.so is the same sources with the host pass instrumented
(argument checks, plans, workspace sizing, error text); the device code is
compiled as usual and never runs here. The C-ABI checks of test_abi.py run
against it in a child python that preloads the sanitizer runtime; any
out-of-bounds access, use after free or double free in the host paths they
reach aborts the child and fails this test."""
import os
import subprocess
import sys

import pytest

from int4_weight_only_block_amd import build as q4build

HERE = os.path.dirname(os.path.abspath(__file__))

pytestmark = pytest.mark.skipif(not os.path.exists(q4build.ASAN_LIB_PATH),
                                reason="libq4dec_asan.so not built (build(asan=True))")


def test_abi_checks_under_asan():
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": q4build.asan_runtime(),
        # python's own allocations are never freed at exit; only memory errors count
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "Q4DEC_LIB": q4build.ASAN_LIB_PATH,
    })
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(HERE, "test_abi.py")]
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900, cwd=os.path.dirname(HERE))
    out = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, out
    assert "AddressSanitizer" not in res.stderr, out
    assert " passed" in res.stdout, out


def test_asan_build_is_instrumented():
    """The child above really loads an instrumented library."""
    syms = subprocess.run(["nm", "-D", q4build.ASAN_LIB_PATH], capture_output=True, text=True).stdout
    assert "__asan_" in syms
