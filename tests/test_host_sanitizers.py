"""The C-ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: tests/test_abi.py (every exported
symbol, every validation path, size arithmetic at the limits) runs in a child
process against libmxgemm_hostsan.so, api.hip's host code built with
-fsanitize=address,undefined (no recovery: any report fails the child), the
clang ASan runtime preloaded. No GPU call is made."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_host_sanitizers():
    sys.path.insert(0, ROOT)
    from mxfp8_decode_gemm_amd import build as b

    try:
        lib = b.build_host_sanitized()
        runtime = b.host_asan_runtime()
    except RuntimeError as e:
        pytest.fail(f"host sanitizer build: {e}")
    env = dict(os.environ)
    env.update({
        "MXG_LIBRARY": lib,
        "LD_PRELOAD": runtime,
        # The interpreter itself is not instrumented: its allocations are
        # not leak-checked.
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
