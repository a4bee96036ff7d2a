"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the library's
host side is rebuilt with both sanitizers (build_lib.build(sanitize=True); the device code is unchanged) and
the ABI tests run against that build in a child process with the sanitizer runtime preloaded. Any report
ends the child with an error."""

import os
import subprocess
import sys

import pytest

from token_verification_row_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_address_and_undefined_behaviour_sanitizers():
    try:
        lib = build_lib.build(sanitize=True)
        runtime = build_lib.asan_runtime()
    except RuntimeError as e:                   # no ROCm toolchain on this host
        pytest.skip(str(e))
    env = dict(os.environ, DV_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest; from token_verification_row_amd import dlmverify as B; "
            f"assert B.LIB_PATH == {lib!r}, B.LIB_PATH; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
