"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host side (layout validation, byte sizing, plane placement, token
routing, launch set-up) is rebuilt with both sanitizers on the host code only
(quantized_kv_cache_quant_amd.build.build_host_sanitized) and the whole CPU ABI
suite (tests/test_abi.py: every export, every validation error, sizing, the
binding's shape checks) runs in a child process that loads that build, with the
sanitizer runtime preloaded.  Any out-of-bounds access, use after free or
undefined behaviour in the host code aborts the child with a report.
"""
import os
import subprocess
import sys

import pytest

from quantized_kv_cache_quant_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_host_sanitizers():
    try:
        lib = build.build_host_sanitized()
        rt = build.sanitizer_runtime()
    except (RuntimeError, OSError, subprocess.CalledProcessError) as e:     # no ROCm toolchain here
        pytest.skip(f"sanitizer build unavailable: {e}")
    env = dict(os.environ, KVQ_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error:" not in report, report[-4000:]
    assert " passed" in r.stdout
