"""The C boundary's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

A copy of the library whose api.cpp is instrumented runs (1) the plain C caller
tests/c/abi_host_check.c and (2) this repository's ABI tests (tests/test_abi.py) through the
Python binding, with the sanitizer runtime preloaded. Every call there is refused or plans
only, so no kernel is launched; any out-of-bounds access, use after free, leak (C caller)
or undefined behaviour in the host checks fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists("/opt/rocm/llvm/bin/clang"), reason="needs ROCm clang")


@pytest.fixture(scope="module")
def san(tmp_path_factory):
    from sparse_attention_score_amd import hostsan
    return hostsan.build(str(tmp_path_factory.mktemp("hostsan")))


def test_c_caller_under_sanitizers(san):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([san["c_check"]], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host checks ok" in r.stdout


def test_abi_suite_under_sanitizers(san):
    # the Python interpreter is not instrumented: leak checking is off, errors still abort
    env = dict(os.environ, LD_PRELOAD=san["runtime"], SPARSE_ATTN_LIB=san["lib"],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        "-k", "not exports_only and not plain_c_caller"],
                       capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
