"""The C ABI's argument checks under host-side AddressSanitizer and
UndefinedBehaviorSanitizer: api.hip's host code rebuilt with both
sanitizers (device code unchanged), then tests/test_abi.py run against that
library in a child process with the ASan runtime preloaded. Any sanitizer
report aborts the child (halt_on_error) and fails this test. CPU only: the
ABI tests make no GPU call."""

import os
import subprocess
import sys

import pytest

from runtime_mixed_precision_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime not found")
    if not all(os.path.exists(os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o")) for s in B.SOURCES):
        B.build()
    lib = B.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, AUTOFP_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "passed" in res.stdout
