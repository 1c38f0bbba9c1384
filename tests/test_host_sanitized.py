"""The host-side tests of libtq.so rerun against a build whose host sources
(codebook construction, C-ABI validation and dispatch) carry
AddressSanitizer and UndefinedBehaviorSanitizer; any report aborts the child
process and fails this test.  CPU only: no device call is made."""
import os
import subprocess
import sys

import pytest

from kv_cache_vector_quantize_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_tests_under_asan_and_ubsan():
    if not os.path.exists(B.SAN_LIB):
        B.build_sanitized()
    try:
        rt = B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, TQ_LIBRARY=B.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_lib_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert "passed" in r.stdout
