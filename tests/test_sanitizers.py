"""The oracle's pins and the C-ABI's host-side checks, run again against
builds of the same sources with AddressSanitizer and UndefinedBehavior-
Sanitizer (tests/sanitize/build.py; host code only, no GPU).  A sanitizer
report aborts the child run, which fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_pins_and_abi_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, os.path.join(ROOT, "tests", "sanitize"))
    import build as san
    oracle_lib, host_lib = san.build(str(tmp_path))
    env = dict(os.environ,
               LD_PRELOAD=" ".join(san.runtime_preload()),
               # python and torch are not instrumented: no leak report, and no
               # new/delete pairing check across their allocators
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               KLA_ORACLE_LIB=oracle_lib, KLA_TEST_LIB=host_lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail
