"""Sanitizer tier: the C oracle built with AddressSanitizer and
UndefinedBehaviorSanitizer (any report aborts), and the oracle's pin tests
run against that build in a child process with libasan preloaded.  An
out-of-bounds index or an overflow in the plain loops would otherwise only
show as a wrong value somewhere, or not at all."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PIN_TESTS = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
PIN_TESTS = [t for t in PIN_TESTS if not t.endswith("test_oracle_sanitized.py")]


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan is not installed")
    from oracle.build import build
    lib = build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan, KVD_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PIN_TESTS, "tests/test_gates_and_sizing.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
