"""The oracle's C code built with AddressSanitizer and UndefinedBehaviorSanitizer, and the
CPU pins run against that build in a child process (libasan preloaded): any
out-of-bounds access, use after free, signed overflow or misaligned access in oracle.c
fails the test."""
import os
import subprocess
import sys

import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _libasan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    except OSError:
        return None
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_libasan() is None, reason="gcc's libasan is not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = O.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    env = dict(os.environ, FP8BS_ORACLE_LIB=lib, LD_PRELOAD=_libasan(), OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
