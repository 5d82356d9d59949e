"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_main.cpp drives every oracle entry point over the tiny shapes
the brute-force pins sweep (and the edge cases: zero-length requests, padding
and out-of-range slots, checkpoints, both layouts, widened and rolling
buffers, residual fusion with a row map, every CCA depthwise mode, the row
copies). Any out-of-bounds access, use of freed memory or undefined operation
in the oracle aborts the run."""
import os
import subprocess

from oracle.build import build_sanitized


def test_oracle_runs_clean_under_asan_and_ubsan():
    exe = build_sanitized()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle sanitizer run: ok" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
