"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
oracle function on small layers that reach the edges of its loops (one
token, k = 1, k = E, per-row scales, bf16 input, RMSNorm + residual, a union
wider than one 64-lane group, experts left out of the table), built with
every sanitizer report fatal (oracle/sanitize_check.c)."""
import os
import subprocess

import oracle


def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    exe = oracle.build_sanitized(str(tmp_path))
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "sanitized oracle: all ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
