"""The phase-trace build (lib/libmoe_trace.so): same results as the oracle on
the paths of every traced kernel, and complete, ordered workgroup records.
The trace library is loaded in a child process, since a process holds the
one library the package chose at import."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_trace_build_records_and_results():
    env = dict(os.environ, MOE_PHASE_TRACE="1")
    p = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "trace_check.py")],
                       env=env, capture_output=True, text=True, timeout=110)
    print(p.stdout)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.count(" ok ") == 3, p.stdout
