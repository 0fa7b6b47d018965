"""bench.py's command-line contract, checked without a GPU: the one-GPU
limit and the batch-invariant mode's batch limits are refused before any
device work, with a message and a non-zero status."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    msg = json.loads(lines[0])
    assert "one GPU" in msg["error"]


def test_batch_invariant_past_its_limits_is_refused():
    r = run("--workload", "prefill512", "--batch-invariant", "--no-cpu")
    assert r.returncode != 0
    assert "batch limits" in r.stderr
