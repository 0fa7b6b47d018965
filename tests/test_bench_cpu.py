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


def test_per_launch_bytes_and_source_hashes():
    # the algorithmic bytes bench.py divides by, and the counter-summary
    # hashes, for every workload it offers
    sys.path.insert(0, ROOT)
    import bench
    from synth import configs
    for name in ("decode1", "verify8", "prefill512", "chain48", "decode1_perrow",
                 "verify8_perrow", "prefill512_perrow", "decode1_int8", "verify8_int8",
                 "prefill512_int8", "decode1_int2", "verify8_int2", "prefill512_int2"):
        w = configs.WORKLOADS[name]
        gu, dn = bench.matrix_bytes(w)
        assert gu + dn == w.blob_bytes
        assert len(bench.kernel_source_hash(name)) == 16
    assert bench.matrix_bytes(configs.WORKLOADS["decode1"]) == (13369344, 6684672)
    assert bench.matrix_bytes(configs.WORKLOADS["decode1_int8"]) == (2 * (12582912 + 393216),
                                                                     12582912 + 393216)
