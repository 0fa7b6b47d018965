"""Run in a child process by tests/test_gpu_trace.py (MOE_PHASE_TRACE=1 in its
environment, so the package loads lib/libmoe_trace.so): small layers on the
paths of every traced kernel; checks that their outputs still match the CPU
oracle and that the workgroup records are complete and ordered.  Prints one
line per case and exits non-zero on the first failure."""
import os
import sys

assert os.environ.get("MOE_PHASE_TRACE") == "1"
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import int4_routed_expert_softmax_amd as moe  # noqa: E402
import oracle  # noqa: E402
from synth import configs  # noqa: E402

assert moe.LIB_PATH.endswith("libmoe_trace.so"), moe.LIB_PATH
DEV = torch.device("cuda:0")


def layer(name, d, f, E, k, T, zipf=True):
    w = configs.Workload(name, d=d, f=f, n_experts=E, top_k=k, T=T, seed=11, zipf=zipf)
    Wr, bias = configs.router(w)
    x, _ = configs.tokens(w)
    blobs = configs.experts(w)
    dims = moe.Dims(d, f, E, k)
    blobs_d = torch.from_numpy(blobs).to(DEV)
    table = torch.tensor([blobs_d[e].data_ptr() for e in range(E)], dtype=torch.int64, device=DEV)
    out = torch.empty(T, d, dtype=torch.float32, device=DEV)
    moe.moe_trace_reset()
    moe.moe_layer_forward(dims, torch.from_numpy(x).to(DEV), torch.from_numpy(Wr).to(DEV),
                          torch.from_numpy(bias).to(DEV), table, out,
                          ws=moe.make_workspace(dims, T, DEV))
    torch.cuda.synchronize()
    ref = oracle.layer_forward(x, Wr, bias, list(blobs), d, f, k)["out"]
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref).max() / np.abs(ref).max()
    assert err <= 2e-3, (name, err)
    return err


def check(kernel, expect_tags=None, need_points=0):
    r = moe.moe_trace_read(kernel).astype(np.int64)
    r = r[r[:, 0] > 0]
    assert len(r) > 0, f"{kernel}: no records"
    start, end = r[:, 0], r[:, 6]
    assert (end >= start).all() and (end - start < 100_000_000).all(), kernel  # < 1 s
    for i in range(1, 6):
        p = r[:, i]
        hit = p > 0
        assert (p[hit] >= start[hit]).all() and (p[hit] <= end[hit]).all(), (kernel, i)
    if need_points:
        live = r[r[:, 1] > 0]
        assert len(live) > 0, kernel
        for i in range(1, need_points):
            assert (live[:, i + 1] >= live[:, i]).all(), (kernel, i)
    tags = set((r[:, 7] & 0xFF).tolist())
    if expect_tags is not None:
        assert tags <= expect_tags, (kernel, tags)
    return len(r)


# one token: router front end (logits + digit split), single-token gate/up, down + combine
e = layer("trace_t1", 512, 512, 32, 8, 1)
n = (check("router_front", {1, 3}), check("gateup_gemv", {0, 1}, need_points=5),
     check("down_t1", {1}, need_points=2))
print(f"trace: one token ok (rel err {e:.2e}; records {n})", flush=True)
# 5 tokens: router front (logits in two halves + x pack), routing block, thin GEMMs
e = layer("trace_t5", 512, 512, 32, 8, 5)
n = (check("router_front", {1, 2}), check("route_small", {1}, need_points=4),
     check("gateup_thin", {1}, need_points=3), check("down_thin", {1}, need_points=3))
print(f"trace: five tokens ok (rel err {e:.2e}; records {n})", flush=True)
# hot experts: the mixed launch
e = layer("trace_hot", 512, 512, 8, 1, 70)
n = (check("gateup_mixed", {1, 2, 3}), check("down_mixed", {1, 2, 3}))
tags = set((moe.moe_trace_read("gateup_mixed")[:, 7] & 0xFF).tolist())
assert 1 in tags, tags
print(f"trace: mixed launch ok (rel err {e:.2e}; records {n})", flush=True)
