"""Helpers shared by the GPU tests: upload a seeded layer, run the library's
entry points through the C ABI, compare with the CPU oracle."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
import synth
from synth import configs

DEV = torch.device("cuda:0")
REL_TOL = 2e-3  # max-abs-error <= 2e-3 * max|ref|


def say(msg: str):
    print(msg, flush=True)


class DeviceLayer:
    """One layer's router and experts resident in HBM."""

    def __init__(self, w: configs.Workload, layer: int = 0, Wr=None, bias="default", blobs=None):
        self.w = w
        if Wr is None:
            Wr, b0 = configs.router(w, layer)
            if isinstance(bias, str):
                bias = b0
        elif isinstance(bias, str):
            bias = None
        self.Wr, self.bias = Wr, bias
        self.blobs = configs.experts(w, layer) if blobs is None else blobs
        self.dims = moe.Dims(w.d, w.f, w.n_experts, w.top_k, group_size=w.group,
                             code_bits=w.bits)
        self.Wr_d = torch.from_numpy(np.ascontiguousarray(Wr)).to(DEV)
        self.bias_d = None if bias is None else torch.from_numpy(bias).to(DEV)
        self.blobs_d = torch.from_numpy(self.blobs).to(DEV)
        self.table = torch.tensor([self.blobs_d[e].data_ptr() for e in range(w.n_experts)],
                                  dtype=torch.int64, device=DEV)

    def x_device(self, x, is_bf16):
        if is_bf16:
            return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)

    def route(self, xd):
        T = xd.shape[0]
        k = self.w.top_k
        idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
        wts = torch.empty(T, k, dtype=torch.float32, device=DEV)
        ws = moe.make_workspace(self.dims, T, DEV)
        moe.moe_route(self.dims, xd, self.Wr_d, self.bias_d, idx, wts, ws)
        torch.cuda.synchronize()
        return idx.cpu().numpy(), wts.cpu().numpy()

    def union(self, idx_np):
        T, k = idx_np.shape
        cap = min(self.w.n_experts, T * k)
        idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).to(DEV)
        uniq = torch.full((cap,), -7, dtype=torch.int32, device=DEV)
        nu = torch.zeros(1, dtype=torch.int32, device=DEV)
        offs = torch.full((cap + 1,), -7, dtype=torch.int32, device=DEV)
        rows = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        moe.moe_union(self.dims, idx, uniq, nu, offs, rows)
        torch.cuda.synchronize()
        return uniq.cpu().numpy(), int(nu.item()), offs.cpu().numpy(), rows.cpu().numpy()

    def forward(self, xd, flags=0, ws=None, out=None, stats=None, eps=1e-6):
        T = xd.shape[0]
        if out is None:
            out = torch.empty(T, self.w.d, dtype=torch.float32, device=DEV)
        if stats is None:
            stats = torch.zeros(1 + self.w.n_experts, dtype=torch.int32, device=DEV)
        if ws is None:
            ws = moe.make_workspace(self.dims, T, DEV)
        moe.moe_layer_forward(self.dims, xd, self.Wr_d, self.bias_d, self.table, out, flags=flags,
                              rms_eps=eps, stats=stats, ws=ws)
        torch.cuda.synchronize()
        self.last_ws = ws
        return out, stats

    def oracle_table(self):
        return [self.blobs[e] for e in range(self.w.n_experts)]


def record_margin(case: str, rel: float, **extra):
    """Append a case's measured max-abs-error / max|ref| to the file named by
    MOE_PARITY_LOG (one JSON object a line), when that variable is set."""
    path = os.environ.get("MOE_PARITY_LOG")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as fh:
        fh.write(json.dumps({"case": case, "rel_err": float(rel), "tol": REL_TOL, **extra}) + "\n")


def assert_close(got, ref, what="output", case=None):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref).max()
    tol = REL_TOL * np.abs(ref).max()
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.3e}"
    rel = err / max(np.abs(ref).max(), 1e-300)
    if case is not None:
        record_margin(case, rel, what=what)
    return rel


def check_layer_routing(dims, ws, T: int, ref: dict, what: str = "layer call"):
    """The routing a layer call left in its workspace (the lists its expert
    kernels walked) against the oracle's: ids, union, offsets and slot lists
    bit-exact, weights within 1e-6 relative."""
    r = moe.workspace_routing(dims, T, ws)
    torch.cuda.synchronize()
    k = dims.top_k
    idx = r["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, ref["idx"]), f"{what}: routing indices differ from the oracle"
    np.testing.assert_allclose(r["topk_w"].cpu().numpy(), ref["w"], rtol=1e-6, atol=1e-7,
                               err_msg=f"{what}: router weights")
    U = int(r["n_uniq"].item())
    assert U == ref["U"], f"{what}: U {U} != {ref['U']}"
    uniq, offs, rows = (r[n].cpu().numpy() for n in ("uniq", "offsets", "rows"))
    assert np.array_equal(uniq[:U], ref["uniq"]) and np.all(uniq[U:] == -1), f"{what}: union"
    assert np.array_equal(offs[:U + 1], ref["offsets"]), f"{what}: offsets"
    assert np.all(offs[U + 1:] == T * k), f"{what}: offsets past U"
    assert np.array_equal(rows, ref["rows"]), f"{what}: per-expert slot lists"
    return U


def check_union(layer: DeviceLayer, idx: np.ndarray):
    uniq, U, offs, rows = layer.union(idx)
    ru, ro, rr = oracle.union(idx, layer.w.n_experts)
    assert U == len(ru)
    assert np.array_equal(uniq[:U], ru) and np.all(uniq[U:] == -1)
    assert np.array_equal(offs[:U + 1], ro) and np.all(offs[U + 1:] == idx.size)
    assert np.array_equal(rows, rr)
    return U
