"""Phase timelines of the layer's kernels, from the phase-trace build.

    python int4_routed_expert_softmax_amd/phase_trace.py [--workload decode1] [--calls 3]

(by path, not with -m: the package must load its library after this script has
chosen the trace build).

Runs the named synthetic workload (the seeded GLM-5.2-shaped layers of
synth/configs.py, resident in HBM, rotating over --layers of them) through
lib/libmoe_trace.so, the library built with MOE_PHASE_TRACE (build.py
--trace), and after each of --calls layer calls prints, per traced kernel, the
spread of its workgroups' start times and of the time each spent between its
trace points (include/moe.h, moe_trace_read).  Times come from the device's
100 MHz clock, so they resolve 10 ns.  The trace build is for measurement:
its kernels write one record per workgroup besides their work.
"""
from __future__ import annotations

import argparse
import os
import sys

# The trace build must be chosen before the package loads its library.
os.environ["MOE_PHASE_TRACE"] = "1"
_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import numpy as np  # noqa: E402

import int4_routed_expert_softmax_amd as moe  # noqa: E402

if not moe.LIB_PATH.endswith("libmoe_trace.so"):
    raise SystemExit("phase_trace: the package was imported before this script chose the trace "
                     "build; run it by path (python int4_routed_expert_softmax_amd/phase_trace.py)")

# Names of the trace points of each kernel (index = point 1..5).
POINTS = {
    "gateup_gemv": ["sorts", "merges", "union", "rows (first wave)", "rows (all waves)"],
    "route_small": ["sorts", "merges", "union", "published"],
    "down_t1": ["rows (first wave)", "rows (all waves)"],
    "router_front": [],
    "gateup_thin": ["first copies issued", "first stage landed", "last stage done"],
    "down_thin": ["first copies issued", "first stage landed", "last stage done"],
    "gateup_mixed": [],
    "down_mixed": [],
}
TAGS = {"router_front": {1: "logits", 2: "x pack", 3: "digit split"},
        "gateup_mixed": {1: "M-blocked", 2: "thin", 3: "empty slot"},
        "down_mixed": {1: "M-blocked", 2: "thin", 3: "empty slot"}}


def us(ticks):
    return np.asarray(ticks, dtype=np.float64) * 0.01  # 100 MHz


def q(a):
    """p10 / p50 / p90 / max of a in microseconds."""
    a = np.asarray(a)
    return (f"{np.percentile(a, 10):7.2f} {np.percentile(a, 50):7.2f} "
            f"{np.percentile(a, 90):7.2f} {a.max():7.2f}")


def summarize(name, rec):
    """Text lines for one kernel's records (uint64 [n][8])."""
    rec = rec.astype(np.int64)
    rec = rec[rec[:, 0] > 0]
    if len(rec) == 0:
        return []
    t0 = rec[:, 0].min()
    lines = [f"{name}: {len(rec)} workgroups, first start to last end "
             f"{us(rec[:, 6].max() - t0):.2f} us   (us: p10 p50 p90 max)"]
    tags = rec[:, 7] & 0xFF
    groups = [(TAGS[name].get(int(t), f"tag {t}"), tags == t) for t in sorted(set(tags.tolist()))] \
        if name in TAGS else [("all", np.ones(len(rec), bool))]
    for label, sel in groups:
        r = rec[sel]
        if name in TAGS:
            lines.append(f"  {label}: {len(r)} workgroups")
        # workgroups that reached point 1 (or, without points, all of them)
        pts = POINTS[name]
        if pts:
            live = r[r[:, 1] > 0]
            if len(live) < len(r):
                lines.append(f"    {len(r) - len(live)} without work (ended at once)")
            r = live
        if len(r) == 0:
            continue
        row = lambda label, v: lines.append(f"    {label:<42s} {q(us(v))}")
        row("start, after the first workgroup's", r[:, 0] - t0)
        prev, prev_name = r[:, 0], "start"
        for i, pn in enumerate(pts, start=1):
            reached = r[:, i] > 0
            if not reached.any():
                continue
            row(f"{prev_name} -> {pn}", (r[:, i] - prev)[reached])
            prev, prev_name = np.where(reached, r[:, i], prev), pn
        row(f"{prev_name} -> end", r[:, 6] - prev)
        row("workgroup, start -> end", r[:, 6] - r[:, 0])
        row("end, after the first workgroup's start", r[:, 6] - t0)
    return lines


def main():
    import torch
    from synth import configs

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="decode1",
                    choices=["decode1", "verify8", "prefill512", "decode1_int8", "verify8_int8",
                             "decode1_int2", "verify8_int2"])
    ap.add_argument("--layers", type=int, default=None, help="rotating resident layers")
    ap.add_argument("--calls", type=int, default=3, help="traced calls (after 10 untimed ones)")
    a = ap.parse_args()
    w = configs.WORKLOADS[a.workload]
    L = a.layers or (2 if w.T > 8 else 4)
    dev = torch.device("cuda:0")
    dims = moe.Dims(w.d, w.f, w.n_experts, w.top_k, group_size=w.group, code_bits=w.bits)
    layers = []
    for l in range(L):
        Wr, bias = configs.router(w, l)
        blobs = torch.from_numpy(configs.experts(w, l)).to(dev)
        table = torch.tensor([blobs[e].data_ptr() for e in range(w.n_experts)],
                             dtype=torch.int64, device=dev)
        x, bf = configs.tokens(w, l)
        xd = (torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) if bf
              else torch.from_numpy(x).to(dev))
        layers.append((torch.from_numpy(Wr).to(dev), torch.from_numpy(bias).to(dev), blobs,
                       table, xd))
        print(f"phase_trace: layer {l} resident", file=sys.stderr, flush=True)
    out = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
    ws = moe.make_workspace(dims, w.T, dev)
    stats = torch.zeros(1 + w.n_experts, dtype=torch.int32, device=dev)

    def call(i):
        Wr, b, _, t, xd = layers[i % L]
        moe.moe_layer_forward(dims, xd, Wr, b, t, out, stats=stats, ws=ws)

    for i in range(10):
        call(i)
    torch.cuda.synchronize()
    print(f"# {a.workload}: d={w.d} f={w.f} E={w.n_experts} top-{w.top_k} T={w.T}, int{w.bits} "
          f"experts, {L} rotating layers; one traced layer call each\n")
    for c in range(a.calls):
        moe.moe_trace_reset()
        call(c)
        torch.cuda.synchronize()
        print(f"## call {c}: {int(stats[0].item())} distinct experts")
        for name in moe.TRACES:
            for line in summarize(name, moe.moe_trace_read(name)):
                print(line)
        print(flush=True)


if __name__ == "__main__":
    main()
