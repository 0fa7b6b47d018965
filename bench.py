"""Benchmark of the gfx950 int4 routed-expert MoE layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode1]
                    [--layers R] [--cpu-seconds S | --no-cpu]

A step is one full layer forward (router, top-k, union, expert FFNs, combine)
over one batch of seeded synthetic tokens.  The default workload is a
GLM-5.2-shaped MoE layer at decode batch 1 (d=6144, f=2048, 256 experts,
top-8, gs64 int4, about 20 MB per expert).  Steps rotate over R independently
seeded layers, all resident in HBM, so that the 160 MB one decode step reads
are not served from the 256 MB Infinity Cache of the previous step.

Prints one JSON line: whole-layer tokens/s (value, K plain steps), expert-weight
GB/s, the dominant kernel's roofline (its algorithmic bytes per launch over its
average duration, measured with HIP events recorded around every launch of a
second run of the same K steps) and the CPU oracle's throughput on a bounded
sample.  `traffic` comes from the committed rocprofv3 counter summary in
profiles/ while the HIP sources still match the hash recorded there.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "MoE-layer tokens/s + int4 expert-weight HBM GB/s (% peak), d=6144 top-8/256"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default 200; chain48: 64)")
    p.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10; chain48: 2)")
    p.add_argument("--workload", default="decode1",
                   choices=["decode1", "verify8", "prefill512", "chain48", "decode1_perrow",
                            "verify8_perrow", "prefill512_perrow", "decode1_int8", "verify8_int8",
                            "prefill512_int8", "decode1_int2", "verify8_int2", "prefill512_int2"])
    p.add_argument("--layers", type=int, default=8, help="independent layers to rotate over")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="decode1: skip the verify8 and prefill512 figures on the same layers")
    p.add_argument("--host-tier", type=int, default=0, metavar="SLOTS",
                   help="decode1 / verify8 with one layer's experts in pinned host memory behind an "
                        "HBM cache of SLOTS expert slots (moe_layer_forward_cached); each step is "
                        "a new batch of tokens")
    p.add_argument("--batch-invariant", action="store_true",
                   help="verify8: run the batch with MOE_BATCH_INVARIANT (each token computed "
                        "exactly as in a one-token call)")
    p.add_argument("--int8-act", action="store_true",
                   help="run the layer with MOE_INT8_ACT: integer activations (int8 per 64-column "
                        "group, exact group dot products on the int8 matrix cores)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run 20 plain device-to-device copies of this many MiB (the known-size "
                        "reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 20}), flush=True)


# Sources the gate/up kernel of each path is built from: the one-token
# GEMV path (decode, chain) and the grouped GEMM (batches of 2+ tokens).
GATEUP_SOURCES = ("cache.h", "device_util.h", "ffn_gemv.hip", "moe_internal.h", "pack.h",
                  "select.h", "small_route.h", "trace.h")
GEMM_SOURCES = ("device_util.h", "ffn_mfma.hip", "moe_internal.h", "pack.h", "small_route.h",
                "trace.h")


def matrix_bytes(w):
    """(gate + up, down) bytes of one expert: codes (w.bits per weight) and
    fp16 scales (one per 64 weights of a row, or one per row)."""
    sg = w.d // 64 if w.group else 1
    sd = w.f // 64 if w.group else 1
    codes = w.f * w.d * w.bits // 8
    return 2 * (codes + 2 * w.f * sg), codes + 2 * w.d * sd


def gateup_sources(workload):
    gemv = workload.startswith(("decode1", "chain48"))  # one token: every width, either activation
    return GATEUP_SOURCES if gemv else GEMM_SOURCES


def kernel_source_hash(workload="decode1"):
    """sha256 of the gate/up kernel's sources for this workload: a counter
    summary is only reused while it matches."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_routed_expert_softmax_amd", "csrc")
    for name in gateup_sources(workload):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary,
    or None when that summary was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"gateup_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha") != kernel_source_hash(workload):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    a = parse()
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    if a.gpus != 1:
        print(json.dumps({"error": f"--gpus {a.gpus}: this benchmark runs on one GPU only; the "
                          "layer is measured at one GPU's share"}), flush=True)
        sys.exit(2)

    if a.workload == "chain48":
        a.steps = 64 if a.steps is None else a.steps
        a.warmup = 2 if a.warmup is None else a.warmup
        return run_chain(a)
    a.steps = 200 if a.steps is None else a.steps
    a.warmup = 10 if a.warmup is None else a.warmup
    if a.host_tier:
        return run_host_tier(a)

    import torch

    import int4_routed_expert_softmax_amd as moe
    from synth import configs

    w = configs.WORKLOADS[a.workload]
    if a.batch_invariant and (w.T > 8 or w.T * w.top_k > 64):
        sys.exit(f"--batch-invariant: {w.name} has T={w.T}, past the single-token family's "
                 "batch limits (T <= 8, T * k <= 64)")
    dev = torch.device("cuda:0")

    print(f"bench: {w.name} T={w.T} layers={a.layers} generating + uploading "
          f"{a.layers * w.n_experts * w.blob_bytes / 1e9:.1f} GB", file=sys.stderr, flush=True)
    layers = []
    for l in range(a.layers):
        Wr, bias = configs.router(w, l)
        blobs = torch.from_numpy(configs.experts(w, l)).to(dev)
        table = torch.tensor([blobs[e].data_ptr() for e in range(w.n_experts)], dtype=torch.int64,
                             device=dev)
        layers.append(dict(Wr=torch.from_numpy(Wr).to(dev),
                           bias=None if bias is None else torch.from_numpy(bias).to(dev),
                           blobs=blobs, table=table))
        print(f"bench: layer {l} resident", file=sys.stderr, flush=True)

    res = measure(moe, torch, w, layers, a.steps, a.warmup, a.batch_invariant,
                  lambda l: configs.tokens(w, l), i8=a.int8_act)
    res["config"]["workload"] += f", {a.layers} rotating HBM-resident layers"
    ceil = hbm_ceiling(moe, torch)
    res["hbm_read_ceiling"] = ceil
    for key in ("roofline", "roofline_down"):
        res[key]["frac_of_read_ceiling"] = round(res[key]["achieved"] / ceil["GBps"], 4)
    if w.T > 8 and not a.int8_act:
        res["mfma"] = mfma_figures(moe, torch, w, layers[0], res.pop("_gateup"))
    res.pop("_gateup", None)
    if a.workload == "decode1" and not a.no_extra and not a.int8_act:
        # the other two single-layer workloads, measured on the same resident
        # layers (same shape and weight distributions; their own token recipes)
        extra = {}
        for name in ("verify8", "prefill512"):
            wx = configs.WORKLOADS[name]
            K = min(a.steps, 50 if wx.T > 8 else a.steps)
            r = measure(moe, torch, wx, layers, K, a.warmup, False,
                        lambda l, wx=wx: configs.tokens(wx, l))
            r["config"]["workload"] += (f", on the {a.layers} rotating layers of this run "
                                        f"(decode1's seeded experts)")
            if wx.T > 8:
                r["mfma"] = mfma_figures(moe, torch, wx, layers[0], r.pop("_gateup"))
            r.pop("_gateup", None)
            for key in ("roofline", "roofline_down"):
                r[key]["frac_of_read_ceiling"] = round(r[key]["achieved"] / ceil["GBps"], 4)
            for k_ in ("metric", "unit", "n_gpus", "higher_is_better", "scaling", "vs_baseline",
                       "data"):
                r.pop(k_, None)
            extra[name] = r
            print(f"bench: {name} {r['value']} tokens/s, gate/up {r['roofline']['achieved']} GB/s",
                  file=sys.stderr, flush=True)
        res["other_workloads"] = extra
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(res), flush=True)


def measure(moe, torch, w, layers, K, warmup, inv, tokens, i8=False):
    """One workload on resident layers: `warmup` untimed steps, then K steps
    timed as one HIP graph replay (step i on layer i mod len(layers), each
    layer with its own seeded tokens), K eager steps for comparison, K more
    with HIP events around every gate/up and down launch (the roofline), and
    K with an event pair around each step (the spread).  i8: the layer calls
    take MOE_INT8_ACT."""
    dev = torch.device("cuda:0")
    R = len(layers)
    dims = moe.Dims(w.d, w.f, w.n_experts, w.top_k, group_size=w.group, code_bits=w.bits)
    blob = w.blob_bytes
    nib_gu, nib_dn = matrix_bytes(w)
    xs = []
    for l in range(R):
        x, bf = tokens(l)
        xs.append(torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16) if bf
                  else torch.from_numpy(np.ascontiguousarray(x)).to(dev))
    out = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
    stats = torch.zeros(R, 1 + w.n_experts, dtype=torch.int32, device=dev)
    ws = moe.make_workspace(dims, w.T, dev)
    stream = torch.cuda.current_stream()
    flags = (moe.MOE_BATCH_INVARIANT if inv else 0) | (moe.MOE_INT8_ACT if i8 else 0)
    # the library's choice: every layer takes the int8-digit GEMV kernels for
    # one token (or with the flag), int4 layers also for shapes off the 512
    # grid; other batches take the grouped GEMM (fp16 MFMA, or int8 MFMA with
    # integer activations)
    gemv = w.T == 1 or inv or (w.bits == 4 and (w.d % 512 or w.f % 512))

    def step(i, s=None):
        L = layers[i % R]
        moe.moe_layer_forward(dims, xs[i % R], L["Wr"], L["bias"], L["table"], out, flags=flags,
                              stats=stats[i % R], ws=ws,
                              stream=stream.cuda_stream if s is None else s)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # K steps with plain launches (Python enqueues every call)
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / K
    # the distinct experts of each layer, from the layer calls' own counts
    U = stats[:, 0].cpu().numpy().astype(np.float64)
    hot = stats[0, 1:].cpu().numpy()

    # the timed region: the same K steps as one HIP graph (the library only
    # enqueues kernels and allocates nothing), replayed once after a warm
    # replay, so no host launch overhead sits between the steps
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(K):
            step(i, side.cuda_stream)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del graph

    # the same K steps again with every launch of the FFN kernels recording
    # HIP events on the launch stream (recording adds launch overhead, so the
    # step rate above is measured without it); a projection may run as a thin
    # and an M-blocked launch, whose durations add up per step
    dur = ffn_launch_durations(moe, torch, K, step)

    # and once more with an event pair around every step (their spread)
    sev = ([torch.cuda.Event(enable_timing=True) for _ in range(K)],
           [torch.cuda.Event(enable_timing=True) for _ in range(K)])
    torch.cuda.synchronize()
    for i in range(K):
        sev[0][i].record()
        step(i)
        sev[1][i].record()
    torch.cuda.synchronize()
    step_us = np.array([s_.elapsed_time(e_) for s_, e_ in zip(*sev)]) * 1e3

    sec = (t1 - t0) / K
    u_steps = np.array([U[i % R] for i in range(K)])
    tok_s = w.T / sec
    weight_bytes_step = u_steps.mean() * blob
    gu_bytes = u_steps * nib_gu
    dn_bytes = u_steps * nib_dn
    gu_gbps = float(np.mean(gu_bytes / dur["gateup"]) / 1e9)
    dn_gbps = float(np.mean(dn_bytes / dur["down"]) / 1e9)
    del ws
    torch.cuda.empty_cache()
    return {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "ms_per_step_eager": round(eager * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"int{w.bits} weights x int8 activations (one scale per 64 columns, as int8 "
                  f"digits), i32 dot, f32 accumulate" if gemv and i8 else
                  f"int{w.bits} weights x int8-digit activations, i32 dot, f32 accumulate" if gemv else
                  f"int{w.bits} weights x int8 activations (one scale per 64 columns), MFMA i32 "
                  f"per group, f32 accumulate" if i8 else
                  f"int{w.bits} weights as fp16 x fp16 activations, MFMA f32 accumulate"),
        "data": "synthetic (seeded; random-init GLM-5.2-shaped experts)",
        "config": {"workload": f"{w.name}: one MoE layer, d={w.d} f={w.f} E={w.n_experts} "
                               f"top-{w.top_k}, T={w.T} tokens "
                               f"({'bf16' if w.x_bf16 else 'fp32'} x), "
                               f"{'gs64' if w.group else 'per-row'} int{w.bits} experts "
                               f"({blob} B each)" + (", MOE_BATCH_INVARIANT" if inv else "")
                               + (", MOE_INT8_ACT" if i8 else ""),
                   "T": w.T, "d": w.d, "f": w.f, "n_experts": w.n_experts, "top_k": w.top_k,
                   "layers_rotated": R, "distinct_experts_per_step": float(u_steps.mean())},
        "step_us_p10_p50_p90": [round(float(v), 2) for v in np.percentile(step_us, [10, 50, 90])],
        "expert_weight_GBps": round(weight_bytes_step / sec / 1e9, 1),
        "expert_weight_frac_hbm_peak": round(weight_bytes_step / sec / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "gateup (gate+up projections, SwiGLU)",
                     "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": committed_traffic(w.name + ("_i8act" if i8 else "")),
                     "bytes_per_launch": float(gu_bytes.mean()),
                     "avg_launch_us": round(float(dur["gateup"].mean() * 1e6), 3),
                     "launch_us_p10_p50_p90": [round(float(v) * 1e6, 3) for v in
                                               np.percentile(dur["gateup"], [10, 50, 90])]},
        "roofline_down": {"bound": "hbm", "achieved": round(dn_gbps, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(dn_gbps / HBM_PEAK_GBPS, 4),
                          "bytes_per_launch": float(dn_bytes.mean()),
                          "avg_launch_us": round(float(dur["down"].mean() * 1e6), 3)},
        "_gateup": {"dur": dur["gateup"], "hot_counts": hot, "x0": xs[0], "dims": dims},
    }


MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published


def hbm_ceiling(moe, torch, gib=4):
    """Read bandwidth of a plain streaming kernel (moe_hbm_read_probe) over
    `gib` GiB, far past the 256 MB Infinity Cache: the best of a few grid
    sizes, each timed with HIP events over 5 launches after one untimed."""
    n = gib << 30
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
        moe.moe_hbm_read_probe(buf, sink, blocks)
        reps = 5
        ev = ([torch.cuda.Event(enable_timing=True) for _ in range(reps)],
              [torch.cuda.Event(enable_timing=True) for _ in range(reps)])
        h = moe.moe_timing_arm("read_probe", *ev)
        for _ in range(reps):
            moe.moe_hbm_read_probe(buf, sink, blocks)
        torch.cuda.synchronize()
        assert moe.moe_timing_disarm(h) == reps
        t = float(np.mean([s_.elapsed_time(e_) for s_, e_ in zip(*ev)])) * 1e-3
        gbps = n / t / 1e9
        if best is None or gbps > best["GBps"]:
            best = {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                    "bytes": n, "blocks": blocks}
    del buf
    torch.cuda.empty_cache()
    best["kind"] = ("plain streaming read kernel (16-byte non-temporal loads, 8 in flight per "
                    "lane), best grid of 1024/2048/4096/8192 blocks x 256 threads")
    return best


def ffn_launch_durations(moe, torch, K, step):
    """Per-step seconds of the gate/up and the down projection over K steps:
    HIP events around every launch of each kernel (the single-token GEMV, or
    the grouped GEMM's thin and M-blocked launches, summed per step)."""
    kinds = {"gateup": ("gateup", "gateup_thin"), "down": ("down", "down_thin")}
    names = [n for v in kinds.values() for n in v]
    ev = {n: ([torch.cuda.Event(enable_timing=True) for _ in range(K)],
              [torch.cuda.Event(enable_timing=True) for _ in range(K)]) for n in names}
    arms = {n: moe.moe_timing_arm(n, *ev[n]) for n in names}
    torch.cuda.synchronize()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    counts = {n: moe.moe_timing_disarm(arms[n]) for n in names}
    out = {}
    for kind, parts in kinds.items():
        tot = np.zeros(K)
        for n in parts:
            assert counts[n] in (0, K), counts
            if counts[n] == K:
                tot += np.array([s.elapsed_time(e) for s, e in zip(*ev[n])]) * 1e-3
        assert tot.min() > 0, (kind, counts)
        out[kind] = tot
    return out


def mfma_figures(moe, torch, w, L0, g):
    """fp16 MFMA throughput of the grouped gate/up GEMM: for the whole layer
    (useful flops 2 * T*k * d * 2f over its measured launches), and for one
    expert alone at M = 512 tokens and at the token count of layer 0's hottest
    expert (from the layer call's own per-expert counts), each through
    moe_expert_ffn (same kernels) timed with HIP events over 20 launches."""
    dev = torch.device("cuda:0")
    dims = g["dims"]
    layer_flops = 2.0 * w.T * w.top_k * w.d * 2 * w.f
    layer_tflops = layer_flops / float(g["dur"].mean()) / 1e12
    cnt = g["hot_counts"]
    hot_e = int(np.argmax(cnt))
    xd = g["x0"]
    out = {"layer_gateup_tflops": round(layer_tflops, 1),
           "layer_gateup_frac": round(layer_tflops / MFMA_PEAK_TFLOPS, 4),
           "peak_tflops": MFMA_PEAK_TFLOPS, "dtype": "fp16 x fp16 -> fp32 (v_mfma_f32_16x16x32_f16)"}
    for label, e, n in (("m512", 0, 512), ("hot", hot_e, int(cnt[hot_e]))):
        n = min(n, xd.shape[0])
        blob = L0["blobs"][e]
        y = torch.empty(n, w.d, dtype=torch.float32, device=dev)
        ws = moe.make_workspace(dims, n, dev)
        for _ in range(3):
            moe.moe_expert_ffn(dims, blob, xd[:n], None, n, y, ws)
        reps = 20
        ev = ([torch.cuda.Event(enable_timing=True) for _ in range(reps)],
              [torch.cuda.Event(enable_timing=True) for _ in range(reps)])
        # int8 and int2 experts run the thin GEMM at every size
        kname = "gateup" if n > 16 and w.bits == 4 else "gateup_thin"
        h = moe.moe_timing_arm(kname, *ev)
        torch.cuda.synchronize()
        for _ in range(reps):
            moe.moe_expert_ffn(dims, blob, xd[:n], None, n, y, ws)
        torch.cuda.synchronize()
        assert moe.moe_timing_disarm(h) == reps
        t = float(np.mean([s_.elapsed_time(e_) for s_, e_ in zip(*ev)])) * 1e-3
        flops = 2.0 * n * w.d * 2 * w.f
        tf = flops / t / 1e12
        out[label] = {"expert": e, "M": n, "gateup_us": round(t * 1e6, 2), "tflops": round(tf, 1),
                      "frac": round(tf / MFMA_PEAK_TFLOPS, 4)}
    return out


HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction, published


def run_host_tier(a):
    """One layer's 256 experts at home in pinned host memory mapped into the
    device, behind an HBM cache of --host-tier slots.  Every step is a new
    batch of tokens (warm-up steps fill the cache); misses are copied from
    host memory by the library's fill kernel, hits are read from HBM.  The
    step rate includes the copies: what the layer costs when the experts
    do not all fit in HBM."""
    import ctypes

    import torch

    import int4_routed_expert_softmax_amd as moe
    from synth import configs

    w = configs.WORKLOADS[a.workload]
    if w.T > 8 or w.T * w.top_k > 64:
        sys.exit(f"--host-tier: {w.name} has T={w.T}, past the cached layer's batch limits")
    S = a.host_tier
    dev = torch.device("cuda:0")
    dims = moe.Dims(w.d, w.f, w.n_experts, w.top_k, group_size=w.group)
    blob = w.blob_bytes
    if not (min(w.n_experts, w.T * w.top_k) <= S <= w.n_experts):
        sys.exit(f"--host-tier {S}: slots must lie in [{min(w.n_experts, w.T * w.top_k)}, "
                 f"{w.n_experts}]")
    print(f"bench: {w.name} host tier, pinning {w.n_experts * blob / 1e9:.1f} GB of experts",
          file=sys.stderr, flush=True)
    blobs = configs.experts(w, 0)
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    hptr, dptr = ctypes.c_void_p(), ctypes.c_void_p()
    if hip.hipHostMalloc(ctypes.byref(hptr), ctypes.c_size_t(blobs.nbytes), ctypes.c_uint(2)) != 0:
        sys.exit("hipHostMalloc failed")
    try:
        ctypes.memmove(hptr, blobs.ctypes.data, blobs.nbytes)
        del blobs
        if hip.hipHostGetDevicePointer(ctypes.byref(dptr), hptr, ctypes.c_uint(0)) != 0:
            sys.exit("hipHostGetDevicePointer failed")
        home = torch.tensor([dptr.value + e * blob for e in range(w.n_experts)], dtype=torch.int64,
                            device=dev)
        Wr, bias = configs.router(w, 0)
        Wr, bias = torch.from_numpy(Wr).to(dev), torch.from_numpy(bias).to(dev)
        n = a.warmup + a.steps
        xs = [configs.tokens(w, s)[0] for s in range(n)]
        x = torch.from_numpy(np.stack(xs)).to(dev)  # [n][T][d]
        slots = torch.empty(S * blob, dtype=torch.uint8, device=dev)
        state = moe.make_cache_state(dims, S, dev)
        out = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
        ws = moe.make_workspace(dims, w.T, dev)

        flags = moe.MOE_INT8_ACT if a.int8_act else 0

        def step(i):
            moe.moe_layer_forward_cached(dims, x[i], Wr, bias, home, slots, S, state, out,
                                         flags=flags, ws=ws)

        for i in range(a.warmup):
            step(i)
        torch.cuda.synchronize()
        h0 = moe.cache_header(state)
        t0 = time.perf_counter()
        for i in range(a.warmup, n):
            step(i)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / a.steps
        h1 = moe.cache_header(state)
    finally:
        torch.cuda.synchronize()
        hip.hipHostFree(hptr)
    hits, misses = h1["hits"] - h0["hits"], h1["misses"] - h0["misses"]
    host_bytes = misses * blob / a.steps
    host_gbps = host_bytes / sec / 1e9
    res = {
        "metric": METRIC, "value": round(w.T / sec, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("int4 weights x int8 activations (one scale per 64 columns), i32 dot, f32 "
                  "accumulate" if a.int8_act else
                  "int4 weights x int8-digit activations, i32 dot, f32 accumulate"),
        "data": "synthetic (seeded; random-init GLM-5.2-shaped experts)",
        "config": {"workload": f"{w.name} host tier: one layer, d={w.d} f={w.f} E={w.n_experts} "
                               f"top-{w.top_k}, T={w.T}, experts in pinned host memory behind "
                               f"{S} HBM slots, a new batch of tokens per step"
                               + (", MOE_INT8_ACT" if a.int8_act else ""),
                   "T": w.T, "d": w.d, "f": w.f, "n_experts": w.n_experts, "top_k": w.top_k,
                   "slots": S},
        "cache": {"hit_rate": round(hits / max(hits + misses, 1), 4),
                  "hits_per_step": round(hits / a.steps, 3),
                  "misses_per_step": round(misses / a.steps, 3),
                  "host_bytes_per_step": round(host_bytes),
                  # copied bytes over the whole step time (copies and compute):
                  # a lower bound on the link rate the copy kernel reaches
                  "host_GBps_over_step": round(host_gbps, 2),
                  "host_link_peak_GBps": HOST_LINK_PEAK_GBPS},
    }
    print(json.dumps(res), flush=True)


def run_chain(a):
    """48 chained decode layers, h <- h + MoE_l(RMSNorm(h)), one token per
    step, all 48 x 256 experts resident.  Each step starts from a fresh seeded
    h0; layer 0 reads it and writes h in place for the other 47.  The timed
    steps are one HIP graph of K x 48 layer calls."""
    import torch

    import int4_routed_expert_softmax_amd as moe
    from synth import configs

    w = configs.WORKLOADS["chain48"]
    dev = torch.device("cuda:0")
    dims = moe.Dims(w.d, w.f, w.n_experts, w.top_k, group_size=w.group)
    blob = w.blob_bytes
    nib_gu, nib_dn = matrix_bytes(w)
    L = w.layers
    K, Wm = a.steps, a.warmup
    eps = 1e-6
    flags = moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL | (moe.MOE_INT8_ACT if a.int8_act else 0)
    print(f"bench: chain48 generating + uploading {L * w.n_experts * blob / 1e9:.1f} GB",
          file=sys.stderr, flush=True)
    layers = []
    t_up = time.perf_counter()
    for l in range(L):
        Wr, bias = configs.router(w, l)
        blobs = torch.from_numpy(configs.experts(w, l)).to(dev)
        table = torch.tensor([blobs[e].data_ptr() for e in range(w.n_experts)], dtype=torch.int64,
                             device=dev)
        layers.append((torch.from_numpy(Wr).to(dev), torch.from_numpy(bias).to(dev), blobs, table))
        print(f"bench: layer {l} resident ({time.perf_counter() - t_up:.0f} s)", file=sys.stderr,
              flush=True)
    n_h0 = Wm + K
    h0 = torch.from_numpy(np.concatenate([configs.tokens(w, s % 64)[0] for s in range(n_h0)])).to(dev)
    h = torch.empty(n_h0, w.d, dtype=torch.float32, device=dev)
    stats = torch.zeros(n_h0, L, 1 + w.n_experts, dtype=torch.int32, device=dev)
    ws = moe.make_workspace(dims, 1, dev)

    def step(s, stream):
        for l in range(L):
            Wr, bias, _, table = layers[l]
            x = h0[s:s + 1] if l == 0 else h[s:s + 1]
            moe.moe_layer_forward(dims, x, Wr, bias, table, h[s:s + 1], flags=flags, rms_eps=eps,
                                  stats=stats[s, l], ws=ws, stream=stream)

    cur = torch.cuda.current_stream()
    for s in range(Wm):
        step(s, cur.cuda_stream)
    torch.cuda.synchronize()

    # eager timing of the same K steps (launch-bound reference)
    t0 = time.perf_counter()
    for s in range(Wm, Wm + K):
        step(s, cur.cuda_stream)
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / K

    # the timed region: one replay of a graph holding the K steps
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for s in range(Wm, Wm + K):
            step(s, side.cuda_stream)
    torch.cuda.synchronize()
    g.replay()  # warm replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = (t1 - t0) / K
    U = stats[Wm:, :, 0].cpu().numpy().astype(np.float64)  # [K][L]
    weight_bytes_step = U.sum(axis=1).mean() * blob

    # instrumented eager pass: HIP events around every gate/up and down launch.
    # Enqueuing a 48-layer step with events takes the host longer than the GPU
    # takes to run it; a drained queue would stamp each start event while the
    # GPU waits for the host.  So every step is enqueued behind a spin kernel
    # that lasts longer than the enqueue, and its 144 launches run back to back.
    t_enq = time.perf_counter()
    step(Wm, cur.cuda_stream)
    t_enq = time.perf_counter() - t_enq
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1 << 20)
    e1.record()
    torch.cuda.synchronize()
    spin_per_s = (1 << 20) / (e0.elapsed_time(e1) * 1e-3)
    spin = int(min(3.0 * t_enq * spin_per_s, 1 << 34))
    n_launch = K * L
    ev = {k: ([torch.cuda.Event(enable_timing=True) for _ in range(n_launch)],
              [torch.cuda.Event(enable_timing=True) for _ in range(n_launch)]) for k in ("gateup", "down")}
    arms = {k: moe.moe_timing_arm(k, *ev[k]) for k in ev}
    for s in range(Wm, Wm + K):
        torch.cuda._sleep(spin)
        step(s, cur.cuda_stream)
    torch.cuda.synchronize()
    counts = {k: moe.moe_timing_disarm(arms[k]) for k in arms}
    assert all(c == n_launch for c in counts.values()), counts
    dur = {k: np.array([x.elapsed_time(y) for x, y in zip(*ev[k])]) * 1e-3 for k in ev}
    for k in dur:
        q = np.percentile(dur[k], [10, 50, 90, 99]) * 1e6
        print(f"bench: chain48 {k} event us p10 {q[0]:.2f} p50 {q[1]:.2f} p90 {q[2]:.2f} "
              f"p99 {q[3]:.2f}; by layer mean " +
              " ".join(f"{v:.1f}" for v in dur[k].reshape(K, L).mean(axis=0)[:6] * 1e6) + " ...",
              file=sys.stderr, flush=True)
    u_launch = U.reshape(-1)
    gu_gbps = float(np.mean(u_launch * nib_gu / dur["gateup"]) / 1e9)
    dn_gbps = float(np.mean(u_launch * nib_dn / dur["down"]) / 1e9)

    res = {
        "metric": METRIC,
        "value": round(1.0 / sec, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4 weights x int8 activations (one scale per 64 columns, as int8 digits), "
                  "i32 dot, f32 accumulate" if a.int8_act else
                  "int4 weights x int8-digit activations, i32 dot, f32 accumulate" if w.T <= 8 else
                  "int4 weights dequantised to fp16 x fp16 activations, MFMA f32 accumulate"),
        "data": "synthetic (seeded; random-init GLM-5.2-shaped experts, 48 fresh layers)",
        "config": {"workload": f"chain48: {L} chained decode layers h <- h + MoE(RMSNorm(h)), T=1, "
                               f"d={w.d} f={w.f} E={w.n_experts} top-{w.top_k}, all "
                               f"{L * w.n_experts} experts resident ({L * w.n_experts * blob / 1e9:.1f} GB), "
                               f"one HIP graph of {K} steps" + (", MOE_INT8_ACT" if a.int8_act else ""),
                   "T": 1, "d": w.d, "f": w.f, "n_experts": w.n_experts, "top_k": w.top_k,
                   "layers": L, "distinct_experts_per_layer": float(U.mean())},
        "ms_per_step_eager": round(eager * 1e3, 4),
        "expert_weight_GBps": round(weight_bytes_step / sec / 1e9, 1),
        "expert_weight_frac_hbm_peak": round(weight_bytes_step / sec / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "gateup (gate+up projections, SwiGLU)",
                     "achieved": round(gu_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gu_gbps / HBM_PEAK_GBPS, 4), "traffic": committed_traffic("decode1"),
                     "bytes_per_launch": float(u_launch.mean() * nib_gu),
                     "avg_launch_us": round(float(dur["gateup"].mean() * 1e6), 3)},
        "roofline_down": {"bound": "hbm", "achieved": round(dn_gbps, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(dn_gbps / HBM_PEAK_GBPS, 4),
                          "bytes_per_launch": float(u_launch.mean() * nib_dn),
                          "avg_launch_us": round(float(dur["down"].mean() * 1e6), 3)},
    }
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_baseline_chain(w, a.cpu_seconds, a.int8_act)
    print(json.dumps(res), flush=True)


def cpu_baseline_chain(w, seconds, i8=False):
    """The CPU oracle on the chain: layer after layer of step 0 (RMSNorm,
    residual; i8: integer activations), each layer's experts generated on
    demand, until `seconds` have passed; tokens/s = layers/s / 48."""
    import oracle
    from synth import configs

    h, _ = configs.tokens(w, 0)
    n = 0
    t_ffn = 0.0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n < w.layers:
        Wr, bias = configs.router(w, n)
        idx, _, _ = oracle.route(oracle.rmsnorm(h, 1e-6), Wr, bias, w.top_k)
        table = [None] * w.n_experts
        for e in set(int(e) for e in idx.reshape(-1)):
            table[e] = configs.one_expert(w, n, e)
        t1 = time.perf_counter()
        h = oracle.layer_forward(h, Wr, bias, table, w.d, w.f, w.top_k,
                                 flags=3 | (oracle.I8ACT if i8 else 0),
                                 eps=1e-6)["out"].astype(np.float32)
        t_ffn += time.perf_counter() - t1
        n += 1
    cores = oracle.omp_threads()
    return {"value": round(n / t_ffn / w.layers, 5), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n} chained layers of step 0 (fp64 C oracle, OpenMP over output rows; "
                      f"expert generation excluded), {t_ffn:.1f} s"}


def cpu_baseline(w, seconds):
    """The CPU oracle, as it is, on single-token layer forwards of layer 0 of
    the same workload, repeated until `seconds` have passed."""
    import oracle
    from synth import configs

    Wr, bias = configs.router(w, 0)
    table = list(configs.experts(w, 0))
    x, bf = configs.tokens(w, 0)

    def run(secs):
        n = 0
        t0 = time.perf_counter()
        while True:
            t = n % x.shape[0]
            oracle.layer_forward(x[t:t + 1], Wr, bias, table, w.d, w.f, w.top_k, x_bf16=bf,
                                 group=w.group)
            n += 1
            if time.perf_counter() - t0 >= secs:
                break
        return n, time.perf_counter() - t0

    cores = oracle.omp_threads()
    n, dt = run(seconds)
    # the same oracle on one thread, over a quarter of the time
    oracle.omp_threads(1)
    n1, dt1 = run(seconds / 4)
    oracle.omp_threads(cores)
    return {"value": round(n / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} single-token forwards of {w.name} layer 0 (fp64 C oracle, OpenMP over "
                      f"output rows), {dt:.1f} s",
            "value_1thread": round(n1 / dt1, 4),
            "sample_1thread": f"{n1} forwards on 1 thread, {dt1:.1f} s",
            "cpu_model": cpu_model()}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
