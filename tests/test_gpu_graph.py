"""GPU: layer calls captured in a HIP graph give, on every replay, bit for bit
what the same calls give when enqueued directly.  The library enqueues only
kernels and allocates nothing, so a serving loop (and bench.py's timed
region) may capture its steps; replays are interleaved with eager work and
synchronisations, and every replay is checked."""
import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
from synth import configs

from moe_harness import DEV, DeviceLayer, say
from test_gpu_parity import small

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w,flags", [
    (small("g_t1", 256, 128, 16, 2, 1), 0),                          # one token: GEMV path
    (small("g_t1_res", 256, 128, 16, 2, 1), moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL),
    (small("g_t4", 512, 512, 16, 4, 4), 0),                          # small batch, grouped GEMM
    (small("g_t40", 1024, 512, 64, 8, 40, x_kind="bf16"), 0),        # large batch, grouped GEMM
    (small("g_inv", 512, 512, 32, 4, 6), moe.MOE_BATCH_INVARIANT),
    (small("g_perrow", 512, 512, 32, 8, 5, group=0), 0),
    (small("g_i8act_t3", 512, 512, 16, 4, 3), moe.MOE_INT8_ACT),   # integer activations
    (small("g_i8act_t40", 1024, 512, 64, 8, 40, x_kind="bf16"), moe.MOE_INT8_ACT),
    (small("g_int2_t1", 512, 512, 16, 4, 1, bits=2), 0),           # int2 codes on the GEMV
    (small("g_int8_t1", 512, 512, 16, 4, 1, bits=8), 0),           # int8 codes on the GEMV
    (small("g_int2_inv", 512, 512, 16, 4, 5, bits=2), moe.MOE_BATCH_INVARIANT),
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_graph_replays_match_eager(w, flags):
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    xd = L.x_device(x, bf)
    ws = moe.make_workspace(L.dims, w.T, DEV)
    out = torch.empty(w.T, w.d, dtype=torch.float32, device=DEV)
    stats = torch.zeros(1 + w.n_experts, dtype=torch.int32, device=DEV)

    def call(stream):
        moe.moe_layer_forward(L.dims, xd, L.Wr_d, L.bias_d, L.table, out, flags=flags,
                              stats=stats, ws=ws, stream=stream)

    cur = torch.cuda.current_stream()
    call(cur.cuda_stream)
    torch.cuda.synchronize()
    ref, ref_st = out.clone(), stats.clone()

    side = torch.cuda.Stream()
    side.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call(side.cuda_stream)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        stats.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}: output differs from the eager call"
        assert torch.equal(stats, ref_st), f"replay {r}: counts differ"
        call(cur.cuda_stream)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    say(f"graph: {w.name} flags={flags}: 4 replays bit-identical to the eager call")
