"""GPU parity of the chained decode h <- h + MoE_l(RMSNorm(h)) over the 48
GLM-5.2-shaped layers of the chain workload (d=6144, f=2048, 256 experts,
top-8, fresh seeded router and experts per layer), teacher-forced.

Every layer runs the call the chain benchmark makes: moe_layer_forward with
MOE_PRENORM_RMS | MOE_RESIDUAL, in place (x and out the same buffer), T=1.
Before each layer the oracle routes RMSNorm(h_l) of the GPU's own h_l in fp64;
only the experts it selects are made resident, every other table entry points
at one all-zero blob, so the GPU must pick exactly the same experts (its
per-expert counts are compared too) or its output is wrong.  On the checked
layers the oracle also runs the whole layer on h_l and the GPU output must
match within 2e-3 * max|ref|.  The GPU output is the next layer's input, so a
small fp32 difference never compounds into a different route (teacher
forcing); free-running divergence is not a parity question.
"""
import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
from synth import configs

from moe_harness import DEV, REL_TOL, check_layer_routing, record_margin, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

W = configs.WORKLOADS["chain48"]
EPS = 1e-6
FLAGS = moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL


class Chain:
    def __init__(self):
        self.dims = moe.Dims(W.d, W.f, W.n_experts, W.top_k)
        self.blob_bytes = moe.expert_blob_bytes(self.dims)
        self.ws = moe.make_workspace(self.dims, 1, DEV)
        self.zero = torch.zeros(self.blob_bytes, dtype=torch.uint8, device=DEV)
        self.stats = torch.zeros(1 + W.n_experts, dtype=torch.int32, device=DEV)

    def layer(self, layer: int, h: np.ndarray, check_output: bool, flags=FLAGS) -> np.ndarray:
        Wr, bias = configs.router(W, layer)
        idx, wts, _ = oracle.route(oracle.rmsnorm(h, EPS), Wr, bias, W.top_k)
        sel = sorted(set(int(e) for e in idx.reshape(-1)))
        host = {e: configs.one_expert(W, layer, e) for e in sel}
        resident = torch.from_numpy(np.stack([host[e] for e in sel])).to(DEV)
        ptrs = [self.zero.data_ptr()] * W.n_experts
        for i, e in enumerate(sel):
            ptrs[e] = resident[i].data_ptr()
        table = torch.tensor(ptrs, dtype=torch.int64, device=DEV)
        hd = torch.from_numpy(np.ascontiguousarray(h, dtype=np.float32)).to(DEV)
        self.stats.zero_()
        moe.moe_layer_forward(self.dims, hd, torch.from_numpy(Wr).to(DEV),
                              torch.from_numpy(bias).to(DEV), table, hd, flags=flags,
                              rms_eps=EPS, stats=self.stats, ws=self.ws)
        torch.cuda.synchronize()
        st = self.stats.cpu().numpy()
        cnt = np.bincount(idx.reshape(-1), minlength=W.n_experts)
        assert st[0] == len(sel), f"layer {layer}: U {st[0]} != {len(sel)}"
        assert np.array_equal(st[1:], cnt), f"layer {layer}: per-expert counts differ"
        uq, offs, rows = oracle.union(idx, W.n_experts)
        check_layer_routing(self.dims, self.ws, 1, dict(idx=idx, w=wts, U=len(uq), uniq=uq,
                                                        offsets=offs, rows=rows),
                            f"chain layer {layer}")
        out = hd.cpu().numpy()
        if check_output:
            ref = oracle.layer_forward(h, Wr, bias, [host.get(e) for e in range(W.n_experts)],
                                       W.d, W.f, W.top_k, flags=flags, eps=EPS)
            # the layer's own contribution h_{l+1} - h_l is what the experts compute
            got = out.astype(np.float64) - h
            want = ref["out"] - h
            err = np.abs(got - want).max()
            tol = REL_TOL * np.abs(want).max()
            assert err <= tol, f"layer {layer}: max abs err {err:.3e} > {tol:.3e}"
            rel = err / np.abs(want).max()
            self.worst = max(getattr(self, "worst", 0.0), rel)
            say(f"chain: layer {layer} experts {sel} rel err {rel:.2e}")
        return out


@pytest.fixture(scope="module")
def chain():
    return Chain()


@pytest.mark.parametrize("step", [0, 1, 63], ids=["step0", "step1", "step63"])
def test_chain_teacher_forced(chain, step):
    """Every one of the 48 layers of the step: routing, union and counts
    bit-exact, the layer's contribution within tolerance."""
    h, _ = configs.tokens(W, step)
    say(f"chain: step {step}, h0 |h|max {np.abs(h).max():.3f}")
    chain.worst = 0.0
    for layer in range(W.layers):
        h = chain.layer(layer, h, True)
    assert np.all(np.isfinite(h))
    record_margin(f"chain48 step {step} worst of 48 layers", chain.worst)
    say(f"chain: step {step} done, |h|max {np.abs(h).max():.3f}, worst rel err {chain.worst:.2e}")


def test_chain_teacher_forced_int8_activations(chain):
    """The same chain with MOE_INT8_ACT (each layer's experts on int8
    activations, the oracle's integer-activation layer as reference)."""
    h, _ = configs.tokens(W, 0)
    chain.worst = 0.0
    for layer in range(W.layers):
        h = chain.layer(layer, h, True, flags=FLAGS | moe.MOE_INT8_ACT)
    assert np.all(np.isfinite(h))
    record_margin("chain48 step 0 int8 activations worst of 48 layers", chain.worst)
    say(f"chain int8 activations: step 0 done, worst rel err {chain.worst:.2e}")
