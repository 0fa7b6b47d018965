"""GPU: integer activations (MOE_INT8_ACT; the pages' hand-written integer
dot-product kernels, int4 weights times integer activations — colibri 技术解读
(linlog.top), "int4 量化与手写内核"; the nxmr blog's int8 kernels, «纯C语言»).
Every expert input row (x', and a = silu(g) * u) is int8 per 64-column group
with an fp32 scale max|v| / 127, each group's dot product is exact on the
int8 matrix cores.  Against the oracle's integer-activation layer
(REF_I8ACT): routing, union and slot lists bit-exact (as the call left them
in its workspace), outputs within 2e-3 * max|ref|, on both kernel families
(one token and batch-invariant batches: the single-token GEMV with int8
digits; other batches: the int8 matrix cores), for int4, int8 and int2
codes.  Batch-invariant batches are bit-identical to their one-token calls, and the distance from the unquantised layer (the int8 rounding of the
activations) stays within its derived bound."""
import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
from synth import configs

from moe_harness import DEV, DeviceLayer, assert_close, check_layer_routing, record_margin, say
from test_gpu_parity import full_parity, small

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
I8 = moe.MOE_INT8_ACT
NORM_RES = moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL
# Distance of the integer-activation layer from the unquantised one, as a
# fraction of max|out|: each activation element moves by at most s/2 = max/254
# of its group; over a dot product these errors add like noise (rms about
# max/440 of each group), about 0.5% of an output of the same kind, twice
# (x', then a): about 1% at the largest outputs, bounded here at 3%.
I8_DIST = 3e-2


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("shape", [
    dict(name="t1", d=512, f=512, E=16, k=2, T=1),
    dict(name="T5_bf16", d=512, f=1024, E=32, k=8, T=5, x_kind="bf16"),
    dict(name="T40", d=1024, f=512, E=64, k=8, T=40),          # large batch: split logits
    dict(name="hot", d=512, f=512, E=8, k=1, T=70),            # experts over several M-tiles
    dict(name="kE", d=512, f=512, E=16, k=16, T=3, zipf=False),
    dict(name="perrow_T9", d=512, f=512, E=32, k=4, T=9, group=0),
], ids=lambda v: v["name"] if isinstance(v, dict) else f"int{v}")
def test_i8act_small_shapes(bits, shape):
    sh = dict(shape)
    name = sh.pop("name")
    full_parity(small(f"i8act_i{bits}_{name}", **sh, bits=bits), flags=I8)


@pytest.mark.parametrize("w", [
    small("i8act_t1_odd", 192, 128, 16, 2, 1),        # one token, d and f not multiples of 512
    small("i8act_T3_odd", 320, 192, 32, 4, 3),        # small batch on the single-token kernels
    small("i8act_ragged", 320, 192, 100, 5, 130),     # large batch: digit split + GEMV
], ids=lambda v: v.name)
def test_i8act_other_shapes_on_the_gemv(w):
    """Shapes off the matrix-core grid run the digit GEMV at every batch size,
    with the int8 values in its digit form."""
    full_parity(w, flags=I8)


def test_i8act_prenorm_residual():
    full_parity(small("i8act_chain", 512, 512, 16, 4, 6), flags=I8 | NORM_RES)


def test_i8act_zero_rows():
    """All-zero token rows: every group scale is 0, the codes 0, the output 0
    (plus the residual)."""
    w = small("i8act_zero", 512, 512, 16, 4, 5)
    L = DeviceLayer(w)
    x = np.zeros((w.T, w.d), np.float32)
    out, _ = L.forward(torch.from_numpy(x).to(DEV), flags=I8)
    ref = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k, flags=I8)
    assert not np.abs(ref["out"]).any()
    assert not out.abs().max().item()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("flags,bits", [
    (I8 | moe.MOE_BATCH_INVARIANT, 4),
    (I8 | NORM_RES | moe.MOE_BATCH_INVARIANT, 4),
    (I8 | moe.MOE_BATCH_INVARIANT, 8),
    (I8 | moe.MOE_BATCH_INVARIANT, 2),
])
def test_i8act_batch_matches_single_tokens(flags, bits):
    w = small(f"i8act_inv_i{bits}", 512, 512, 32, 8, 8, x_kind="shared_base", bits=bits)
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    xd = L.x_device(x, bf)
    ws1 = moe.make_workspace(L.dims, 1, DEV)
    solo = []
    for t in range(w.T):
        o, _ = L.forward(xd[t:t + 1].clone(), flags=flags & ~moe.MOE_BATCH_INVARIANT, ws=ws1)
        solo.append(bits_of(o)[0])
    out, _ = L.forward(xd.clone(), flags=flags)
    got = bits_of(out)
    for t in range(w.T):
        assert np.array_equal(got[t], solo[t]), f"token {t} differs from its one-token call"
    say(f"i8act int{bits} flags={flags}: {w.T} tokens bit-identical to their one-token calls")


@pytest.mark.parametrize("name,flags", [("decode1", I8), ("verify8", I8),
                                        ("verify8", I8 | moe.MOE_BATCH_INVARIANT)])
def test_i8act_glm(name, flags):
    L, ref, out = full_parity(W[name], flags=flags)
    # the quantised function's distance from the unquantised layer
    x, bf = configs.tokens(W[name])
    ref0 = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), L.w.d, L.w.f, L.w.top_k,
                                x_bf16=bf)
    dist = np.abs(out.cpu().numpy() - ref0["out"]).max() / np.abs(ref0["out"]).max()
    record_margin(f"{name} flags={flags} int8 activations vs unquantised layer", dist,
                  what="distance", tol=I8_DIST)
    say(f"{name}: int8-activation layer vs the unquantised one: {dist:.2e} of max|out|")
    assert dist <= I8_DIST


def test_i8act_glm_prefill512_every_token():
    w = W["prefill512"]
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    say("prefill512 int8 activations: layer call")
    out, st = L.forward(L.x_device(x, bf), flags=I8)
    say("prefill512 int8 activations: oracle over all 512 tokens")
    ref = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k, x_bf16=True,
                               flags=I8)
    assert st[0].item() == ref["U"]
    check_layer_routing(L.dims, L.last_ws, w.T, ref, "prefill512 int8 activations")
    rel = assert_close(out.cpu().numpy(), ref["out"], "prefill512 int8 activations",
                       case=f"prefill512 flags={I8}")
    say(f"prefill512 int8 activations: U={ref['U']} rel err {rel:.2e}")
