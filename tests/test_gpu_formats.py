"""GPU: int8 and int2 expert codes (the nxmr blog's hand-written int8 and
packed int2 kernels next to packed int4, «纯C语言») on every path the layer
call takes for them, against the CPU oracle with the same code width: routing,
union and slot lists bit-exact (as the call left them in its workspace),
outputs within 2e-3 * max|ref|.  Both widths run one token (and, with
MOE_BATCH_INVARIANT, batches of up to 8) on the single-token kernel family,
as int4 layers do, with 8 (int2) or 32 (int8) bytes of codes per 32-column
chunk, and other batches on the thin grouped GEMM in 16-token tiles.  With
MOE_BATCH_INVARIANT every token of a batch is compared bit for bit with its
one-token call."""
import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
import synth
from synth import configs

from moe_harness import DEV, DeviceLayer, assert_close, check_layer_routing, say
from test_gpu_parity import full_parity, small

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS
NORM_RES = moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL


@pytest.mark.parametrize("bits", [8, 2])
@pytest.mark.parametrize("shape", [
    dict(name="t1", d=512, f=512, E=16, k=2, T=1),
    dict(name="T5_bf16", d=512, f=1024, E=32, k=8, T=5, x_kind="bf16"),
    dict(name="T40", d=1024, f=512, E=64, k=8, T=40),          # large batch: split logits
    dict(name="hot", d=512, f=512, E=8, k=1, T=70),            # experts over several tiles
    dict(name="kE", d=512, f=512, E=16, k=16, T=3, zipf=False),
    dict(name="perrow_T9", d=512, f=512, E=32, k=4, T=9, group=0),
], ids=lambda v: v["name"] if isinstance(v, dict) else f"int{v}")
def test_formats_small_shapes(bits, shape):
    sh = dict(shape)
    name = sh.pop("name")
    full_parity(small(f"i{bits}_{name}", **sh, bits=bits))


@pytest.mark.parametrize("bits", [8, 2])
def test_formats_prenorm_residual(bits):
    w = small(f"i{bits}_chain", 512, 512, 16, 4, 6, bits=bits)
    full_parity(w, flags=NORM_RES)


@pytest.mark.parametrize("bits", [8, 2])
@pytest.mark.parametrize("n", [1, 3, 20, 40])
def test_formats_single_expert(bits, n):
    d, f = 1024, 512
    dims = moe.Dims(d, f, 16, 2, code_bits=bits)
    blob = synth.expert_blob(21, 0, 5, d, f, bits=bits)
    assert moe.expert_blob_bytes(dims) == blob.size
    xf = np.random.default_rng(n + bits).normal(size=(n, d)).astype(np.float32)
    y = torch.empty(n, d, dtype=torch.float32, device=DEV)
    say(f"int{bits} expert_ffn n={n}")
    moe.moe_expert_ffn(dims, torch.from_numpy(blob).to(DEV), torch.from_numpy(xf).to(DEV), None, n,
                       y, moe.make_workspace(dims, n, DEV))
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(blob, xf.astype(np.float64), d, f, bits=bits)
    rel = assert_close(y.cpu().numpy(), ref, f"int{bits} expert_ffn n={n}",
                       case=f"int{bits} expert_ffn n={n}")
    say(f"int{bits} expert_ffn n={n} rel err {rel:.2e}")


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("bits", [8, 2])
@pytest.mark.parametrize("flags", [moe.MOE_BATCH_INVARIANT, NORM_RES | moe.MOE_BATCH_INVARIANT])
def test_formats_batch_matches_single_tokens(bits, flags):
    w = small(f"i{bits}_inv", 512, 512, 32, 8, 8, bits=bits, x_kind="shared_base")
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
    say(f"int{bits} flags={flags}: {w.T} tokens bit-identical to their one-token calls")


@pytest.mark.parametrize("bits", [8, 2])
@pytest.mark.parametrize("shape,flags", [
    (dict(name="t1_bf16", d=512, f=1024, E=32, k=8, T=1, x_kind="bf16"), 0),
    (dict(name="t1_perrow", d=512, f=512, E=16, k=4, T=1, group=0), 0),
    (dict(name="t1_c1", d=1536, f=512, E=16, k=2, T=1), 0),    # one column slice; 24-row down blocks (int2)
    (dict(name="t1_wide", d=8192, f=4096, E=8, k=4, T=1), 0),  # two passes over gate/up and down rows
    (dict(name="t1_res", d=512, f=512, E=16, k=4, T=1), NORM_RES),
    (dict(name="t1_k16", d=512, f=512, E=64, k=16, T=1), 0),   # two experts per down wave
    (dict(name="inv_T5", d=512, f=1024, E=32, k=8, T=5), moe.MOE_BATCH_INVARIANT),
    (dict(name="inv_T8_perrow", d=1024, f=512, E=32, k=4, T=8, group=0),
     NORM_RES | moe.MOE_BATCH_INVARIANT),
], ids=lambda v: v["name"] if isinstance(v, dict) else f"flags{v}")
def test_other_widths_on_the_single_token_kernels(bits, shape, flags):
    """int8 and int2 codes on the digit GEMV: one token, and batch-invariant
    batches."""
    sh = dict(shape)
    name = sh.pop("name")
    full_parity(small(f"i{bits}_{name}", **sh, bits=bits), flags=flags)


@pytest.mark.parametrize("name", ["decode1_int8", "verify8_int8", "decode1_int2", "verify8_int2"])
def test_formats_glm(name):
    full_parity(W[name])


@pytest.mark.parametrize("bits", [8, 2])
def test_formats_glm_prefill512_every_token(bits):
    name = f"prefill512_int{bits}"
    w = W[name]
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    say(f"{name}: layer call")
    out, st = L.forward(L.x_device(x, bf))
    say(f"{name}: oracle over all 512 tokens")
    ref = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k, x_bf16=True,
                               bits=bits)
    assert st[0].item() == ref["U"]
    check_layer_routing(L.dims, L.last_ws, w.T, ref, f"{name} layer call")
    rel = assert_close(out.cpu().numpy(), ref["out"], name, case=f"{name} flags=0")
    say(f"{name}: U={ref['U']} rel err {rel:.2e}")


def test_cached_layer_refuses_other_code_widths():
    dims = moe.Dims(512, 512, 16, 2, code_bits=8)
    dummy = torch.zeros(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_cached(dims, torch.zeros(1, 512, device=DEV), torch.zeros(16, 512, device=DEV),
                                     None, torch.zeros(16, dtype=torch.int64, device=DEV),
                                     torch.zeros(4 * moe.expert_blob_bytes(dims), dtype=torch.uint8,
                                                 device=DEV), 4,
                                     torch.zeros(1024, dtype=torch.int32, device=DEV),
                                     torch.zeros(1, 512, device=DEV),
                                     ws=moe.make_workspace(dims, 1, DEV))
    assert e.value.code == moe.MOE_EUNSUPPORTED
    del dummy
