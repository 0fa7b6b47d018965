"""GPU: MOE_BATCH_INVARIANT, a batched verify that computes exactly the
single-token function.

Drafted tokens are produced one at a time; verifying them in one batch is only
sound if every token of the batch gets the result the one-token call gave it
(README 工作原理 › 诚实的推测解码: drafts and their verification must compute
the same function, pinned to one kernel family).  With the flag, each token's
output row and its per-expert counts must be bit-identical to a T = 1 call on
that token alone, for every batch size up to the small-batch limits, both
input dtypes, RMSNorm + residual and in place.  The batch itself is also held
to the oracle's tolerance, since the flag sends GLM-shaped batches down a path
that batches otherwise do not take.
"""
import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
from synth import configs

from moe_harness import DEV, DeviceLayer, assert_close, check_layer_routing, say

pytestmark = pytest.mark.gpu

INV = moe.MOE_BATCH_INVARIANT
NORM_RES = moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL


def bits(a: torch.Tensor) -> np.ndarray:
    return a.detach().cpu().numpy().view(np.uint32)


def one_by_one(L: DeviceLayer, xd: torch.Tensor, flags: int, in_place: bool):
    """Each token through its own T = 1 call (the decode call, no flag)."""
    T = xd.shape[0]
    outs, cnt = [], np.zeros(L.w.n_experts, np.int64)
    ws = moe.make_workspace(L.dims, 1, DEV)
    for t in range(T):
        xt = xd[t:t + 1].clone()
        out, st = L.forward(xt, flags=flags, ws=ws, out=xt if in_place else None)
        outs.append(bits(out)[0])
        s = st.cpu().numpy()
        assert s[0] == np.count_nonzero(s[1:])
        cnt += s[1:]
    return np.stack(outs), cnt


def check(L: DeviceLayer, x: np.ndarray, bf: bool, flags: int, in_place=False, ref=True):
    w = L.w
    say(f"batch invariance: {w.name} d={w.d} f={w.f} E={w.n_experts} k={w.top_k} T={x.shape[0]} "
        f"flags={flags} bf16={bf} in_place={in_place}")
    xd = L.x_device(x, bf)
    solo, cnt = one_by_one(L, xd, flags, in_place)
    xb = xd.clone()
    out, st = L.forward(xb, flags=flags | INV, out=xb if in_place else None)
    inv_ws = L.last_ws
    got = bits(out)
    for t in range(x.shape[0]):
        assert np.array_equal(got[t], solo[t]), (
            f"token {t}: batched output differs from its single-token output in "
            f"{np.count_nonzero(got[t] != solo[t])} of {w.d} values")
    s = st.cpu().numpy()
    assert np.array_equal(s[1:], cnt), "per-expert counts differ from the single-token calls"
    assert s[0] == np.count_nonzero(cnt)
    plain, _ = L.forward(xd.clone(), flags=flags)
    say(f"batch invariance: without the flag {np.count_nonzero(bits(plain) != got)} of "
        f"{got.size} output values differ from the single-token ones")
    if ref:
        r = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k, x_bf16=bf,
                                 flags=flags)
        assert s[0] == r["U"]
        check_layer_routing(L.dims, inv_ws, x.shape[0], r, f"{w.name} batch-invariant call")
        assert_close(out.cpu().numpy(), r["out"], case=f"{w.name} INV flags={flags}")


@pytest.fixture(scope="module")
def verify8():
    return DeviceLayer(configs.WORKLOADS["verify8"])


@pytest.mark.parametrize("flags", [0, NORM_RES])
def test_verify8_batch_matches_single_tokens(verify8, flags):
    # 8 drafted tokens sharing a base (the verify step's inputs), GLM-5.2 shape
    x, bf = configs.tokens(verify8.w)
    check(verify8, x, bf, flags)


@pytest.mark.parametrize("T", [2, 3, 5])
def test_every_batch_size(verify8, T):
    x, bf = configs.tokens(verify8.w, step=T)
    check(verify8, x[:T], bf, NORM_RES, ref=False)


def test_in_place_with_residual(verify8):
    x, bf = configs.tokens(verify8.w, step=11)
    check(verify8, x[:4], bf, NORM_RES, in_place=True, ref=False)


@pytest.mark.parametrize("w", [
    # d, f multiples of 512: batches would otherwise take the matrix-core path
    configs.Workload("inv_d512_bf16", d=512, f=512, n_experts=64, top_k=8, T=6, seed=31,
                     x_kind="bf16"),
    # d not a multiple of 512, many experts, odd top-k
    configs.Workload("inv_d320_E300", d=320, f=192, n_experts=300, top_k=5, T=7, seed=32),
    # the batch limit T * k = 64
    configs.Workload("inv_k32_T2", d=256, f=128, n_experts=96, top_k=32, T=2, seed=33),
    # rows past 8192 columns: the router's streamed (not register-held) rows
    # and two column passes in gate/up
    configs.Workload("inv_d10240", d=10240, f=192, n_experts=16, top_k=2, T=3, seed=34),
], ids=lambda w: w.name)
def test_small_shapes(w):
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    check(L, x, bf, 0)
    if not bf:
        check(L, x, bf, NORM_RES)


def test_same_tokens_twice(verify8):
    # a batch holding one token twice: both rows equal its single-token output
    x, bf = configs.tokens(verify8.w, step=5)
    check(verify8, np.ascontiguousarray(np.stack([x[0], x[1], x[0]])), bf, NORM_RES, ref=False)
