"""GPU: moe_layer_forward_noalloc, the layer call on the library's own
per-GPU workspace (for callers that cannot allocate), against
moe_layer_forward on a caller workspace with the same inputs.

The two run the same kernels on the same numbers, so outputs, counts and
routing must be bit-identical.  Two calls follow each other on the shared
array, the second smaller than the first (it then sees the first call's
leftovers); a call past the array's size is refused."""
import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
from synth import configs

from moe_harness import DEV, DeviceLayer, say

pytestmark = pytest.mark.gpu

NORM_RES = moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL


def noalloc(L: DeviceLayer, xd, flags=0):
    T = xd.shape[0]
    out = torch.full((T, L.w.d), float("nan"), dtype=torch.float32, device=DEV)
    stats = torch.full((1 + L.w.n_experts,), -1, dtype=torch.int32, device=DEV)
    moe.moe_layer_forward_noalloc(L.dims, xd, L.Wr_d, L.bias_d, L.table, out, flags=flags,
                                  stats=stats)
    torch.cuda.synchronize()
    return out, stats


def same(L: DeviceLayer, x, bf, flags, what):
    xd = L.x_device(np.ascontiguousarray(x), bf)
    say(f"noalloc: {what} T={xd.shape[0]} flags={flags}")
    got, gst = noalloc(L, xd.clone(), flags)
    ref, rst = L.forward(xd.clone(), flags=flags)
    assert torch.equal(gst, rst), f"{what}: counts differ from moe_layer_forward"
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)), \
        f"{what}: output differs from moe_layer_forward"


def test_glm_batch_then_single_token():
    # GLM-5.2 shape: 8 tokens on the grouped GEMM, then one token on the
    # GEMV path (and its RMSNorm + residual form), on the same array
    L = DeviceLayer(configs.WORKLOADS["verify8"])
    x, bf = configs.tokens(L.w)
    same(L, x, bf, 0, "verify8")
    same(L, x[5:6], bf, 0, "decode after verify8")
    same(L, x[2:3], bf, NORM_RES, "decode, RMSNorm + residual")
    # integer activations: int8 rows on the array, then the digit form
    same(L, x, bf, moe.MOE_INT8_ACT, "verify8, int8 activations")
    same(L, x[1:2], bf, moe.MOE_INT8_ACT, "decode, int8 activations")


def test_large_batch_then_small_batch():
    # batches past the small-batch limits (split logits, top-k and union
    # kernels), then a batch of 3
    w = configs.Workload("na_long", d=1024, f=512, n_experts=64, top_k=8, T=300, seed=51)
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    same(L, x, bf, 0, "T=300")
    same(L, x[10:13], bf, moe.MOE_BATCH_INVARIANT, "T=3 batch-invariant")


@pytest.mark.parametrize("bits", [8, 2])
def test_other_code_widths_batch_then_single_token(bits):
    # int8 / int2 codes: a batch on the thin grouped GEMM, then one token and
    # a batch-invariant batch on the single-token kernels, on the same array
    w = configs.Workload(f"na_i{bits}", d=512, f=1024, n_experts=32, top_k=8, T=12, seed=52,
                         bits=bits)
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    same(L, x, bf, 0, f"int{bits} T=12")
    same(L, x[4:5], bf, 0, f"int{bits} decode")
    same(L, x[:5], bf, moe.MOE_BATCH_INVARIANT, f"int{bits} T=5 batch-invariant")


def test_refuses_calls_past_the_array():
    dims = moe.Dims(6144, 2048, 256, 8)
    assert moe.workspace_bytes(dims, 64) <= moe.NOALLOC_SCRATCH_BYTES
    assert moe.workspace_bytes(dims, 512) > moe.NOALLOC_SCRATCH_BYTES
    L = DeviceLayer(configs.WORKLOADS["tiny"])
    x = torch.zeros(512, 256, dtype=torch.float32, device=DEV)
    out = torch.empty(512, 6144, dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(dims, x, L.Wr_d, None, L.table, out)
    assert e.value.code == moe.MOE_ENOSPC
