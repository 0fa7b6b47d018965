"""GPU: per-row int4 experts (scale group 0: one fp16 scale per weight row, the
nxmr blog's per-row scaling, «纯C语言») on every path of the library, against
the CPU oracle, to the same bar as the gs64 experts: routing, union and counts
bit-exact, outputs within 2e-3 * max|ref|.  A per-row expert must also give
bit for bit what the gs64 expert with its row scale repeated over the row's
groups gives: the kernels do the same arithmetic on the same numbers."""
import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
from synth import configs

from moe_harness import DEV, DeviceLayer, assert_close, say
from test_gpu_parity import full_parity, small

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS


@pytest.mark.parametrize("w", [
    small("pr_t1", 256, 128, 16, 2, 1, group=0),               # one token: digit GEMVs
    small("pr_gemv_T5", 320, 192, 32, 4, 5, group=0),          # a small batch on the GEMVs
    small("pr_gemv_T40", 320, 192, 64, 4, 40, group=0),        # a batch past the small limits
    small("pr_mfma_T5", 512, 1024, 32, 8, 5, group=0, x_kind="bf16"),  # 2-wave grouped GEMM
    small("pr_mfma_T70", 1024, 512, 64, 8, 70, group=0),       # 16-wave grouped GEMM
    small("pr_kE", 128, 64, 16, 16, 3, zipf=False, group=0),
], ids=lambda w: w.name)
def test_perrow_small_shapes(w):
    full_parity(w)


@pytest.mark.parametrize("w", [small("pr_chain", 256, 128, 16, 2, 5, group=0),
                               small("pr_chain_mfma", 512, 512, 16, 4, 24, group=0)],
                         ids=lambda w: w.name)
def test_perrow_prenorm_residual(w):
    full_parity(w, flags=moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL)


def _as_gs64(blobs, d, f):
    fd = f * d
    out = []
    for b in blobs:
        s_all = b[3 * fd // 2:].view(np.float16)
        sc = np.concatenate([np.repeat(s_all[:f], d // 64), np.repeat(s_all[f:2 * f], d // 64),
                             np.repeat(s_all[2 * f:], f // 64)])
        out.append(np.concatenate([b[:3 * fd // 2], sc.view(np.uint8)]))
    return np.stack(out)


@pytest.mark.parametrize("T", [1, 4, 40])
def test_perrow_equals_gs64_with_repeated_scales(T):
    w = small(f"pr_eq_T{T}", 512, 512, 32, 4, T, group=0)
    w64 = small(f"g64_eq_T{T}", 512, 512, 32, 4, T)
    L = DeviceLayer(w)
    L64 = DeviceLayer(w64, blobs=_as_gs64(L.blobs, w.d, w.f))
    x, bf = configs.tokens(w)
    out, st = L.forward(L.x_device(x, bf))
    out64, st64 = L64.forward(L64.x_device(x, bf))
    torch.cuda.synchronize()
    assert torch.equal(st, st64)
    assert torch.equal(out, out64), "per-row and repeated-scale gs64 outputs differ"


@pytest.mark.parametrize("n", [3, 21, 150])
def test_perrow_single_expert(n):
    # n = 3: GEMVs; 21: grouped GEMM, 16-wave blocks; 150: 4-wave blocks
    w = W["decode1_perrow"]
    d, f = w.d, w.f
    blob = configs.one_expert(w, 0, 11)
    dims = moe.Dims(d, f, w.n_experts, w.top_k, group_size=0)
    assert moe.expert_blob_bytes(dims) == blob.size
    xf = np.random.default_rng(n).normal(size=(n, d)).astype(np.float32)
    y = torch.empty(n, d, dtype=torch.float32, device=DEV)
    say(f"per-row expert_ffn n={n}")
    moe.moe_expert_ffn(dims, torch.from_numpy(blob).to(DEV), torch.from_numpy(xf).to(DEV), None, n,
                       y, moe.make_workspace(dims, n, DEV))
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(blob, xf.astype(np.float64), d, f, group=0)
    rel = assert_close(y.cpu().numpy(), ref, f"per-row expert_ffn n={n}")
    say(f"per-row expert_ffn n={n} rel err {rel:.2e}")


def test_perrow_batch_invariant():
    w = small("pr_inv", 512, 512, 32, 4, 6, group=0)
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    xd = L.x_device(x, bf)
    out, _ = L.forward(xd, flags=moe.MOE_BATCH_INVARIANT)
    for t in range(w.T):
        o1, _ = L.forward(xd[t:t + 1].contiguous())
        assert torch.equal(out[t], o1[0]), f"token {t} differs from its one-token call"


def test_glm_decode1_perrow():
    full_parity(W["decode1_perrow"])


def test_glm_verify8_perrow():
    full_parity(W["verify8_perrow"])
