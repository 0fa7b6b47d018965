"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: routing indices, union lists and per-expert slot lists (ties to the
lower expert id), both from moe_route / moe_union and as the layer call itself
left them in its workspace (the lists its expert kernels walked: the
single-token gate/up prologue, the small-batch routing block, or the large-batch
top-k and union kernels).  Floating point: layer and expert outputs within
max-abs-error <= 2e-3 * max|ref| (the oracle is fp64); router weights within
1e-6 relative.  Full-size GLM-5.2-shaped layers (d=6144, f=2048, 256 experts,
top-8) run at batch 1, 8 and 512, each compared in full.
"""
import ctypes

import numpy as np
import pytest
import torch

import int4_routed_expert_softmax_amd as moe
import oracle
import synth
from synth import configs

from moe_harness import (DEV, DeviceLayer, assert_close, check_layer_routing, check_union,
                         record_margin, say)

pytestmark = pytest.mark.gpu

W = configs.WORKLOADS


def small(name, d, f, E, k, T, zipf=True, seed=7, x_kind="normal", group=64, bits=4):
    return configs.Workload(name, d=d, f=f, n_experts=E, top_k=k, T=T, seed=seed, zipf=zipf,
                            x_kind=x_kind, group=group, bits=bits)


def full_parity(w: configs.Workload, flags=0, layer=None):
    say(f"parity: {w.name} d={w.d} f={w.f} E={w.n_experts} k={w.top_k} T={w.T} flags={flags}")
    L = layer or DeviceLayer(w)
    x, bf = configs.tokens(w)
    xd = L.x_device(x, bf)
    ref = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k, x_bf16=bf,
                               flags=flags, group=w.group, bits=w.bits)
    if not flags:
        idx, wts = L.route(xd)
        assert np.array_equal(idx, ref["idx"]), "routing indices differ"
        np.testing.assert_allclose(wts, ref["w"], rtol=1e-6, atol=1e-7)
        check_union(L, idx)
    out, stats = L.forward(xd, flags=flags)
    st = stats.cpu().numpy()
    assert st[0] == ref["U"]
    cnt = np.zeros(w.n_experts, np.int64)
    np.add.at(cnt, ref["idx"].reshape(-1), 1)
    assert np.array_equal(st[1:], cnt)
    check_layer_routing(L.dims, L.last_ws, w.T, ref, f"{w.name} layer call")
    rel = assert_close(out.cpu().numpy(), ref["out"], case=f"{w.name} flags={flags}")
    say(f"parity: {w.name} U={ref['U']} rel err {rel:.2e}")
    return L, ref, out


def test_tiny_layer():
    full_parity(W["tiny"])


@pytest.mark.parametrize("w", [
    small("t1", 256, 128, 16, 2, 1),
    small("ragged", 320, 192, 100, 5, 130),
    small("k1", 256, 128, 16, 1, 9),
    small("kE", 128, 64, 16, 16, 3, zipf=False),
    small("wide", 2112, 704, 64, 8, 70),
    # rows wider than one pass of the gate/up blocks (192 chunks of 32)
    small("wide8192_t1", 8192, 256, 16, 2, 1),
    small("wide8192_T3", 8192, 320, 16, 2, 3),
    small("wide10240", 10240, 192, 16, 2, 20),
    small("wide10240_t1", 10240, 192, 16, 2, 1),  # router rows past 8192 columns
    small("bf16", 256, 128, 32, 4, 33, x_kind="bf16"),
    # multi-token batches on the grouped-GEMM path (d, f multiples of 512)
    small("mfma", 512, 512, 16, 4, 40),
    small("mfma_ragged", 1024, 512, 64, 8, 75),
    small("mfma_bf16", 512, 1024, 32, 4, 37, x_kind="bf16"),
    small("mfma_k1_hot", 512, 512, 8, 1, 70),
    # batches of 2..16 tokens on the grouped GEMM's small block shape
    small("mfma_T2", 512, 512, 16, 4, 2),
    small("mfma_T5_bf16", 512, 1024, 32, 8, 5, x_kind="bf16"),
    small("mfma_T16", 1024, 512, 64, 8, 16, zipf=False),
    # rows past the pack's 6144-column register path (max, then convert): x
    # packed beside the router (small batch) and by the pack kernel, and a
    small("mfma_x7168_T5", 7168, 512, 16, 4, 5),
    small("mfma_x7168", 7168, 512, 16, 4, 40),
    small("mfma_a7168", 512, 7168, 16, 4, 12),
    # small batches whose top-k merges several 64-expert groups
    small("small_E1024_k4", 256, 128, 1024, 4, 2),
    small("small_E300_k5", 256, 128, 300, 5, 3),
    small("small_E64_k32", 256, 128, 64, 32, 2, zipf=False),
    # the ABI's limits: 1024 experts, top-32 (a batch union beyond one wave)
    small("maxE_k32", 256, 128, 1024, 32, 3),
    small("maxE_k32_mfma", 512, 512, 1024, 32, 12, zipf=False),
    # a long batch: 1500 tokens x 8 picks over 256 experts, uniform and skewed
    small("long1500", 512, 512, 256, 8, 1500, zipf=False),
    small("long1500_zipf", 512, 512, 256, 8, 1500),
], ids=lambda w: w.name)
def test_edge_shapes(w):
    full_parity(w)


@pytest.mark.parametrize("w", [small("chainlike", 256, 128, 16, 2, 5),
                               small("chainlike_mfma", 512, 512, 16, 4, 24),
                               small("chainlike_mfma_T4", 512, 512, 16, 4, 4)],
                         ids=lambda w: w.name)
def test_prenorm_residual(w):
    full_parity(w, flags=moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL)
    full_parity(w, flags=moe.MOE_PRENORM_RMS)
    full_parity(w, flags=moe.MOE_RESIDUAL)


def test_all_ties_choose_lowest_ids():
    w = small("ties", 256, 128, 16, 4, 6, zipf=False)
    L = DeviceLayer(w, Wr=np.zeros((16, 256), np.float32), bias=None)
    x, _ = configs.tokens(w)
    idx, wts = L.route(L.x_device(x, False))
    assert np.array_equal(idx, np.tile(np.arange(4), (6, 1)))
    assert np.all(wts == np.float32(0.25))


@pytest.mark.parametrize("E,k,T", [(300, 5, 3), (1024, 4, 2), (256, 8, 1), (64, 32, 2),
                                   # batches past the small limits: summed logit ranges,
                                   # then one wave's bitonic top-k per token
                                   (300, 5, 20), (1024, 4, 17)])
def test_small_batch_ties_across_groups(E, k, T):
    # zero router rows: each logit is its bias, 1 for the last expert of
    # every 64-expert group and 0 elsewhere, so the picks are those experts
    # in id order, then the lowest ids: ties within and across groups, all
    # decided by the lower-id rule, in the layer call's own top-k and in
    # moe_route's
    w = small(f"ties_E{E}_k{k}", 256, 128, E, k, T, zipf=False)
    bias = (np.arange(E) % 64 == 63).astype(np.float32)
    L = DeviceLayer(w, Wr=np.zeros((E, 256), np.float32), bias=bias)
    full_parity(w, layer=L)


def test_output_aligned_to_4_bytes_only():
    # out starts one float into its allocation: the combine takes its scalar
    # form (the 16-byte one needs an aligned out)
    w = small("unaligned_out", 512, 512, 16, 4, 20)
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    buf = torch.full((w.T * w.d + 1,), -7.0, dtype=torch.float32, device=DEV)
    out = buf[1:].view(w.T, w.d)
    L.forward(L.x_device(x, bf), out=out)
    ref = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k, x_bf16=bf)
    assert_close(out.cpu().numpy(), ref["out"])
    assert buf[0].item() == -7.0


def test_zero_down_with_residual_leaves_h_unchanged():
    w = small("zerodown", 256, 128, 16, 2, 3)
    blobs = configs.experts(w).copy()
    nib, nsc = synth.blob_sizes(w.d, w.f)
    per = nsc // 3
    blobs[:, nib + 4 * per: nib + 6 * per] = 0  # down scales = +0.0
    L = DeviceLayer(w, blobs=blobs)
    h = configs.tokens(w)[0] * 3
    hd = L.x_device(h, False)
    out, _ = L.forward(hd, flags=moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL)
    assert torch.equal(out.cpu(), torch.from_numpy(h))


@pytest.mark.parametrize("w", [small("inplace", 256, 128, 16, 2, 4),
                               small("inplace_mfma", 512, 512, 16, 4, 20),
                               small("inplace_mfma_T3", 512, 512, 16, 2, 3)],
                         ids=lambda w: w.name)
def test_in_place_residual(w):
    L = DeviceLayer(w)
    h = configs.tokens(w)[0]
    hd = L.x_device(h, False)
    ref, _ = L.forward(hd.clone(), flags=moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL)
    L.forward(hd, flags=moe.MOE_PRENORM_RMS | moe.MOE_RESIDUAL, out=hd)
    assert torch.equal(hd, ref)


# ---------------------------------------------------------------- GLM-shaped


@pytest.fixture(scope="module")
def decode_layer():
    return DeviceLayer(W["decode1"])


def test_glm_decode_batch1(decode_layer):
    full_parity(W["decode1"], layer=decode_layer)


def test_glm_decode_deterministic_and_placement_invariant(decode_layer):
    L = decode_layer
    x, _ = configs.tokens(W["decode1"])
    xd = L.x_device(x, False)
    a, _ = L.forward(xd)
    b, _ = L.forward(xd)
    assert torch.equal(a, b), "two runs differ"
    # the same bytes at other device addresses: a reversed copy of the expert array
    moved = torch.flip(L.blobs_d, dims=[0]).contiguous()
    E = W["decode1"].n_experts
    L2 = DeviceLayer.__new__(DeviceLayer)
    L2.__dict__.update(L.__dict__)
    L2.table = torch.tensor([moved[E - 1 - e].data_ptr() for e in range(E)], dtype=torch.int64,
                            device=DEV)
    c, _ = L2.forward(xd)
    assert torch.equal(a, c), "output depends on where the expert bytes live"


def test_glm_expert_ffn_device_and_host_mapped(decode_layer):
    w = W["decode1"]
    L = decode_layer
    e = 3
    blob = L.blobs[e]
    x = configs.tokens(W["verify8"])[0][:5]
    xd = torch.from_numpy(x).to(DEV)
    rows = torch.tensor([4, 0, 2], dtype=torch.int32, device=DEV)
    y = torch.empty(3, w.d, dtype=torch.float32, device=DEV)
    ws = moe.make_workspace(L.dims, 3, DEV)
    moe.moe_expert_ffn(L.dims, L.blobs_d[e], xd, rows, 3, y, ws)
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(blob, x[[4, 0, 2]].astype(np.float64), w.d, w.f)
    rel = assert_close(y.cpu().numpy(), ref, "expert_ffn")
    say(f"expert_ffn GLM n=3 rel err {rel:.2e}")

    # the same blob in pinned host memory mapped into the device address space
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    hptr = ctypes.c_void_p()
    assert hip.hipHostMalloc(ctypes.byref(hptr), ctypes.c_size_t(blob.size), ctypes.c_uint(2)) == 0
    try:
        ctypes.memmove(hptr, blob.ctypes.data, blob.size)
        dptr = ctypes.c_void_p()
        assert hip.hipHostGetDevicePointer(ctypes.byref(dptr), hptr, ctypes.c_uint(0)) == 0
        y2 = torch.empty_like(y)
        moe.moe_expert_ffn(L.dims, dptr.value, xd, rows, 3, y2, ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "host-mapped blob gives a different result"
    finally:
        torch.cuda.synchronize()
        hip.hipHostFree(hptr)

    # bf16 input
    xb = synth.to_bf16_bits(x)
    xbd = torch.from_numpy(xb.view(np.int16)).to(DEV).view(torch.bfloat16)
    y3 = torch.empty(5, w.d, dtype=torch.float32, device=DEV)
    moe.moe_expert_ffn(L.dims, L.blobs_d[e], xbd, None, 5, y3, moe.make_workspace(L.dims, 5, DEV))
    torch.cuda.synchronize()
    ref3 = oracle.expert_ffn(blob, configs.bf16_bits_to_f32(xb).astype(np.float64), w.d, w.f)
    assert_close(y3.cpu().numpy(), ref3, "expert_ffn bf16")


def test_glm_expert_ffn_batched_mfma(decode_layer):
    """Single expert over several rows (the grouped-GEMM path): gathered fp32
    batches spanning three 64-token M-blocks with a ragged tail, one and two
    16-token M-blocks (the small block shape), and a bf16 batch."""
    w = W["decode1"]
    L = decode_layer
    xb, _ = configs.tokens(W["prefill512"])          # bf16 bits [512][d]
    xf = configs.bf16_bits_to_f32(xb)
    rng = np.random.default_rng(5)
    for e, n in [(0, 150), (77, 21), (3, 2), (200, 13)]:
        sel = rng.choice(xf.shape[0], size=n, replace=False).astype(np.int32)
        xd = torch.from_numpy(np.ascontiguousarray(xf * 1.5)).to(DEV)
        rows = torch.from_numpy(sel).to(DEV)
        y = torch.empty(n, w.d, dtype=torch.float32, device=DEV)
        say(f"expert_ffn batched: expert {e} n={n} fp32 gathered")
        moe.moe_expert_ffn(L.dims, L.blobs_d[e], xd, rows, n, y, moe.make_workspace(L.dims, n, DEV))
        torch.cuda.synchronize()
        ref = oracle.expert_ffn(L.blobs[e], (xf[sel] * 1.5).astype(np.float64), w.d, w.f)
        rel = assert_close(y.cpu().numpy(), ref, f"expert_ffn batched e={e} n={n}")
        say(f"expert_ffn batched: expert {e} n={n} rel err {rel:.2e}")
    n = 40
    xbd = torch.from_numpy(xb[:n].view(np.int16)).to(DEV).view(torch.bfloat16)
    y = torch.empty(n, w.d, dtype=torch.float32, device=DEV)
    say(f"expert_ffn batched: expert 5 n={n} bf16")
    moe.moe_expert_ffn(L.dims, L.blobs_d[5], xbd, None, n, y, moe.make_workspace(L.dims, n, DEV))
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(L.blobs[5], xf[:n].astype(np.float64), w.d, w.f)
    rel = assert_close(y.cpu().numpy(), ref, "expert_ffn batched bf16")
    say(f"expert_ffn batched: bf16 n={n} rel err {rel:.2e}")


def test_glm_verify_batch8():
    L, ref, _ = full_parity(W["verify8"])
    say(f"verify8: union of {ref['U']} distinct experts for 64 picks")


def test_glm_prefill512_every_token():
    """The 512-token prefill chunk in full: routing and union through
    moe_route / moe_union and as the layer call left them, and every output
    value of all 512 tokens against one batched oracle layer."""
    w = W["prefill512"]
    L = DeviceLayer(w)
    x, bf = configs.tokens(w)
    xd = L.x_device(x, bf)
    say("prefill512: routing 512 tokens")
    idx, wts = L.route(xd)
    ridx, rw, _ = oracle.route(x, L.Wr, L.bias, w.top_k, x_bf16=True)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(wts, rw, rtol=1e-6, atol=1e-7)
    U = check_union(L, idx)
    say(f"prefill512: U = {U}; layer call")
    out, stats = L.forward(xd)
    assert stats[0].item() == U
    out = out.cpu().numpy()
    say("prefill512: oracle layer over all 512 tokens")
    ref = oracle.layer_forward(x, L.Wr, L.bias, L.oracle_table(), w.d, w.f, w.top_k, x_bf16=True)
    check_layer_routing(L.dims, L.last_ws, w.T, ref, "prefill512 layer call")
    rel = assert_close(out, ref["out"], "prefill512 all tokens", case="prefill512 flags=0")
    # per-token margins too: the worst token against its own max|ref|
    per_tok = np.abs(out - ref["out"]).max(axis=1) / np.abs(ref["out"]).max(axis=1)
    record_margin("prefill512 worst token (own max|ref|)", float(per_tok.max()))
    say(f"prefill512: U={U} rel err {rel:.2e} (worst token against its own max: "
        f"{per_tok.max():.2e})")


def _disjoint_layer(name, d, f, E, k, T):
    """Router rows and tokens that send token t to experts k t .. k t + k - 1
    (every logit of those is 10, every other 0, so the ties inside a token are
    decided by the lower id): T * k distinct picks."""
    w = small(name, d, f, E, k, T, zipf=False)
    Wr = np.zeros((E, d), np.float32)
    for e in range(T * k):
        Wr[e, e // k] = 1.0
    L = DeviceLayer(w, Wr=Wr, bias=None)
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), np.arange(T)] = 10.0
    return w, L, x


@pytest.mark.parametrize("d,f,E,k,T", [
    (256, 128, 64, 8, 8),      # GEMV path, 8 tokens x 8 picks, every pick distinct
    (256, 128, 1024, 32, 2),   # GEMV path, top-32 of 1024
    (512, 512, 64, 8, 8),      # grouped-GEMM path (routing block + M-block map)
    (512, 512, 1024, 32, 2),
])
def test_union_of_64_distinct_picks(d, f, E, k, T):
    """A small batch whose T * k = 64 picks are all different experts (U = 64,
    one past the last lane of the union wave) with and without the
    batch-invariant flag: the layer's own union lists bit-exact, outputs in
    tolerance."""
    w, L, x = _disjoint_layer(f"disjoint_d{d}_E{E}_k{k}_T{T}", d, f, E, k, T)
    say(f"parity: {w.name}")
    ref = oracle.layer_forward(x, L.Wr, None, L.oracle_table(), d, f, k)
    assert ref["U"] == 64
    xd = L.x_device(x, False)
    for flags in (0, moe.MOE_BATCH_INVARIANT):
        out, st = L.forward(xd, flags=flags)
        assert st[0].item() == 64
        check_layer_routing(L.dims, L.last_ws, T, ref, f"{w.name} flags={flags}")
        rel = assert_close(out.cpu().numpy(), ref["out"], case=f"{w.name} flags={flags}")
        say(f"parity: {w.name} flags={flags} U=64 rel err {rel:.2e}")


@pytest.mark.parametrize("counts,x_kind", [
    ((16, 17, 1, 64, 65), "normal"),  # both sides of the thin limit and of a 64-token M-block
    ((3, 16, 2, 40), "bf16"),
])
def test_thin_and_mblocked_experts_side_by_side(counts, x_kind):
    """Token counts chosen per expert (top-1, every token of expert e sends
    its logit to e alone): experts of at most 16 tokens run on the thin
    grouped GEMM, larger ones on the M-blocked GEMM, in the same call."""
    E, d, f = len(counts), 512, 1024
    T = sum(counts)
    w = small(f"counts_{'_'.join(map(str, counts))}", d, f, E, 1, T, zipf=False, x_kind=x_kind)
    Wr = np.zeros((E, d), np.float32)
    Wr[np.arange(E), np.arange(E)] = 1.0
    L = DeviceLayer(w, Wr=Wr, bias=None)
    x = configs.tokens(w)[0]
    xf = configs.bf16_bits_to_f32(x) if x_kind == "bf16" else x.copy()
    owner = np.repeat(np.arange(E), counts)
    xf[:, :E] = 0.0
    xf[np.arange(T), owner] = 10.0
    xin = synth.to_bf16_bits(xf) if x_kind == "bf16" else xf
    say(f"parity: {w.name} T={T}")
    ref = oracle.layer_forward(xin, Wr, None, L.oracle_table(), d, f, 1, x_bf16=x_kind == "bf16")
    assert np.array_equal(np.bincount(ref["idx"].reshape(-1), minlength=E), counts)
    out, st = L.forward(L.x_device(xin, x_kind == "bf16"))
    assert np.array_equal(st.cpu().numpy()[1:], counts)
    check_layer_routing(L.dims, L.last_ws, T, ref, f"{w.name} layer call")
    rel = assert_close(out.cpu().numpy(), ref["out"], case=f"{w.name} flags=0")
    say(f"parity: {w.name} rel err {rel:.2e}")
