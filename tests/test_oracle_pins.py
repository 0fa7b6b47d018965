"""Pins of the CPU oracle against things other than itself: exhaustive
encodings, closed forms, special cases that reduce to textbook routines, brute
force on tiny inputs and the invariants the pages state.

Every oracle function is covered by at least one pin that a plausible slip
(dropped term, wrong sign, swapped index, transposed operand, gate/up swap,
wrong nibble order, wrong scale group) would fail.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth
from synth import configs

# ---------------------------------------------------------------- encodings


def test_nibble_decode_exhaustive():
    # closed form of a two's-complement nibble: ((n ^ 8) - 8)
    for b in range(256):
        row = np.array([b], dtype=np.uint8)
        assert oracle.nibble(row, 0) == ((b & 15) ^ 8) - 8
        assert oracle.nibble(row, 1) == ((b >> 4) ^ 8) - 8


def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ours = np.array([oracle.f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_decode():
    for b in [0x0000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0xC2F7]:
        ref = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        assert oracle.bf16(b) == float(ref)


# ------------------------------------------------------------- blob helpers


def np_dequant(blob, d, f, which):
    """Independent dense dequantisation with numpy vector ops."""
    fd = f * d
    rows, cols = (d, f) if which == 2 else (f, d)
    codes = blob[which * fd // 2:(which + 1) * fd // 2].reshape(rows, cols // 2)
    q = np.empty((rows, cols), dtype=np.int64)
    q[:, 0::2] = ((codes & 15).astype(np.int64) ^ 8) - 8
    q[:, 1::2] = ((codes >> 4).astype(np.int64) ^ 8) - 8
    sb = 3 * fd // 2
    n = fd // 64
    s = blob[sb + 2 * which * n: sb + 2 * (which + 1) * n].view(np.float16).astype(np.float64)
    s = np.repeat(s.reshape(rows, cols // 64), 64, axis=1)
    return q * s


def make_blob(d, f, codes=None, scales=None):
    """Blob from explicit int4 matrices (gate [f][d], up [f][d], down [d][f])
    and fp16 scale matrices, packed element 2i -> low nibble."""
    def pack(q):
        n = (np.asarray(q, dtype=np.int64) & 15).astype(np.uint8)
        return (n[:, 0::2] | (n[:, 1::2] << 4)).reshape(-1)

    nib = np.concatenate([pack(c) for c in codes])
    sc = np.concatenate([np.asarray(s, dtype=np.float16).reshape(-1) for s in scales])
    return np.concatenate([nib, sc.view(np.uint8)])


def np_silu(v):
    return v / (1.0 + np.exp(-v))


# -------------------------------------------------------------- dequant/FFN


@pytest.mark.parametrize("d,f", [(256, 128), (128, 192), (64, 64)])
def test_dequant_brute_force(d, f):
    blob = synth.expert_blob(3, 0, 1, d, f)
    for which in range(3):
        assert np.array_equal(oracle.dequant(blob, d, f, which), np_dequant(blob, d, f, which))


def test_one_hot_weight_gives_scale_times_input():
    d, f = 128, 64
    rng = np.random.default_rng(1)
    x = rng.normal(size=d)
    for r, c, q, s in [(0, 0, 1, 0.5), (5, 77, -8, 0.0078125), (63, 127, 7, 0.01953125)]:
        gate = np.zeros((f, d), int)
        gate[r, c] = q
        blob = make_blob(d, f, [gate, np.zeros((f, d)), np.zeros((d, f))],
                         [np.full((f, d // 64), s), np.ones((f, d // 64)), np.ones((d, f // 64))])
        W = oracle.dequant(blob, d, f, 0)
        assert W[r, c] == q * np.float16(s) and np.count_nonzero(W) == 1
        assert (W @ x)[r] == q * float(np.float16(s)) * x[c]


def test_swiglu_closed_form_with_permutations():
    """gate row r picks x[pg[r]], up row r picks x[pu[r]], down row c picks
    a[pd[c]]; then y[c] = sd*silu(sg*x[pg[pd[c]]]) * su*x[pu[pd[c]]].  d != f and
    distinct permutations catch transposed operands, swapped gate/up and
    wrong indices."""
    d, f = 128, 64
    rng = np.random.default_rng(2)
    pg = rng.permutation(d)[:f]
    pu = rng.permutation(d)[:f]
    pd = rng.integers(0, f, size=d)
    gate = np.zeros((f, d), int)
    up = np.zeros((f, d), int)
    down = np.zeros((d, f), int)
    gate[np.arange(f), pg] = 1
    up[np.arange(f), pu] = 1
    down[np.arange(d), pd] = 1
    sg, su, sd = 0.75, 0.375, 1.5
    blob = make_blob(d, f, [gate, up, down], [np.full((f, d // 64), sg), np.full((f, d // 64), su),
                                              np.full((d, f // 64), sd)])
    x = rng.normal(size=(3, d)) * 2
    y = oracle.expert_ffn(blob, x, d, f)
    for t in range(3):
        g = sg * x[t, pg[pd]]
        u = su * x[t, pu[pd]]
        ref = sd * (g / (1 + np.exp(-g))) * u
        np.testing.assert_allclose(y[t], ref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("d,f,n", [(256, 128, 3), (128, 64, 1), (192, 128, 2)])
def test_ffn_brute_force(d, f, n):
    blob = synth.expert_blob(4, 1, 2, d, f)
    x = np.random.default_rng(3).normal(size=(n, d))
    Wg, Wu, Wd = (np_dequant(blob, d, f, i) for i in range(3))
    ref = (np_silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    y = oracle.expert_ffn(blob, x, d, f)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ------------------------------------------------------ per-row scale format


def np_dequant_perrow(blob, d, f, which):
    """Independent dense dequantisation of a per-row blob: codes as for gs64,
    then the scales gate [f], up [f], down [d], one per row."""
    fd = f * d
    rows, cols = (d, f) if which == 2 else (f, d)
    codes = blob[which * fd // 2:(which + 1) * fd // 2].reshape(rows, cols // 2)
    q = np.empty((rows, cols), dtype=np.int64)
    q[:, 0::2] = ((codes & 15).astype(np.int64) ^ 8) - 8
    q[:, 1::2] = ((codes >> 4).astype(np.int64) ^ 8) - 8
    s_all = blob[3 * fd // 2:].view(np.float16).astype(np.float64)
    beg = [0, f, 2 * f][which]
    return q * s_all[beg:beg + rows][:, None]


def perrow_as_gs64(blob, d, f):
    """The gs64 blob with the same codes whose every 64-weight group carries
    its row's scale."""
    fd = f * d
    s_all = blob[3 * fd // 2:].view(np.float16)
    sg, su, sdn = s_all[:f], s_all[f:2 * f], s_all[2 * f:]
    sc = np.concatenate([np.repeat(sg, d // 64), np.repeat(su, d // 64), np.repeat(sdn, f // 64)])
    return np.concatenate([blob[:3 * fd // 2], sc.view(np.uint8)])


def test_perrow_blob_size_closed_form():
    for d, f in [(256, 128), (6144, 2048)]:
        assert oracle.blob_bytes(d, f, group=0) == 3 * f * d // 2 + 2 * (2 * f + d)
        assert synth.expert_blob(1, 0, 0, d, f, group=0).size == oracle.blob_bytes(d, f, group=0)
    assert oracle.blob_bytes(6144, 2048) == 20054016


@pytest.mark.parametrize("d,f", [(256, 128), (128, 192)])
def test_perrow_dequant_brute_force(d, f):
    blob = synth.expert_blob(3, 0, 1, d, f, group=0)
    for which in range(3):
        assert np.array_equal(oracle.dequant(blob, d, f, which, group=0),
                              np_dequant_perrow(blob, d, f, which))


def test_perrow_is_gs64_with_the_row_scale_in_every_group():
    """A per-row expert computes exactly what the gs64 expert with its row
    scale repeated over the row's groups computes (each weight q * s is the
    same exact number), through the FFN and the whole layer."""
    d, f, E, k, T = 256, 128, 16, 2, 5
    blobs = synth.layer_blobs(9, 0, E, d, f, group=0)
    g64 = [perrow_as_gs64(b, d, f) for b in blobs]
    x = np.random.default_rng(4).normal(size=(T, d))
    for e in (0, 7):
        assert np.array_equal(oracle.expert_ffn(blobs[e], x, d, f, group=0),
                              oracle.expert_ffn(g64[e], x, d, f))
    Wr = (np.random.default_rng(5).normal(size=(E, d)) * 0.02).astype(np.float32)
    xs = x.astype(np.float32)
    a = oracle.layer_forward(xs, Wr, None, list(blobs), d, f, k, group=0)
    b = oracle.layer_forward(xs, Wr, None, g64, d, f, k)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["idx"], b["idx"])


def test_perrow_ffn_brute_force():
    d, f, n = 192, 128, 3
    blob = synth.expert_blob(4, 1, 2, d, f, group=0)
    x = np.random.default_rng(3).normal(size=(n, d))
    Wg, Wu, Wd = (np_dequant_perrow(blob, d, f, i) for i in range(3))
    ref = (np_silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    y = oracle.expert_ffn(blob, x, d, f, group=0)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _set_scales(blob, d, f, which, value, group=None, row=None):
    b = blob.copy()
    fd = f * d
    sb = 3 * fd // 2
    n = fd // 64
    s = b[sb + 2 * which * n: sb + 2 * (which + 1) * n].view(np.float16)
    cols = f if which == 2 else d
    s2 = s.reshape(-1, cols // 64)
    if group is None:
        s2[...] = value if not callable(value) else value(s2)
    else:
        s2[:, group] = value
    return b


def test_zero_scale_group_removes_exactly_its_inputs():
    d, f = 256, 128
    blob = synth.expert_blob(5, 0, 0, d, f)
    x = np.random.default_rng(4).normal(size=(2, d))
    for g in range(d // 64):
        b0 = _set_scales(_set_scales(blob, d, f, 0, 0.0, group=g), d, f, 1, 0.0, group=g)
        x0 = x.copy()
        x0[:, 64 * g:64 * (g + 1)] = 0.0
        assert np.array_equal(oracle.expert_ffn(b0, x, d, f), oracle.expert_ffn(blob, x0, d, f))


def test_down_scale_doubling_doubles_output_exactly():
    d, f = 256, 128
    blob = synth.expert_blob(6, 0, 0, d, f)
    x = np.random.default_rng(5).normal(size=(2, d))
    b2 = _set_scales(blob, d, f, 2, lambda s: s * np.float16(2))
    assert np.array_equal(oracle.expert_ffn(b2, x, d, f), 2 * oracle.expert_ffn(blob, x, d, f))


def test_zero_gate_gives_zero_output():
    d, f = 256, 128
    b = _set_scales(synth.expert_blob(7, 0, 0, d, f), d, f, 0, 0.0)
    y = oracle.expert_ffn(b, np.random.default_rng(6).normal(size=(2, d)), d, f)
    assert np.all(y == 0.0)


def test_silu_limits_and_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1e3) == 1e3
    assert oracle.silu(-1e3) == 0.0 and np.signbit(oracle.silu(-1e3))
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16


# ------------------------------------------------------------------- router


def _np_topk(z, k):
    out = []
    for row in z:
        order = np.lexsort((np.arange(row.size), -row))  # -z ascending, then id
        out.append(order[:k])
    return np.array(out)


@pytest.mark.parametrize("T,d,E,k", [(4, 256, 16, 2), (7, 128, 64, 8), (3, 64, 256, 8)])
def test_route_brute_force(T, d, E, k):
    rng = np.random.default_rng(T * E)
    x = rng.normal(size=(T, d)).astype(np.float32)
    Wr = (0.02 * rng.normal(size=(E, d))).astype(np.float32)
    b = synth.zipf_bias(E)
    idx, w, z = oracle.route(x, Wr, b, k)
    zr = x.astype(np.float64) @ Wr.astype(np.float64).T + b.astype(np.float64)
    np.testing.assert_allclose(z, zr, rtol=0, atol=1e-13)
    assert np.array_equal(idx, _np_topk(z, k))
    p = softmax(zr, axis=1)
    ps = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(w, ps / ps.sum(1, keepdims=True), rtol=1e-13)


def test_route_all_ties_go_to_lowest_ids():
    E, d, k = 16, 64, 4
    x = np.random.default_rng(0).normal(size=(3, d)).astype(np.float32)
    idx, w, _ = oracle.route(x, np.zeros((E, d), np.float32), None, k)
    assert np.array_equal(idx, np.tile(np.arange(k), (3, 1)))
    assert np.all(w == 1.0 / k)


def test_route_partial_tie_breaks_to_lower_id():
    E, d, k = 8, 64, 3
    b = np.array([5, 1, 0, 3, 0, 3, 0, 0], np.float32)  # 3 and 5 tie for 2nd
    x = np.zeros((1, d), np.float32)
    idx, _, _ = oracle.route(x, np.zeros((E, d), np.float32), b, k)
    assert list(idx[0]) == [0, 3, 5]
    b[3] = 0.0  # now 5 is alone in 2nd place and 1 in 3rd
    idx, _, _ = oracle.route(x, np.zeros((E, d), np.float32), b, k)
    assert list(idx[0]) == [0, 5, 1]


def test_route_k_equals_E_is_plain_softmax():
    E, d = 32, 128
    rng = np.random.default_rng(8)
    x = rng.normal(size=(2, d)).astype(np.float32)
    Wr = rng.normal(size=(E, d)).astype(np.float32) * np.float32(0.02)
    idx, w, z = oracle.route(x, Wr, None, E)
    for t in range(2):
        np.testing.assert_allclose(w[t], softmax(z[t])[idx[t]], rtol=1e-14)
        assert np.all(np.diff(z[t, idx[t]]) <= 0)
        assert sorted(idx[t]) == list(range(E))


def test_route_k1_weight_is_one():
    rng = np.random.default_rng(9)
    x = rng.normal(size=(5, 64)).astype(np.float32)
    Wr = rng.normal(size=(16, 64)).astype(np.float32)
    idx, w, z = oracle.route(x, Wr, None, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(z, 1))


def test_renormalised_softmax_equals_softmax_of_selected_logits():
    rng = np.random.default_rng(10)
    x = rng.normal(size=(6, 256)).astype(np.float32)
    Wr = (0.05 * rng.normal(size=(64, 256))).astype(np.float32)
    idx, w, z = oracle.route(x, Wr, synth.zipf_bias(64), 8)
    for t in range(6):
        np.testing.assert_allclose(w[t], softmax(z[t, idx[t]]), rtol=1e-13)


def test_route_bf16_input_is_widened_exactly():
    rng = np.random.default_rng(11)
    x = rng.normal(size=(3, 128)).astype(np.float32)
    xb = synth.to_bf16_bits(x)
    xw = configs.bf16_bits_to_f32(xb)
    Wr = rng.normal(size=(16, 128)).astype(np.float32)
    i1, w1, z1 = oracle.route(xb, Wr, None, 2, x_bf16=True)
    i2, w2, z2 = oracle.route(xw, Wr, None, 2)
    assert np.array_equal(z1, z2) and np.array_equal(i1, i2) and np.array_equal(w1, w2)


# -------------------------------------------------------------------- union


def _naive_union(idx, k):
    s = sorted(set(idx.reshape(-1).tolist()))
    rows = []
    offs = [0]
    for e in s:
        rows += [t * k + j for t in range(idx.shape[0]) for j in range(k) if idx[t, j] == e]
        offs.append(len(rows))
    return np.array(s), np.array(offs), np.array(rows)


@pytest.mark.parametrize("T,E,k,seed", [(1, 256, 8, 0), (8, 256, 8, 1), (64, 16, 2, 2),
                                        (512, 256, 8, 3), (5, 8, 8, 4)])
def test_union_brute_force_and_invariants(T, E, k, seed):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    idx = np.array([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)],
                   dtype=np.int32)
    uniq, offs, rows = oracle.union(idx, E)
    nu, no, nr = _naive_union(idx, k)
    assert np.array_equal(uniq, nu) and np.array_equal(offs, no) and np.array_equal(rows, nr)
    assert offs[-1] == T * k and np.all(np.diff(offs) > 0)
    assert len(uniq) <= min(E, T * k)
    assert sorted(rows.tolist()) == list(range(T * k))
    for u in range(len(uniq)):
        r = rows[offs[u]:offs[u + 1]]
        assert np.all(idx.reshape(-1)[r] == uniq[u]) and np.all(np.diff(r // k) > 0)
    if T == 1:
        assert len(uniq) == k


# -------------------------------------------------------------- RMSNorm


def test_rmsnorm_closed_forms():
    h = np.full(64, 3.0, np.float32)
    assert np.all(oracle.rmsnorm(h, eps=0.0) == 1.0)
    h = np.array([3.0, -4.0] * 32, np.float32)
    xn = oracle.rmsnorm(h, eps=0.0)  # rms = 5/sqrt(2)
    np.testing.assert_allclose(xn, h / (5 / np.sqrt(2)), rtol=1e-7)
    h = np.random.default_rng(0).normal(size=6144).astype(np.float32) * 7
    ref = (h.astype(np.float64) / np.sqrt(np.mean(h.astype(np.float64) ** 2) + 1e-6)).astype(np.float32)
    assert np.array_equal(oracle.rmsnorm(h), ref)


# -------------------------------------------------------------- whole layer


def _tiny_layer(seed=0, E=16, d=256, f=128):
    rng = np.random.default_rng(seed)
    Wr = (0.02 * rng.normal(size=(E, d))).astype(np.float32)
    blobs = [synth.expert_blob(seed + 100, 0, e, d, f) for e in range(E)]
    return Wr, blobs


def test_layer_single_expert_equals_expert_ffn_exactly():
    d, f = 256, 128
    Wr, blobs = _tiny_layer()
    x = np.random.default_rng(1).normal(size=(1, d)).astype(np.float32)
    r = oracle.layer_forward(x, Wr, None, blobs, d, f, k=1)
    e = r["idx"][0, 0]
    assert np.array_equal(r["out"], oracle.expert_ffn(blobs[e], x, d, f))


def test_layer_k_equals_E_is_full_softmax_mixture():
    d, f, E = 128, 64, 8
    Wr, blobs = _tiny_layer(3, E, d, f)
    x = np.random.default_rng(2).normal(size=(2, d)).astype(np.float32)
    r = oracle.layer_forward(x, Wr, None, blobs, d, f, k=E)
    z = x.astype(np.float64) @ Wr.astype(np.float64).T
    ys = np.stack([oracle.expert_ffn(blobs[e], x, d, f) for e in range(E)], 1)  # [T][E][d]
    ref = (softmax(z, axis=1)[:, :, None] * ys).sum(1)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_layer_reads_each_distinct_expert_once():
    d, f = 256, 128
    Wr, blobs = _tiny_layer(4)
    x = np.random.default_rng(3).normal(size=(12, d)).astype(np.float32)
    r = oracle.layer_forward(x, Wr, synth.zipf_bias(16), blobs, d, f, k=2)
    reads = r["reads"]
    assert np.all(reads[r["uniq"]] == 1) and reads.sum() == r["U"]


def test_layer_output_independent_of_placement():
    d, f = 256, 128
    Wr, blobs = _tiny_layer(5)
    x = np.random.default_rng(4).normal(size=(4, d)).astype(np.float32)
    r1 = oracle.layer_forward(x, Wr, None, blobs, d, f, k=2)
    moved = [np.concatenate([np.zeros(37, np.uint8), b])[37:] for b in blobs]  # other addresses
    r2 = oracle.layer_forward(x, Wr, None, moved, d, f, k=2)
    assert np.array_equal(r1["out"], r2["out"])


def test_layer_unselected_experts_may_be_absent():
    d, f = 256, 128
    Wr, blobs = _tiny_layer(6)
    x = np.random.default_rng(5).normal(size=(2, d)).astype(np.float32)
    r1 = oracle.layer_forward(x, Wr, None, blobs, d, f, k=2)
    sparse = [b if e in set(r1["uniq"].tolist()) else None for e, b in enumerate(blobs)]
    r2 = oracle.layer_forward(x, Wr, None, sparse, d, f, k=2)
    assert np.array_equal(r1["out"], r2["out"])
    with pytest.raises(ValueError):
        oracle.layer_forward(x, Wr, None, [None] * 16, d, f, k=2)


def test_layer_residual_with_zero_down_leaves_h_unchanged():
    d, f = 256, 128
    Wr, blobs = _tiny_layer(7)
    blobs = [_set_scales(b, d, f, 2, 0.0) for b in blobs]
    h = np.random.default_rng(6).normal(size=(1, d)).astype(np.float32) * 3
    r = oracle.layer_forward(h, Wr, None, blobs, d, f, k=2,
                             flags=oracle.PRENORM | oracle.RESIDUAL)
    assert np.array_equal(r["out"].astype(np.float32), h)


def test_layer_prenorm_routes_on_normalised_input():
    d, f = 256, 128
    Wr, blobs = _tiny_layer(8)
    h = np.random.default_rng(7).normal(size=(3, d)).astype(np.float32) * 5
    r = oracle.layer_forward(h, Wr, None, blobs, d, f, k=2, flags=oracle.PRENORM)
    xn = np.stack([oracle.rmsnorm(row) for row in h])
    r2 = oracle.layer_forward(xn, Wr, None, blobs, d, f, k=2)
    assert np.array_equal(r["out"], r2["out"]) and np.array_equal(r["idx"], r2["idx"])


def test_tiny_workload_golden():
    """The tiny workload's outputs against the committed fixture written by
    tests/golden/make_golden.py (which calls only the oracle): guards the oracle
    against silent drift once its pins pass."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_layer.json")
    g = json.load(open(path))
    w = configs.WORKLOADS["tiny"]
    Wr, bias = configs.router(w)
    x, _ = configs.tokens(w)
    r = oracle.layer_forward(x, Wr, bias, list(configs.experts(w)), w.d, w.f, w.top_k)
    assert r["idx"].tolist() == g["idx"]
    assert r["uniq"].tolist() == g["uniq"] and r["rows"].tolist() == g["rows"]
    np.testing.assert_allclose(r["out"], np.array(g["out"]), rtol=1e-12, atol=1e-12)


# ------------------------------------------------- int8 and int2 code formats
# (the nxmr blog's hand-written int8 and packed int2 kernels, «纯C语言»)


def np_codes(packed_rows: np.ndarray, cols: int, bits: int) -> np.ndarray:
    """Independent unpacking: int8 = the byte as two's complement; int2 =
    four fields per byte, lowest first, two's complement of width 2."""
    b = packed_rows.astype(np.int64)
    if bits == 8:
        return np.where(b >= 128, b - 256, b)
    fields = np.stack([(b >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(b.shape[0], cols)
    return np.where(fields >= 2, fields - 4, fields)


def np_dequant_bits(blob, d, f, which, bits, group=64):
    fd = f * d
    cb = fd * bits // 8
    rows, cols = (d, f) if which == 2 else (f, d)
    q = np_codes(blob[which * cb:(which + 1) * cb].reshape(rows, cols * bits // 8), cols, bits)
    s_all = blob[3 * cb:].view(np.float16).astype(np.float64)
    if group:
        ng = [f * (d // 64), f * (d // 64), d * (f // 64)]
        beg = sum(ng[:which])
        s = s_all[beg:beg + ng[which]].reshape(rows, cols // 64)
        return q * np.repeat(s, 64, axis=1)
    beg = [0, f, 2 * f][which]
    return q * s_all[beg:beg + rows][:, None]


def test_int8_and_int2_decode_exhaustive():
    for b in range(256):
        row = np.array([b], np.uint8)
        assert oracle.code(row, 0, 8) == (b ^ 128) - 128
        for j in range(4):
            v = (b >> (2 * j)) & 3
            assert oracle.code(row, j, 2) == (v ^ 2) - 2
    # int4 through the same accessor is the nibble decode
    for b in range(256):
        row = np.array([b], np.uint8)
        assert oracle.code(row, 0, 4) == oracle.nibble(row, 0)
        assert oracle.code(row, 1, 4) == oracle.nibble(row, 1)


@pytest.mark.parametrize("bits", [8, 2])
def test_code_format_blob_sizes(bits):
    for d, f in [(6144, 2048), (256, 128)]:
        nb = 3 * f * d * bits // 8
        assert oracle.blob_bytes(d, f, bits=bits) == nb + 2 * 3 * f * d // 64
        assert oracle.blob_bytes(d, f, group=0, bits=bits) == nb + 2 * (2 * f + d)
        assert synth.expert_blob(1, 0, 0, d, f, bits=bits).size == oracle.blob_bytes(d, f, bits=bits)


@pytest.mark.parametrize("bits,group,d,f", [(8, 64, 256, 128), (2, 64, 128, 192),
                                            (8, 0, 192, 64), (2, 0, 64, 128)])
def test_code_format_dequant_brute_force(bits, group, d, f):
    blob = synth.expert_blob(5, 0, 3, d, f, group=group, bits=bits)
    for which in range(3):
        assert np.array_equal(oracle.dequant(blob, d, f, which, group=group, bits=bits),
                              np_dequant_bits(blob, d, f, which, bits, group))


@pytest.mark.parametrize("bits", [8, 2])
def test_code_format_ffn_brute_force(bits):
    d, f, n = 256, 128, 3
    blob = synth.expert_blob(6, 0, 1, d, f, bits=bits)
    x = np.random.default_rng(9).normal(size=(n, d))
    Wg, Wu, Wd = (np_dequant_bits(blob, d, f, i, bits) for i in range(3))
    ref = (np_silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    y = oracle.expert_ffn(blob, x, d, f, bits=bits)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("bits", [8, 2])
def test_code_format_layer_brute_force(bits):
    """A small layer: numpy routing (full sort, softmax over all experts,
    renormalised), numpy SwiGLU on the numpy-dequantised experts, ascending
    slot combine; against the oracle's layer."""
    d, f, E, k, T = 128, 64, 8, 3, 5
    rng = np.random.default_rng(bits)
    Wr = (rng.normal(size=(E, d)) * 0.05).astype(np.float32)
    x = rng.normal(size=(T, d)).astype(np.float32)
    blobs = [synth.expert_blob(7, 0, e, d, f, bits=bits) for e in range(E)]
    r = oracle.layer_forward(x, Wr, None, blobs, d, f, k, bits=bits)
    z = x.astype(np.float64) @ Wr.astype(np.float64).T
    out = np.zeros((T, d))
    for t in range(T):
        order = np.lexsort((np.arange(E), -z[t]))[:k]
        assert np.array_equal(r["idx"][t], order)
        p = softmax(z[t])[order]
        p /= p.sum()
        for j, e in enumerate(order):
            Wg, Wu, Wd = (np_dequant_bits(blobs[e], d, f, i, bits) for i in range(3))
            xt = x[t].astype(np.float64)
            out[t] += p[j] * (Wd @ (np_silu(Wg @ xt) * (Wu @ xt)))
    np.testing.assert_allclose(r["out"], out, rtol=1e-10, atol=1e-12 * np.abs(out).max())


# ---------------------------------------------------------- integer activations


def test_quant_i8_invariants_and_ties():
    rng = np.random.default_rng(17)
    rows = [rng.normal(size=256) * 10.0 ** rng.integers(-6, 6),
            np.concatenate([np.zeros(64), rng.normal(size=192)]),            # a group of zeros
            np.concatenate([np.zeros(63), [-3.0], rng.uniform(-1, 1, 64)]),  # one non-zero, negative
            rng.uniform(-1e-30, 1e-30, 128)]
    for v in rows:
        v = v.astype(np.float32)
        q, s = oracle.quant_i8(v)
        assert np.abs(q.astype(np.int64)).max() <= 127
        for g in range(v.size // 64):
            vg, qg = v[64 * g:64 * g + 64].astype(np.float64), q[64 * g:64 * g + 64]
            m = np.abs(vg).max()
            if m == 0:
                assert s[g] == 0 and not qg.any()
                continue
            i = int(np.argmax(np.abs(vg)))
            assert qg[i] == (127 if vg[i] > 0 else -127)           # the group's max is +-127
            assert s[g] == np.float32(np.float32(m) / np.float32(127))
            err = np.abs(vg - qg.astype(np.float64) * float(s[g]))
            assert err.max() <= 0.5 * float(s[g]) * (1 + 2.0 ** -20)  # round to nearest
    # integers with a 127 in the group: scale 1, codes equal to the values;
    # halves go to the even neighbour
    v = np.zeros(64, dtype=np.float32)
    v[:8] = [127, 0.5, 1.5, 2.5, -0.5, -1.5, 3.0, -126]
    q, s = oracle.quant_i8(v)
    assert s[0] == 1.0
    assert list(q[:8]) == [127, 0, 2, 2, 0, -2, 3, -126]


def grid_rows(rng, n, d, step=2.0 ** -4):
    """Rows whose every 64-group holds integers times step with a +-127 in
    it: on the int8 grid of their own group scale (s = step exactly)."""
    q = rng.integers(-127, 128, size=(n, d))
    q[:, ::64] = 127 * rng.choice([-1, 1], size=(n, d // 64))
    return (q * step).astype(np.float32)


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_i8act_ffn_exact_gateup_and_bounded_down(bits):
    """x on the int8 grid of its group scales reproduces x exactly, so gate
    and up are the exact products; the only difference from the fp64 FFN is
    the rounding of a to int8, bounded per output by sum_r |Wd[c,r]| s_a/2
    (s_a: the fp32 scale of r's group of a)."""
    d, f, n = 256, 128, 3
    rng = np.random.default_rng(30 + bits)
    blob = synth.expert_blob(8, 0, 3, d, f, bits=bits)
    x = grid_rows(rng, n, d)
    Wg, Wu, Wd = (np_dequant(blob, d, f, i) if bits == 4 else np_dequant_bits(blob, d, f, i, bits)
                  for i in range(3))
    xd = x.astype(np.float64)
    a = np_silu(xd @ Wg.T) * (xd @ Wu.T)
    exact = a @ Wd.T
    y = oracle.expert_ffn_i8act(blob, x, d, f, bits=bits)
    a32 = a.astype(np.float32)
    for t in range(n):
        s_a = np.repeat(np.abs(a32[t]).reshape(-1, 64).max(axis=1).astype(np.float32)
                        / np.float32(127), 64).astype(np.float64)
        bound = np.abs(Wd) @ (0.5 * s_a) * (1 + 1e-6) + 1e-9 * np.abs(exact[t]).max()
        assert np.all(np.abs(y[t] - exact[t]) <= bound)
        # and the rounding of a is really there: not the exact FFN
        assert np.abs(y[t] - exact[t]).max() > 0


def test_i8act_perrow_is_gs64_with_the_row_scale():
    d, f = 256, 128
    blob = synth.expert_blob(9, 0, 1, d, f, group=0)
    x = np.random.default_rng(4).normal(size=(2, d)).astype(np.float32)
    y_row = oracle.expert_ffn_i8act(blob, x, d, f, group=0)
    y_gs = oracle.expert_ffn_i8act(perrow_as_gs64(blob, d, f), x, d, f, group=64)
    assert np.array_equal(y_row, y_gs)


def test_i8act_layer_is_the_mixture_of_integer_expert_ffns():
    d, f, E, k, T = 128, 64, 8, 3, 5
    rng = np.random.default_rng(12)
    Wr = (rng.normal(size=(E, d)) * 0.05).astype(np.float32)
    x = rng.normal(size=(T, d)).astype(np.float32)
    blobs = [synth.expert_blob(7, 1, e, d, f) for e in range(E)]
    r = oracle.layer_forward(x, Wr, None, blobs, d, f, k, flags=oracle.I8ACT)
    r0 = oracle.layer_forward(x, Wr, None, blobs, d, f, k)
    assert np.array_equal(r["idx"], r0["idx"]) and np.array_equal(r["w"], r0["w"])
    out = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = r["idx"][t, j]
            out[t] += r["w"][t, j] * oracle.expert_ffn_i8act(blobs[e], x[t], d, f)[0]
    np.testing.assert_allclose(r["out"], out, rtol=1e-13, atol=1e-15 * np.abs(out).max())
