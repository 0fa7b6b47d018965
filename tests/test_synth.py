"""The seeded input generator: determinism, random access, encodings and the
distributions the workloads ask for."""
import numpy as np
import pytest

import synth
from synth import configs


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 (state advanced by the golden gamma before each
    # output) starts with these outputs; they are the generator's published
    # reference values (e.g. the test vectors shipped with the xoshiro family).
    out = [synth.lib().synth_draw(0, i) for i in range(3)]
    assert out == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_random_access_and_determinism():
    k = synth.key(7, 3, synth.T_NIB, 11)
    a = synth.random_bytes(7, 3, synth.T_NIB, 1000, expert=11)
    b = synth.random_bytes(7, 3, synth.T_NIB, 1000, expert=11)
    assert np.array_equal(a, b)
    # byte i is byte i%8 of draw i//8
    d = synth.draws(k, 125)
    assert np.array_equal(a, d.view(np.uint8))
    # distinct streams differ
    c = synth.random_bytes(7, 3, synth.T_NIB, 1000, expert=12)
    assert not np.array_equal(a, c)


def test_nibbles_uniform():
    b = synth.random_bytes(1, 0, synth.T_NIB, 1 << 16)
    nib = np.concatenate([b & 15, b >> 4])
    cnt = np.bincount(nib, minlength=16)
    exp = nib.size / 16
    chi2 = ((cnt - exp) ** 2 / exp).sum()
    assert chi2 < 50  # 15 dof, p ~ 1e-5


def test_normal_moments():
    x = synth.normal(5, 0, synth.T_X, 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    w = synth.normal(5, 0, synth.T_WR, 200000, std=0.02)
    assert abs(w.std() - 0.02) < 0.0003


def test_f16_encoder_matches_numpy_rne():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.uniform(0.005, 0.02, 2000), rng.normal(0, 100, 2000),
                           rng.uniform(-1e-5, 1e-5, 500), [0.0, 65504.0, 65519.9, 1e-8]])
    for v in vals:
        assert synth.f64_to_f16_bits(float(v)) == int(np.float16(v).view(np.uint16)), v


def test_bf16_encoder_matches_torch_rne():
    torch = pytest.importorskip("torch")
    x = synth.normal(9, 0, synth.T_X, 5000)
    ours = synth.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_expert_blob_layout_and_scales():
    w = configs.WORKLOADS["tiny"]
    blob = configs.one_expert(w, 0, 3)
    nib, nsc = synth.blob_sizes(w.d, w.f)
    assert blob.size == w.blob_bytes == nib + 2 * nsc == 52224
    s = blob[nib:].view(np.float16).astype(np.float64)
    assert s.min() >= 0.005 - 1e-5 and s.max() <= 0.02
    assert np.array_equal(blob, configs.experts(w, 0, 3, 1)[0])


def test_workload_sizes():
    g = configs.WORKLOADS["decode1"]
    assert g.blob_bytes == 20054016
    assert 3 * g.d * g.f // 2 == 18874368  # ~19 MB of codes per expert


def test_zipf_bias():
    b = synth.zipf_bias(256)
    assert b[0] == 0.0 and np.all(np.diff(b) < 0)
    assert abs(b[255] - (-1.1 * np.log(256))) < 1e-6


def test_verify_batch_shares_a_base():
    w = configs.WORKLOADS["verify8"]
    x, bf = configs.tokens(w, 0)
    assert not bf and x.shape == (8, 6144)
    # rows are base + 0.3*noise: pairwise correlation ~ 1/(1+0.09)
    c = np.corrcoef(x)
    assert np.all(c[np.triu_indices(8, 1)] > 0.85)
