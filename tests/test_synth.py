"""The seeded generators: determinism, shapes, and the skew each workload claims."""
import numpy as np

import oracle
import synth


def test_deterministic():
    wl = synth.WORKLOADS["tiny"]
    a, b = synth.logits(wl), synth.logits(wl)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(synth.hidden(wl), synth.hidden(wl))
    assert a.dtype == np.float32 and a.shape == (wl.T, wl.E)


def test_bf16_bits():
    v = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -2.5, 0.0], np.float32)
    assert synth.f32_to_bf16_bits(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0]
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v[[0, 3]])), v[[0, 3]])


def test_zipf_hot_cold_ratio_about_5():
    wl = synth.WORKLOADS["zipf"]
    idx, _ = oracle.route(synth.logits(wl), wl.k)
    c = np.bincount(idx.ravel(), minlength=wl.E)
    assert 4.0 <= c.max() / c.min() <= 6.0


def test_decode_hot_share_about_80_percent():
    wl = synth.WORKLOADS["decode_hot"]
    idx, _ = oracle.route(synth.logits(wl), wl.k)
    share = np.isin(idx, synth.hot_set(wl.E, wl.seed)).mean()
    assert 0.75 <= share <= 0.85
    # the hot set spreads over several ranks, not one
    assert len(set((synth.hot_set(wl.E, wl.seed) // wl.L).tolist())) >= 3


def test_dirichlet_is_strongly_skewed():
    wl = synth.WORKLOADS["dirichlet_waves"].with_(T=2048)
    idx, _ = oracle.route(synth.logits(wl), wl.k)
    s = oracle.stats(np.bincount(idx.ravel(), minlength=wl.E).astype(np.int32), wl.R)
    assert s["expert_max_over_mean"] > 10 and s["rank_gini"] > 0.3


def test_swiglu_weight_shapes():
    wl = synth.WORKLOADS["local_layer"].with_(E=2, H=64, I=32)
    gu, dn = synth.swiglu_weights(wl)
    assert gu.shape == (2, 64, 64) and dn.shape == (2, 64, 32) and gu.dtype == np.uint16
    f = synth.bf16_bits_to_f32(gu)
    assert 0.015 < f.std() < 0.025
