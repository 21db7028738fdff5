"""Pins of the oracle's expert stage and combine (MoE systems survey, section 1.1,
eq. (1) and EP flow step 4).

Independent checks: the identity invariant (dispatch then combine with identity
experts returns x), the closed form for (e+1)-scaled experts, torch's CPU bf16
conversion (library routine) for the rounding, and exact rational arithmetic
(fractions.Fraction) for the single-precision fused multiply-add chain.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import load_golden


def _route_dispatch(T, E, k, R, W, H, dtype, seed):
    g = np.random.default_rng(seed)
    l = g.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route(l, k)
    x = g.standard_normal((T, H)).astype(np.float32)
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    return idx, w, x, oracle.dispatch(x, idx, E, R, W)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_experts_give_back_x(dtype):
    T, E, k, R, W, H = 60, 16, 4, 4, 2, 32
    idx, w, x, d = _route_dispatch(T, E, k, R, W, H, dtype, seed=1)
    y = oracle.combine_f64(d["send_buf"], w, d["pos"], T)
    np.testing.assert_allclose(y, oracle.as_f64(x), rtol=1e-15, atol=0)


def test_scaled_experts_closed_form_bf16():
    T, E, k, R, W, H = 80, 8, 2, 4, 1, 16
    idx, w, x, d = _route_dispatch(T, E, k, R, W, H, "bf16", seed=2)
    out = oracle.expert_scale(d["send_buf"], d["expert_offsets"], d["expert_counts"])
    y = oracle.combine_f64(out, w, d["pos"], T)
    factor = (w * (idx + 1)).sum(1)
    ref = oracle.as_f64(x) * factor[:, None]
    # only the bf16 rounding of each expert output (unit roundoff 2^-8) separates them
    bound = (w * (idx + 1)).sum(1)[:, None] * np.abs(oracle.as_f64(x)) * 2.0**-8
    assert np.all(np.abs(y - ref) <= bound + 1e-300)


def test_expert_scale_rounding_matches_torch_bf16():
    g = np.random.default_rng(3)
    E, H = 256, 64
    counts = np.full(E, 2, np.int32)
    offs = (np.arange(E) * 2).astype(np.int32)
    send = synth.f32_to_bf16_bits(g.standard_normal((2 * E, H)).astype(np.float32) * 3)
    out = oracle.expert_scale(send, offs, counts)
    scale = np.repeat(np.arange(1, E + 1, dtype=np.float32), 2)[:, None]
    prod = torch.from_numpy(synth.bf16_bits_to_f32(send) * scale)  # exact in fp32 (<= 17 bits)
    ref = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(out, ref)


def test_expert_scale_f32_rounding():
    g = np.random.default_rng(4)
    send = g.standard_normal((6, 8)).astype(np.float32)
    out = oracle.expert_scale(send, np.array([0, 2, 4], np.int32), np.array([2, 2, 2], np.int32))
    for n in range(6):
        e = n // 2
        # fp32 product is correctly rounded by IEEE; numpy float32 multiply is the library routine
        np.testing.assert_array_equal(out[n], send[n] * np.float32(e + 1))


def test_round_bf16_matches_torch_on_fp32_inputs():
    g = np.random.default_rng(5)
    v = np.concatenate([g.standard_normal(5000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 5000),
                        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3.0e38, 1e-40], np.float32)])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(a)) for a in v], np.uint16)
    np.testing.assert_array_equal(got, ref)


def _nearest_f32(q: Fraction) -> np.float32:
    """Round a rational to the nearest fp32, ties to the even significand (brute force)."""
    f = np.float32(float(q))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_f32fma_chain_exact_rational():
    T, E, k, R, W, H = 12, 8, 3, 2, 1, 5
    idx, w, x, d = _route_dispatch(T, E, k, R, W, H, "f32", seed=6)
    out = oracle.expert_scale(d["send_buf"], d["expert_offsets"], d["expert_counts"])
    w32 = w.astype(np.float32)
    y = oracle.combine_f32fma(out, w32, d["pos"], T)
    for t in range(T):
        for h in range(H):
            acc = np.float32(0.0)
            for i in range(k):
                q = Fraction(float(w32[t, i])) * Fraction(float(out[d["pos"][t, i], h])) + Fraction(float(acc))
                acc = _nearest_f32(q)
            assert y[t, h] == acc


def test_f32fma_bf16_identity_experts_exact():
    # bf16 x, identity experts: sum(w) = 1 within a few fp32 ulps, far inside half a bf16 ulp
    T, E, k, R, W, H = 64, 64, 6, 8, 1, 32
    idx, w, x, d = _route_dispatch(T, E, k, R, W, H, "bf16", seed=7)
    y = oracle.combine_f32fma(d["send_buf"], w.astype(np.float32), d["pos"], T)
    np.testing.assert_array_equal(y, x)


def test_f32fma_close_to_f64():
    T, E, k, R, W, H = 50, 16, 4, 4, 1, 64
    idx, w, x, d = _route_dispatch(T, E, k, R, W, H, "f32", seed=8)
    out = oracle.expert_scale(d["send_buf"], d["expert_offsets"], d["expert_counts"])
    y32 = oracle.combine_f32fma(out, w.astype(np.float32), d["pos"], T)
    y64 = oracle.combine_f64(out, w, d["pos"], T)
    mag = (np.abs(w)[:, :, None] * np.abs(out[d["pos"]])).sum(1)
    assert np.all(np.abs(y32 - y64) <= (k + 2) * 2.0**-24 * mag + 1e-30)


def test_dropped_pick_contributes_nothing():
    out = np.array([[1.0, 2.0], [10.0, 20.0]], np.float32)
    pos = np.array([[0, -1], [1, 7]], np.int32)
    w = np.array([[0.5, 0.5], [0.25, 0.75]])
    y = oracle.combine_f64(out, w, pos, 2)
    assert y.tolist() == [[0.5, 1.0], [2.5, 5.0]]


def test_golden_tiny_combine_factor():
    g = load_golden("dispatch_waves_tiny.txt")
    E, k, R, W = (int(g[n][0]) for n in ("E", "k", "R", "W"))
    l = np.array(g["logits"], np.float32)
    idx, w = oracle.route(l, k)
    x = np.ones((4, 8), np.float32)
    d = oracle.dispatch(x, idx, E, R, W)
    out = oracle.expert_scale(d["send_buf"], d["expert_offsets"], d["expert_counts"])
    y = oracle.combine_f64(out, w, d["pos"], 4)
    np.testing.assert_allclose(y[:, 0], g["combine_factor"], rtol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scaled_tokens_equals_composed_path(dtype):
    # the sampled-token shortcut must reproduce dispatch -> expert -> combine exactly
    T, E, k, R, W, H = 70, 32, 4, 4, 2, 40
    idx, w, x, d = _route_dispatch(T, E, k, R, W, H, dtype, seed=9)
    out = oracle.expert_scale(d["send_buf"], d["expert_offsets"], d["expert_counts"])
    w32 = w.astype(np.float32)
    y64 = oracle.combine_f64(out, w, d["pos"], T)
    yq = oracle.combine_f32fma(out, w32, d["pos"], T)
    toks = np.array([0, 5, 69, 33, 33, 12])
    s64, sq = oracle.scaled_tokens(x, idx, w, E, toks, w32=w32)
    np.testing.assert_array_equal(s64, y64[toks])
    np.testing.assert_array_equal(sq, yq[toks])


def test_signed_zero_survives_identity_experts():
    # -0 is the additive identity: a sum of -0 terms is -0, so identity experts
    # give back a -0 input bit for bit; +0 stays +0.
    x = np.array([[-0.0, 0.0, 1.5, -2.0]], np.float32)
    idx = np.array([[0, 1]], np.int32)
    w = np.array([[0.75, 0.25]])
    d = oracle.dispatch(x, idx, 2, 1, 1)
    y32 = oracle.combine_f32fma(d["send_buf"], w.astype(np.float32), d["pos"], 1)
    assert y32.view(np.uint32).tolist() == x.view(np.uint32).tolist()
    y64 = oracle.combine_f64(d["send_buf"], w, d["pos"], 1)
    assert np.signbit(y64[0, 0]) and not np.signbit(y64[0, 1])
    xb = synth.f32_to_bf16_bits(x)
    yb = oracle.combine_f32fma(oracle.dispatch(xb, idx, 2, 1, 1)["send_buf"],
                               w.astype(np.float32), d["pos"], 1)
    assert yb.tolist() == xb.tolist()
