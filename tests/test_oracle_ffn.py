"""Pins of the oracle's SwiGLU expert FFN (the local-layer workload's expert).

Independent checks: torch's float64 matmul + silu (library routines) on random
rows, scipy's expit for the one-hot/identity special case, the zero
up-projection, exact power-of-two scalings, and expert selection.
"""
import numpy as np
import scipy.special
import torch

import oracle
import synth


def _weights(E, H, I, seed, std=0.1):
    g = np.random.default_rng(seed)
    gu = synth.f32_to_bf16_bits(g.standard_normal((E, 2 * I, H)).astype(np.float32) * std)
    dn = synth.f32_to_bf16_bits(g.standard_normal((E, H, I)).astype(np.float32) * std)
    return gu, dn


def _rows(n, H, seed):
    return synth.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((n, H)).astype(np.float32))


def f64(bits):
    return oracle.bf16_to_f64(bits)


def test_matches_torch_float64():
    E, H, I, n = 3, 64, 48, 12
    gu, dn = _weights(E, H, I, 1)
    rows = _rows(n, H, 2)
    re = np.arange(n) % E
    o64, o16, gus = oracle.expert_swiglu_rows(rows, re, gu, dn, want_gu=True)
    o64b, o16b = oracle.expert_swiglu_rows(rows, re, gu, dn)
    assert np.array_equal(o64, o64b) and np.array_equal(o16, o16b)
    for r in range(n):
        e = re[r]
        s = torch.from_numpy(f64(rows[r]))
        Wg = torch.from_numpy(f64(gu[e, :I]))
        Wu = torch.from_numpy(f64(gu[e, I:]))
        Wd = torch.from_numpy(f64(dn[e]))
        # the pre-activation sums the oracle reports are the two projections
        np.testing.assert_allclose(gus[r, :I], (Wg @ s).numpy(), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(gus[r, I:], (Wu @ s).numpy(), rtol=1e-13, atol=1e-13)
        h = torch.nn.functional.silu(Wg @ s) * (Wu @ s)
        h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)  # bf16 intermediate
        ref = (Wd @ h).numpy()
        # rare double-rounding ties of the bf16 intermediate aside, the sums agree
        np.testing.assert_allclose(o64[r], ref, rtol=0, atol=2e-4)
        np.testing.assert_allclose(o64[r], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max() + 1e-14)
    # the bf16 output is within half a bf16 ulp (unit roundoff 2^-8 bound) of the double output
    assert np.all(np.abs(f64(o16) - o64) <= np.abs(o64) * 2.0**-8 + 1e-300)


def test_zero_up_projection_gives_zero():
    E, H, I = 2, 32, 16
    gu, dn = _weights(E, H, I, 3)
    gu[:, I:, :] = 0
    o64, o16 = oracle.expert_swiglu_rows(_rows(5, H, 4), [0, 1, 0, 1, 1], gu, dn)
    assert np.all(o64 == 0.0)


def test_one_hot_identity_case_uses_silu():
    # H == I, gate row j = c * e_j, up row j = e_j, down = identity:
    # out_j = bf16( silu(c * s_j) * s_j )
    H = I = 16
    c = 0.75
    gu = np.zeros((1, 2 * I, H), np.uint16)
    dn = np.zeros((1, H, I), np.uint16)
    for j in range(I):
        gu[0, j, j] = synth.f32_to_bf16_bits(np.array([c], np.float32))[0]
        gu[0, I + j, j] = synth.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
        dn[0, j, j] = synth.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    rows = _rows(4, H, 5)
    o64, o16 = oracle.expert_swiglu_rows(rows, [0, 0, 0, 0], gu, dn)
    s = f64(rows)
    z = c * s
    ref = z * scipy.special.expit(z) * s
    np.testing.assert_allclose(o64, ref, rtol=2.0**-8, atol=0)


def test_power_of_two_scalings_are_exact():
    E, H, I = 2, 32, 24
    gu, dn = _weights(E, H, I, 6)
    rows = _rows(6, H, 7)
    # expert 1 = expert 0 with the up-projection doubled and down halved
    gu[1] = gu[0]
    dn[1] = dn[0]
    up = f64(gu[0, I:]) * 2.0
    gu[1, I:] = synth.f32_to_bf16_bits(up.astype(np.float32))
    a64, _ = oracle.expert_swiglu_rows(rows, [0] * 6, gu, dn)
    b64, _ = oracle.expert_swiglu_rows(rows, [1] * 6, gu, dn)
    np.testing.assert_array_equal(b64, 2.0 * a64)


def test_expert_selection():
    E, H, I = 4, 32, 16
    gu, dn = _weights(E, H, I, 8)
    rows = _rows(8, H, 9)
    re = np.array([3, 1, 0, 2, 2, 3, 1, 0])
    o64, _ = oracle.expert_swiglu_rows(rows, re, gu, dn)
    for r in range(8):
        one, _ = oracle.expert_swiglu_rows(rows[r:r + 1], [re[r]], gu, dn)
        np.testing.assert_array_equal(one[0], o64[r])
        other, _ = oracle.expert_swiglu_rows(rows[r:r + 1], [(re[r] + 1) % E], gu, dn)
        assert not np.array_equal(other[0], o64[r])
