"""Error bound for the GPU's SwiGLU expert rows against the oracle's (tests only).

The oracle evaluates each row in double: g and u exactly (up to double
rounding), h = round_bf16(SiLU(g) * u), out = sum_j Wd[c][j] h_j. The kernel
accumulates g, u and out in fp32 (MFMA) and evaluates SiLU(g) * u in fp32, then
rounds h and out to bf16. Where the exact h lies within the kernel's fp32 error
of a bf16 rounding boundary, the two sides may round h to neighbouring bf16
values; every other difference is fp32 accumulation and the final rounding.
The bound below adds those terms up, element by element, from quantities the
oracle reports (g, u, out) and absolute-value sums of the operands:

    dg_j  = gamma_H * sum_h |Wg[j][h] s_h|          fp32 sum of H exact products
    du_j  = gamma_H * sum_h |Wu[j][h] s_h|
    dh_j  = |SiLU'(g_j) u_j| dg_j + |SiLU(g_j)| du_j + 8 u_32 |SiLU(g_j) u_j|
            (the last term: the kernel's SiLU, at most 4.6 u_32 from the exact
            one over 16M arguments in [-100, 100], and the product with u)
    flip_j = max |r(h_j +- dh_j) - r(h_j)|            r = round to bf16
    E_c   = sum_j |Wd[c][j]| flip_j + gamma_I sum_j |Wd[c][j]| (|h_j| + flip_j)
    |got_c - out_c| <= E_c (1 + 2^-8) + 2^-8 |out_c|   final bf16 rounding

with u_32 = 2^-24 and gamma_n = n u_32 / (1 - n u_32). A wrong expert, row or
column shows as an error of the order of the outputs themselves, far above it.
"""
from __future__ import annotations

import numpy as np

import oracle

U32 = 2.0**-24


def gamma(n: int) -> float:
    return n * U32 / (1.0 - n * U32)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round doubles to 8 significant bits, ties to even (normal range)."""
    m, ex = np.frexp(v)  # v = m 2^ex, |m| in [0.5, 1)
    return np.ldexp(np.rint(np.ldexp(m, 8)), ex - 8)


def _silu(g):
    return g / (1.0 + np.exp(-g))


def _dsilu(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def swiglu_rows_bound(x_rows_bits, row_expert, gu_bits, dn_bits):
    """(out_f64 [n,H], out_bf16 bits [n,H], bound [n,H]) for the rows."""
    o64, o16, gus = oracle.expert_swiglu_rows(x_rows_bits, row_expert, gu_bits, dn_bits,
                                              want_gu=True)
    n, H = o64.shape
    I = dn_bits.shape[2]
    re = np.asarray(row_expert)
    s_abs = np.abs(oracle.bf16_to_f64(x_rows_bits))
    bound = np.empty_like(o64)
    for e in np.unique(re):
        sel = np.nonzero(re == e)[0]
        w_gu = np.abs(oracle.bf16_to_f64(gu_bits[e]))      # [2I, H]
        w_dn = oracle.bf16_to_f64(dn_bits[e])              # [H, I]
        abs_sums = s_abs[sel] @ w_gu.T                      # [m, 2I]
        g, u = gus[sel, :I], gus[sel, I:]
        dg = gamma(H) * abs_sums[:, :I]
        du = gamma(H) * abs_sums[:, I:]
        h = _silu(g) * u
        dh = np.abs(_dsilu(g) * u) * dg + np.abs(_silu(g)) * du + 8 * U32 * np.abs(h)
        dh = dh * 1.01 + 1e-30  # second-order terms
        r0 = round_bf16(h)
        flip = np.maximum(np.abs(round_bf16(h + dh) - r0), np.abs(round_bf16(h - dh) - r0))
        a_dn = np.abs(w_dn)
        E = flip @ a_dn.T + gamma(I) * ((np.abs(r0) + flip) @ a_dn.T)   # [m, H]
        bound[sel] = E * (1 + 2.0**-8) + 2.0**-8 * np.abs(o64[sel]) + 1e-30
    return o64, o16, bound


# Second, statistical bar: without a flip of h an output is off by its fp32
# accumulation and its own rounding only, well inside 2^-7 |out| + a small
# absolute term; flips are rare events (the exact h must sit within the fp32
# error of a rounding boundary), so at most this fraction of the outputs may
# exceed that tight bar. A systematic mistake (a dropped K step, a wrong
# scale) moves most outputs past it.
TIGHT_FRACTION = 1e-3


def check_rows(got_bits, o64, bound, tight_atol=2e-3):
    got = oracle.bf16_to_f64(got_bits)
    err = np.abs(got - o64)
    bad = err > bound
    assert not bad.any(), (f"{bad.sum()} of {bad.size} outside the rounding bound; max err "
                           f"{err.max()}, max err/bound {(err / bound).max():.3f}")
    loose = float((err > 2.0**-7 * np.abs(o64) + tight_atol).mean())
    assert loose <= TIGHT_FRACTION, f"{loose:.2e} of the outputs beyond 2^-7|out| + {tight_atol}"
    return float((err / bound).max())
