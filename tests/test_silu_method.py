"""The FFN epilogue's short SiLU, its steps replayed in float32 on the host.

The kernel evaluates SiLU(g) = g / (1 + e^-g) as num / (1 + e^-|g|), num = g
for g >= 0 and g e^-|g| below: e^-|g| as 2^t with t = -|g| log2(e) split into
a rounded float product and its error (log2(e) held as a float plus its
remainder), the error carried to first order after the exponential; the
reciprocal refined by one Newton step. Here each hardware operation is
replaced by its correctly rounded float32 counterpart (exp2 and the
reciprocal rounded from double), so the test pins the method and its
constants; the device's own exp2 and reciprocal add at most an ulp each.
The FFN's tolerance allows 8 x 2^-24 for the SiLU and the product with u."""
import numpy as np

F = np.float32
L1 = F(1.44269504)
L2 = F(1.925963033500011e-08)
LN2 = F(0.693147181)


def _fma(a, b, c):
    # float32 fma: the double product of two floats is exact, one rounding
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F)


def silu_short(g):
    g = g.astype(F)
    a = -np.abs(g)
    t = (a * L1).astype(F)
    tl = (_fma(a, np.full_like(a, L1), -t) + (a * L2).astype(F)).astype(F)
    e0 = np.exp2(t.astype(np.float64)).astype(F)
    e = _fma(e0, (tl * LN2).astype(F), e0)
    d = (F(1) + e).astype(F)
    r = (1.0 / d.astype(np.float64)).astype(F)
    r = _fma(r, _fma(-d, r, np.ones_like(d)), r)
    num = np.where(g >= 0, g, (g * e).astype(F)).astype(F)
    return (num * r).astype(F)


def test_constants_split_log2e():
    # L1 is log2(e) rounded to float; L1 + L2 (L2 itself a float) is log2(e)
    # to ~1e-15, far below what a float argument of the exponential resolves
    assert L1 == F(np.log2(np.e))
    assert abs(float(L1) + float(L2) - np.log2(np.e)) < 2e-15
    assert abs(float(LN2) - np.log(2.0)) < 2e-8


def test_short_silu_relative_error():
    rng = np.random.default_rng(7)
    g = np.concatenate([rng.uniform(-20, 20, 1 << 20),
                        np.sign(rng.uniform(-1, 1, 1 << 20)) *
                        np.exp(rng.uniform(np.log(1e-6), np.log(87.0), 1 << 20)),
                        [0.0, -0.0, 1e-30, -1e-30, 87.0, -87.0]]).astype(F)
    got = silu_short(g).astype(np.float64)
    gd = g.astype(np.float64)
    exact = gd / (1.0 + np.exp(-gd))
    nz = exact != 0
    rel = np.abs(got[nz] - exact[nz]) / np.abs(exact[nz])
    # 4.2 x 2^-24 here, 4.6 x 2^-24 measured on the device (its exp2 and
    # reciprocal within an ulp); the FFN tolerance allows 8 x 2^-24
    assert rel.max() < 5 * 2.0**-24, rel.max() / 2.0**-24
    assert np.all(got[~nz] == 0)


def test_short_silu_limits():
    g = np.array([100.0, -100.0, 1e30, -1e30], F)
    got = silu_short(g)
    assert got[0] == F(100.0) and got[2] == F(1e30)
    assert abs(float(got[1])) < 1e-40 and got[3] == 0
