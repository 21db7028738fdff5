"""moe_stats against the oracle over expert counts that take each way through
the statistics code: all ordered pairs (up to 128 values) and the sorted
closed form (beyond), power-of-two and ragged sizes, one rank and one expert
per rank, zeros, ties and large counts. Bar: every field identical (integer
numerators, one double division each)."""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = [
    # (E, R, kind)
    (1, 1, "random"), (64, 8, "random"), (128, 128, "random"), (129, 3, "random"),
    (200, 8, "random"), (200, 200, "ties"), (256, 1, "skew"), (256, 32, "zeros"),
    (320, 5, "random"), (320, 320, "random"), (1000, 8, "skew"), (1023, 3, "ties"),
    (1024, 1024, "random"), (1024, 1, "large"), (1024, 8, "equal"),
]


def _counts(E, kind, seed):
    g = np.random.default_rng(seed)
    if kind == "random":
        c = g.integers(0, 5000, E)
    elif kind == "ties":
        c = g.integers(0, 4, E) * 1000
    elif kind == "skew":
        c = np.floor(g.pareto(0.8, E) * 100)
    elif kind == "zeros":
        c = g.integers(0, 50, E) * (g.random(E) < 0.3)
    elif kind == "large":  # totals close to 2^31
        c = np.full(E, (2**31 - 1) // E - 7)
        c[::5] += 5
    else:  # equal
        c = np.full(E, 777)
    return c.astype(np.int32)


@pytest.mark.parametrize("E,R,kind", CASES)
def test_stats_match_oracle(E, R, kind):
    print(f"[stats] E={E} R={R} {kind}", flush=True)
    c = _counts(E, kind, seed=E * 7 + R)
    got = moe.stats(torch.from_numpy(c).to(DEV), R)
    assert got == oracle.stats(c, R)
