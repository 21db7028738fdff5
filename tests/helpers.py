"""Small shared helpers for the tests (no method arithmetic)."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    """Parse a 'key v v v | v v' fixture: '|' separates rows of a 2-D value."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            rows = [r.split() for r in rest.split("|")]
            vals = [[float(v) for v in r] for r in rows]
            out[key] = vals[0] if len(vals) == 1 else vals
    return out


def bucket_rank_of_expert(E: int, R: int, W: int) -> np.ndarray:
    """Position of each expert's bucket when buckets are sorted by (wave, rank, slot).

    Obtained by sorting the key tuples with Python's sort (the layout reading:
    expert e on rank e // L, slot e % L, wave slot * W // L)."""
    L = E // R
    keys = [((e % L) * W // L, e // L, e % L) for e in range(E)]
    order = sorted(range(E), key=lambda e: keys[e])
    rank = np.empty(E, np.int64)
    for j, e in enumerate(order):
        rank[e] = j
    return rank
