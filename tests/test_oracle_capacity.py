"""Pins of the oracle's capacity-factor dispatch (survey section 1.2 eq. (3) and
EP flow step 2: drop beyond the expert capacity, pad unused capacity with
zeros) against the hand-worked golden, an independent sort-based brute force,
and the limits the definition fixes."""
import numpy as np
import pytest

import oracle
from helpers import bucket_rank_of_expert, load_golden


def test_golden_capacity_example():
    g = load_golden("capacity_tiny.txt")
    T, E, k, R, W = (int(g[n][0]) for n in ("T", "E", "k", "R", "W"))
    cap = int(g["capacity"][0])
    assert oracle.expert_capacity(k, g["f"][0], T, E) == cap
    idx = np.array(g["topk_idx"], np.int32)
    x = (np.arange(T * 4, dtype=np.float32) + 1).reshape(T, 4)
    d = oracle.dispatch_capacity(x, idx, E, R, W, cap)
    for key in ("kept_counts", "expert_offsets", "rank_counts", "rank_offsets", "wave_offsets",
                "row_token"):
        np.testing.assert_array_equal(d[key], np.array(g[key], np.int32).ravel(), err_msg=key)
    np.testing.assert_array_equal(d["pos"], np.array(g["pos"], np.int32))
    rt = d["row_token"]
    np.testing.assert_array_equal(d["send_buf"][rt >= 0], x[rt[rt >= 0]])
    assert (d["send_buf"][rt < 0] == 0).all()


@pytest.mark.parametrize("k,f,T,E,want", [(2, 1.25, 256, 8, 80), (6, 1.0, 4096, 64, 384),
                                          (1, 1.1, 10, 3, 4), (2, 1.0, 7, 4, 4), (8, 0.0, 99, 16, 0),
                                          (2, 0.5, 6, 4, 2)])
def test_capacity_formula_closed_forms(k, f, T, E, want):
    assert oracle.expert_capacity(k, f, T, E) == want


def test_capacity_formula_rejects_negative():
    assert oracle.expert_capacity(2, -0.5, 10, 4) == -1


def _brute(idx, E, R, W, cap):
    """Kept picks from the definition by sorting: each expert's picks in
    (token, pick) order, the first cap kept, rows laid out bucket after bucket."""
    T, k = idx.shape
    brank = bucket_rank_of_expert(E, R, W)
    pos = np.full((T, k), -1, np.int64)
    row_token = np.full(E * cap, -1, np.int64)
    for e in range(E):
        picks = sorted((t, i) for t in range(T) for i in range(k) if idx[t, i] == e)
        for j, (t, i) in enumerate(picks[:cap]):
            pos[t, i] = brank[e] * cap + j
            row_token[brank[e] * cap + j] = t
    return pos, row_token


@pytest.mark.parametrize("seed,T,E,k,R,W,cap", [(0, 40, 8, 2, 4, 1, 7), (1, 33, 12, 3, 3, 2, 5),
                                                (2, 64, 16, 4, 4, 4, 1), (3, 17, 6, 6, 2, 3, 9),
                                                (4, 50, 8, 1, 2, 2, 0)])
def test_against_sort_brute_force(seed, T, E, k, R, W, cap):
    g = np.random.default_rng(seed)
    # skewed routing so that some experts overflow and others are padded
    p = g.dirichlet(np.full(E, 0.4))
    idx = np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    idx[g.random((T, k)) < 0.05] = -1  # a few invalid picks
    x = g.standard_normal((T, 8)).astype(np.float32)
    d = oracle.dispatch_capacity(x, idx, E, R, W, cap)
    pos, rt = _brute(idx, E, R, W, cap)
    np.testing.assert_array_equal(d["pos"], pos)
    np.testing.assert_array_equal(d["row_token"], rt)
    ec = np.bincount(idx[idx >= 0], minlength=E)
    np.testing.assert_array_equal(d["kept_counts"], np.minimum(ec, cap))
    assert (d["pos"] >= 0).sum() == np.minimum(ec, cap).sum()
    np.testing.assert_array_equal(d["send_buf"][rt >= 0], x[rt[rt >= 0]])
    assert (d["send_buf"][rt < 0] == 0).all()
    # whole buckets per (wave, rank): each of the W*R segments holds L/W buckets
    L = E // R
    assert (d["rank_counts"] == (L // W) * cap).all()
    np.testing.assert_array_equal(d["rank_offsets"], np.arange(W * R) * (L // W) * cap)
    assert d["wave_offsets"][-1] == E * cap


def test_ample_capacity_is_plain_dispatch_in_padded_buckets():
    g = np.random.default_rng(7)
    T, E, k, R, W = 100, 8, 2, 4, 2
    logits = g.standard_normal((T, E)).astype(np.float32)
    idx, _ = oracle.route(logits, k)
    x = g.standard_normal((T, 16)).astype(np.float32)
    plain = oracle.dispatch(x, idx, E, R, W)
    cap = int(plain["expert_counts"].max())
    d = oracle.dispatch_capacity(x, idx, E, R, W, cap)
    np.testing.assert_array_equal(d["kept_counts"], plain["expert_counts"])
    brank = bucket_rank_of_expert(E, R, W)
    e_of = idx.astype(np.int64)
    rel = plain["pos"] - plain["expert_offsets"][e_of]
    np.testing.assert_array_equal(d["pos"], brank[e_of] * cap + rel)


def test_zero_capacity_drops_everything():
    g = np.random.default_rng(9)
    idx = g.integers(0, 8, size=(20, 2)).astype(np.int32)
    x = g.standard_normal((20, 4)).astype(np.float32)
    d = oracle.dispatch_capacity(x, idx, 8, 2, 1, 0)
    assert (d["pos"] == -1).all() and d["rows"] == 0
    assert (d["kept_counts"] == 0).all()
