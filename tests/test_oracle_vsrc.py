"""Pins of the oracle's virtual-source exchange (MoE systems survey section 1.1,
EP flow steps 2-4; irregular AllToAll page: Alltoallv counts and displacements)
against a hand-worked example, a sort-based brute force written from the
layout definitions alone, the identities of the count matrices, and the round
trip of the combine direction."""
import numpy as np
import pytest

import oracle
import synth
from helpers import load_golden


def _tokens_of(rows_x, x):
    """Token of each row, for x with distinct rows (row t is all t)."""
    return rows_x[:, 0].astype(np.int64)


@pytest.mark.parametrize("W", [1, 2])
def test_golden_hand_worked(W):
    g = load_golden("vsrc_tiny.txt")
    T, E, k, R = (int(g[n][0]) for n in ("T", "E", "k", "R"))
    idx = np.array(g["topk_idx"], np.int32)
    x = np.repeat(np.arange(T, dtype=np.float32)[:, None], 4, axis=1)
    w = np.full((T, k), 0.5)
    v = oracle.vsrc_exchange(x, idx, w, E, R, W)
    p = f"W{W}_"
    eq = np.testing.assert_array_equal
    eq(v["src_counts"], np.array(g["src_counts"], np.int32))
    eq(v["expert_counts"], np.array(g["expert_counts"], np.int32))
    eq(v["expert_offsets"], np.array(g["expert_offsets"], np.int32))
    eq(v["src_offsets"], np.array(g[p + "src_offsets"], np.int32))
    eq(v["send_counts"].reshape(R, -1), np.array(g[p + "send_counts"], np.int32))
    eq(v["send_offsets"].reshape(R, -1), np.array(g[p + "send_offsets"], np.int32))
    eq(v["recv_counts"].reshape(R, -1), np.array(g[p + "recv_counts"], np.int32))
    eq(v["recv_offsets"].reshape(R, -1), np.array(g[p + "recv_offsets"], np.int32))
    eq(v["pos"], np.array(g[p + "pos"], np.int32))
    eq(_tokens_of(v["send"], x), np.array(g[p + "send_token"], np.int64))
    eq(_tokens_of(v["recv"], x), np.array(g[p + "recv_token"], np.int64))
    eq(_tokens_of(v["grouped"], x), np.array(g["grouped_token"], np.int64))


def _brute(idx, E, R, W):
    """Send, recv and regrouped pick order from the layout definitions by
    Python sorts of key tuples: source buffer (wave, destination, slot, token),
    recv (destination, wave, source, slot, token), regrouped (expert, token)."""
    T, k = idx.shape
    L, Ts = E // R, T // R
    picks = [(t, i, int(idx[t, i])) for t in range(T) for i in range(k) if 0 <= idx[t, i] < E]

    def wave(e):
        return (e % L) * W // L

    send, pos = [], {}
    src_offsets = np.zeros((R, E), np.int64)
    bucket_key = lambda e: (wave(e), e // L, e % L)  # noqa: E731
    for s in range(R):
        mine = sorted((p for p in picks if p[0] // Ts == s),
                      key=lambda p: (*bucket_key(p[2]), p[0]))
        for j, p in enumerate(mine):
            pos[(p[0], p[1])] = s * Ts * k + j
        for e in range(E):  # rows of the source's buckets that come before e's
            src_offsets[s, e] = s * Ts * k + sum(bucket_key(p[2]) < bucket_key(e) for p in mine)
        send += mine
    recv = sorted(picks, key=lambda p: (p[2] // L, wave(p[2]), p[0] // Ts, p[2] % L, p[0]))
    grouped = sorted(picks, key=lambda p: (p[2], p[0]))
    return send, pos, recv, grouped, src_offsets


CASES = [(0, 24, 8, 2, 4, 1), (1, 30, 12, 3, 3, 2), (2, 32, 16, 4, 2, 4), (3, 18, 6, 6, 6, 1),
         (4, 40, 16, 2, 1, 2), (5, 16, 8, 8, 2, 2)]


@pytest.mark.parametrize("seed,T,E,k,R,W", CASES)
def test_against_sort_brute_force(seed, T, E, k, R, W):
    g = np.random.default_rng(seed)
    # skewed, some experts never picked, some ids invalid (-1): those picks are not sent
    pop = g.dirichlet(np.full(E, 0.4))
    idx = np.stack([g.choice(E, k, replace=False, p=pop) for _ in range(T)]).astype(np.int32)
    idx[g.random((T, k)) < 0.05] = -1
    x = (np.arange(T, dtype=np.float32)[:, None] * 16 + np.arange(4, dtype=np.float32))
    w = g.random((T, k))
    v = oracle.vsrc_exchange(x, idx, w, E, R, W)
    send, pos, recv, grouped, src_offsets = _brute(idx, E, R, W)
    np.testing.assert_array_equal(v["src_offsets"], src_offsets)
    n = len(send)
    Ts = T // R
    # source shards keep their own row ranges; unused rows (invalid picks) are zero
    used = np.zeros(T * k, bool)
    for (t, i), r in pos.items():
        assert v["pos"][t, i] == r
        used[r] = True
    assert (v["pos"][idx < 0] == -1).all()
    np.testing.assert_array_equal(v["send"][used], x[[p[0] for p in send]])
    assert (v["send"][~used] == 0).all()
    np.testing.assert_array_equal(v["recv"][:n], x[[p[0] for p in recv]])
    np.testing.assert_array_equal(v["grouped"][:n], x[[p[0] for p in grouped]])
    # count matrices: what each source sends sums to its valid picks; what each
    # destination receives sums to its experts' picks; the two sides transpose
    sc, rc = v["send_counts"], v["recv_counts"]
    for s in range(R):
        assert sc[s].sum() == (idx[s * Ts:(s + 1) * Ts] >= 0).sum()
    ecount = np.bincount(idx[idx >= 0], minlength=E)
    L = E // R
    for d in range(R):
        assert rc[d].sum() == ecount[d * L:(d + 1) * L].sum()
    np.testing.assert_array_equal(rc, sc.transpose(2, 1, 0))
    np.testing.assert_array_equal(v["src_counts"].sum(axis=0), ecount)
    assert sc.sum() == n
    np.testing.assert_array_equal(v["expert_counts"], ecount)


@pytest.mark.parametrize("seed,T,E,k,R,W", CASES)
def test_round_trip_and_combine(seed, T, E, k, R, W):
    """With expert e the map (e+1)*I, the rows that come back to a source are
    (e+1) * x of that pick, and y = sum_i w_i (e_i + 1) x."""
    g = np.random.default_rng(100 + seed)
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    x = g.standard_normal((T, 8)).astype(np.float32)
    w = g.random((T, k))
    v = oracle.vsrc_exchange(x, idx, w, E, R, W)
    for t in range(T):
        for i in range(k):
            np.testing.assert_array_equal(v["back_send"][v["pos"][t, i]],
                                          np.float32(idx[t, i] + 1) * x[t])
    y64 = ((np.asarray(w, np.float32).astype(np.float64) * (idx + 1))[:, :, None]
           * x.astype(np.float64)[:, None, :]).sum(axis=1)
    np.testing.assert_allclose(v["y"].astype(np.float64), y64, rtol=1e-5, atol=1e-5)


def test_one_source_is_the_one_rank_dispatch():
    """R = 1: one source, one destination; send and recv are the single rank's
    dispatch buffer and the regrouped rows are in plain expert order."""
    wl = synth.WORKLOADS["tiny"].with_(R=1)
    logits, x = synth.logits(wl), synth.hidden(wl)
    idx, w = oracle.route(logits, wl.k)
    v = oracle.vsrc_exchange(x, idx, w, wl.E, 1, 1)
    order = np.argsort(idx.reshape(-1), kind="stable")
    np.testing.assert_array_equal(v["send"], x[order // wl.k])
    np.testing.assert_array_equal(v["recv"], v["send"])
    np.testing.assert_array_equal(v["grouped"], v["send"])


@pytest.mark.parametrize("name", ["tiny", "zipf", "dirichlet_waves", "decode_hot"])
def test_workloads_regroup_to_expert_order(name):
    """On every configuration (token count cut for speed) the regrouped rows of
    all destinations are the picks stably sorted by expert id."""
    wl = synth.WORKLOADS[name]
    wl = wl.with_(T=min(wl.T, 512), H=min(wl.H, 64))
    logits, x = synth.logits(wl), synth.hidden(wl)
    idx, w = oracle.route(logits, wl.k)
    v = oracle.vsrc_exchange(x, idx, w, wl.E, wl.R, wl.W)
    order = np.argsort(idx.reshape(-1), kind="stable")
    np.testing.assert_array_equal(v["grouped"], x[order // wl.k])


def test_rejects_unequal_shards():
    with pytest.raises(ValueError):
        oracle.vsrc_exchange(np.zeros((10, 4), np.float32), np.zeros((10, 2), np.int32),
                             np.zeros((10, 2)), 8, 4, 1)
