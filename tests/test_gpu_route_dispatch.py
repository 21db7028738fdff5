"""moe_route_dispatch (routing, index stage, statistics and the dispatch copy; the
routing kernel and the one-launch dispatch when all T*k picks fit one 1024-pick
batch) against the oracle and against the separate moe_route +
moe_dispatch_index + moe_dispatch_copy + moe_stats calls (the multi-launch
index stage), on the GPU.

Bars: indices, counts, offsets, positions, row maps, statistics and send rows
bit-exact; weights within 1e-6 relative of the oracle and identical to
moe_route's. Cases cover the one-launch form (the decode workload, whose 1024
picks fill the batch exactly; the tiny workload; one token; one expert; k = E;
E = 1024; k = 32; waves; ties; fp32 rows of 16 bytes) and the three-launch
form beyond one batch.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth
from test_gpu_parity import DEV, INDEX_KEYS, assert_weights, check_index, dev, host, shape_of


def _edge(T, H, E, k, R, W, dtype="bf16", routing="iid", seed=3):
    return synth.Workload("edge", T=T, H=H, dtype=dtype, E=E, k=k, R=R, W=W, routing=routing,
                          seed=seed)


pytestmark = pytest.mark.gpu

CASES = {
    "decode_hot": synth.WORKLOADS["decode_hot"],
    "tiny": synth.WORKLOADS["tiny"],
    "T1_k1_E1": _edge(1, 8, 1, 1, 1, 1),
    "T1": _edge(1, 64, 8, 2, 4, 1),
    "k_eq_E": _edge(37, 16, 8, 8, 2, 2),
    "E1024_k1_T1024": _edge(1024, 16, 1024, 1, 8, 4),
    "E64_k32_T32": _edge(32, 64, 64, 32, 4, 2),
    "waves_ragged": _edge(100, 256, 64, 6, 4, 4),
    "ties": _edge(200, 16, 16, 4, 4, 2, routing="ties"),
    "E6_scalar_route": _edge(123, 8, 6, 3, 3, 1),
    "f32_row16B": _edge(64, 4, 16, 4, 4, 1, dtype="f32"),
    # beyond one batch: the routing kernel with counting, placing, copy
    "zipf_three_launches": synth.WORKLOADS["zipf"],
    "T1025_k1": _edge(1025, 32, 16, 1, 4, 2),
}


def _oracle(wl, logits, x):
    idx_o, w_o = oracle.route(logits, wl.k)
    ref = oracle.dispatch(x, idx_o, wl.E, wl.R, wl.W)
    return idx_o, w_o, ref


def _fused(wl, logits_d, x_d, stats=True):
    shape = shape_of(wl, logits_d.shape[0])
    out = moe.alloc_dispatch(shape, DEV)
    out["send_buf"].view(torch.uint8).fill_(0xA5)
    idx = torch.empty((shape.T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((shape.T, wl.k), dtype=torch.float32, device=DEV)
    raw = torch.empty((moe.STATS_BYTES,), dtype=torch.uint8, device=DEV) if stats else None
    moe.route_dispatch(logits_d, x_d, shape, out, idx, w, stats=raw)
    return idx, w, out, raw


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_route_dispatch_parity(name):
    wl = CASES[name]
    print(f"[route_dispatch] {name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} R={wl.R} W={wl.W} "
          f"{'one-launch dispatch' if wl.T * wl.k <= 1024 else 'three launches'}", flush=True)
    logits, x = synth.logits(wl), synth.hidden(wl)
    idx_o, w_o, ref = _oracle(wl, logits, x)
    ld, xd = dev(logits), dev(x)
    idx, w, out, raw = _fused(wl, ld, xd)
    # the separate calls on the same inputs (count + place + copy launches)
    idx_s, w_s = moe.route(ld, wl.k)
    sep = moe.alloc_dispatch(shape_of(wl), DEV)
    moe.dispatch_index(idx_s, shape_of(wl), sep)
    moe.dispatch_copy(xd, sep["pos"], shape_of(wl), sep["send_buf"])
    st_s = moe.stats(sep["expert_counts"], wl.R)
    torch.cuda.synchronize()

    np.testing.assert_array_equal(host(idx), idx_o)
    assert_weights(host(w), w_o)
    check_index(out, ref)
    n = ref["nrows"]
    np.testing.assert_array_equal(host(out["send_buf"])[:n], ref["send_buf"])
    assert moe.stats_to_dict(raw) == oracle.stats(ref["expert_counts"], wl.R)
    assert torch.equal(idx, idx_s) and torch.equal(w, w_s)
    for key in INDEX_KEYS:
        assert torch.equal(out[key], sep[key]), key
    assert torch.equal(out["row_token"][:n], sep["row_token"][:n])
    assert torch.equal(_bits(out["send_buf"][:n]), _bits(sep["send_buf"][:n]))
    assert moe.stats_to_dict(raw) == st_s


def test_route_dispatch_repeat_and_no_stats():
    """The decode workload twice into the same buffers (the second call without
    statistics): identical outputs."""
    wl = synth.WORKLOADS["decode_hot"]
    logits, x = dev(synth.logits(wl)), dev(synth.hidden(wl))
    idx, w, out, raw = _fused(wl, logits, x)
    torch.cuda.synchronize()
    first = {key: v.clone() for key, v in out.items()}
    shape = shape_of(wl)
    out["send_buf"].view(torch.uint8).fill_(0)
    moe.route_dispatch(logits, x, shape, out, idx, w, stats=None)
    torch.cuda.synchronize()
    for key in INDEX_KEYS + ("row_token", "send_buf"):
        assert torch.equal(_bits(out[key]) if key == "send_buf" else out[key],
                           _bits(first[key]) if key == "send_buf" else first[key]), key


def test_route_dispatch_empty():
    empty = synth.Workload("edge", T=0, H=16, dtype="bf16", E=8, k=2, R=4, W=2, routing="iid",
                           seed=1)
    shape = shape_of(empty)
    out = moe.alloc_dispatch(shape, DEV)
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "wave_offsets"):
        out[key].fill_(-7)
    raw = torch.full((moe.STATS_BYTES,), 0xAB, dtype=torch.uint8, device=DEV)
    idx = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    w = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    moe.route_dispatch(torch.empty((0, 8), dtype=torch.float32, device=DEV),
                       torch.empty((0, 16), dtype=torch.bfloat16, device=DEV), shape, out, idx, w,
                       stats=raw)
    torch.cuda.synchronize()
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "wave_offsets"):
        assert (host(out[key]) == 0).all(), key
    assert moe.stats_to_dict(raw)["total"] == 0


@pytest.mark.parametrize("T,E,k,R,W", [(128, 128, 8, 16, 1), (300, 16, 3, 4, 2), (1, 4, 1, 2, 1)])
def test_one_launch_dispatch_dropped_ids(T, E, k, R, W):
    """moe_dispatch's one-launch form with ids outside [0, E) among the picks
    (dropped: not counted, pos = -1, no row): equal to the oracle and to the
    count + place + copy launches, every output."""
    wl = _edge(T, 64, E, k, R, W, seed=T)
    print(f"[dispatch one launch] dropped ids: T={T} E={E} k={k} R={R} W={W}", flush=True)
    x = synth.hidden(wl)
    idx_o, _ = oracle.route(synth.logits(wl), k)
    g = np.random.default_rng(T)
    drop = g.random(idx_o.shape) < 0.2
    idx_o = np.where(drop, g.choice([-1, E, E + 7, -100], idx_o.shape), idx_o).astype(np.int32)
    ref = oracle.dispatch(x, idx_o, E, R, W)
    xd, idd = dev(x), dev(idx_o)
    got = moe.dispatch(xd, idd, E, R, W)
    sep = moe.alloc_dispatch(shape_of(wl), DEV)
    moe.dispatch_index(idd, shape_of(wl), sep)
    moe.dispatch_copy(xd, sep["pos"], shape_of(wl), sep["send_buf"])
    torch.cuda.synchronize()
    check_index(got, ref)
    n = ref["nrows"]
    np.testing.assert_array_equal(host(got["send_buf"])[:n], ref["send_buf"])
    for key in INDEX_KEYS:
        assert torch.equal(got[key], sep[key]), key
    assert torch.equal(got["row_token"][:n], sep["row_token"][:n])
    assert torch.equal(_bits(got["send_buf"][:n]), _bits(sep["send_buf"][:n]))
