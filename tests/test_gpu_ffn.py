"""Parity of the MFMA grouped SwiGLU expert FFN with the oracle, on the GPU.

The GPU accumulates in fp32 in MFMA order; the oracle in double. Both round the
intermediate h and the output to bf16. Bar: |out_gpu - out_f64| <= 2^-7 |out_f64|
+ atol, where atol covers the rare bf16 rounding of an h element that falls on
the other side of a tie (each moves an output by |Wd| * ulp(h), ~1e-4 here);
a wrong row, expert, weight or index shows up as O(0.1-1) errors.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth
from test_gpu_parity import dev, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ffn_setup(wl, std):
    logits, x = synth.logits(wl), synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=std)
    idx_o, w_o = oracle.route(logits, wl.k)
    ec, _ = oracle.counts(idx_o, wl.E, wl.R, wl.W)
    eo, _, _ = oracle.offsets(ec, wl.R, wl.W)
    nrows = int(ec.sum())
    pos, rt = oracle.positions(idx_o, wl.E, eo, nrows)
    return logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt


def _row_expert(ec, eo, rows):
    nonempty = np.nonzero(ec > 0)[0]
    starts = eo[nonempty]
    order = np.argsort(starts)
    return nonempty[order][np.searchsorted(starts[order], rows, side="right") - 1]


def _check_rows(got_bits, o64, atol):
    got = oracle.bf16_to_f64(got_bits)
    err = np.abs(got - o64)
    bad = err > 2.0**-7 * np.abs(o64) + atol
    assert not bad.any(), f"{bad.sum()} of {bad.size} outside tolerance; max err {err.max()}"


def _run_gpu(wl, x, gu, dn, idx_o):
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    out = moe.dispatch(dev(x), dev(idx_o), wl.E, wl.R, wl.W)
    eo_gpu = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                               dev(gu), dev(dn))
    return shape, out, eo_gpu


@pytest.mark.parametrize("T,E,H,I,k,seed", [(300, 4, 256, 128, 2, 1), (77, 5, 128, 64, 3, 2),
                                            (1000, 16, 256, 192, 2, 3)])
def test_swiglu_small_full(T, E, H, I, k, seed):
    wl = synth.Workload("ffn", T=T, H=H, dtype="bf16", E=E, k=k, R=1, W=1, routing="zipf0.5",
                        expert="swiglu", I=I, seed=seed)
    print(f"[ffn] T={T} E={E} H={H} I={I} k={k}", flush=True)
    logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt = _ffn_setup(wl, std=0.1)
    shape, out, eo_gpu = _run_gpu(wl, x, gu, dn, idx_o)
    torch.cuda.synchronize()
    nrows = int(ec.sum())
    rows = np.arange(nrows)
    o64, _ = oracle.expert_swiglu_rows(x[rt[rows]], _row_expert(ec, eo, rows), gu, dn)
    _check_rows(host(eo_gpu), o64, atol=2e-3)


@pytest.mark.parametrize("H,I", [(128, 64), (256, 128)])  # 128- and 256-row tile paths
def test_swiglu_empty_and_ragged_experts(H, I):
    # experts with 0, 1 and 257 rows (m-tile tails of both tile sizes), routed by hand
    E, k = 4, 1
    T = 259
    idx = np.zeros((T, k), np.int32)
    idx[:257, 0] = 2
    idx[257, 0] = 0
    idx[258, 0] = 3
    wl = synth.Workload("ffn", T=T, H=H, dtype="bf16", E=E, k=k, R=1, W=1, routing="iid",
                        expert="swiglu", I=I, seed=4)
    x = synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=0.1)
    ec, _ = oracle.counts(idx, E, 1, 1)
    eo, _, _ = oracle.offsets(ec, 1, 1)
    pos, rt = oracle.positions(idx, E, eo, T)
    shape, out, eo_gpu = _run_gpu(wl, x, gu, dn, idx)
    torch.cuda.synchronize()
    rows = np.arange(T)
    o64, _ = oracle.expert_swiglu_rows(x[rt], _row_expert(ec, eo, rows), gu, dn)
    _check_rows(host(eo_gpu), o64, atol=2e-3)


def test_swiglu_validation():
    wl = synth.WORKLOADS["local_layer"]
    sh = moe.Shape(8, 4096, 16, 2, 1, 1, torch.bfloat16)
    assert moe.expert_swiglu_workspace_bytes(sh, 1408) == 16 * 1408 * 2
    assert moe.expert_swiglu_workspace_bytes(sh, 100) == 0
    t = torch.empty(16, dtype=torch.uint8, device=DEV)
    cs = sh.c()
    L = moe.lib()
    import ctypes
    P = ctypes.c_void_p(t.data_ptr())
    assert L.moe_expert_swiglu(ctypes.byref(cs), 100, P, P, P, P, P, P, P, 1 << 30, None) == -1
    sh32 = moe.Shape(8, 4096, 16, 2, 1, 1, torch.float32).c()
    assert L.moe_expert_swiglu(ctypes.byref(sh32), 1408, P, P, P, P, P, P, P, 1 << 30, None) == -4
    assert L.moe_expert_swiglu(ctypes.byref(cs), 1408, P, P, P, P, P, P, P, 10, None) == -3
    del wl


def test_local_layer_full_size_sampled():
    """The local-layer workload at full size (T=8192, E=16, H=4096, I=1408,
    weights N(0, 0.02^2)): FFN rows sampled across every expert, and combined
    tokens end to end."""
    wl = synth.WORKLOADS["local_layer"]
    print(f"[ffn] local_layer full T={wl.T} H={wl.H} E={wl.E} I={wl.I}", flush=True)
    logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt = _ffn_setup(wl, std=0.02)
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    idx, w = moe.route(dev(logits), wl.k)
    out = moe.dispatch(dev(x), idx, wl.E, wl.R, wl.W)
    eo_gpu = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                               dev(gu), dev(dn))
    y = moe.combine(eo_gpu, w, out["pos"], shape)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), idx_o)
    np.testing.assert_array_equal(host(out["pos"]), pos)

    g = np.random.default_rng(7)
    firsts = eo[ec > 0]
    lasts = (eo + ec - 1)[ec > 0]
    rows = np.unique(np.concatenate([firsts, lasts, g.integers(0, int(ec.sum()), 24)]))
    o64, _ = oracle.expert_swiglu_rows(x[rt[rows]], _row_expert(ec, eo, rows), gu, dn)
    got = host(eo_gpu[torch.from_numpy(rows).to(DEV)])
    _check_rows(got, o64, atol=1e-3)

    # combined tokens: y_t = sum_i w_ti * bf16(FFN_{e_ti}(x_t)) (expert rows are
    # stored in bf16); each term carries the FFN tolerance, y its own rounding
    toks = np.unique(np.concatenate([[0, wl.T - 1], g.integers(0, wl.T, 6)]))
    y_ref = np.zeros((len(toks), wl.H))
    bound = np.zeros((len(toks), wl.H))
    for j, t in enumerate(toks):
        o64, o16 = oracle.expert_swiglu_rows(np.repeat(x[t:t + 1], wl.k, 0), idx_o[t], gu, dn)
        terms = w_o[t][:, None] * oracle.bf16_to_f64(o16)
        y_ref[j] = terms.sum(0)
        bound[j] = (w_o[t][:, None] * (2.0**-7 * np.abs(o64) + 1e-3)).sum(0)
    yg = oracle.bf16_to_f64(host(y[torch.from_numpy(toks).to(DEV)]))
    err = np.abs(yg - y_ref)
    assert (err <= bound + 2.0**-8 * np.abs(y_ref)).all(), f"max combine err {err.max()}"


def test_swiglu_chains_follow_caller_stream():
    """On a stream of the caller's own, with no synchronisation between calls:
    the side-stream chain must start after the dispatch queued before it and
    the combine queued after it must see both chains' rows."""
    wl = synth.Workload("ffn", T=2048, H=256, dtype="bf16", E=16, k=2, R=1, W=1,
                        routing="zipf0.5", expert="swiglu", I=192, seed=5)
    print(f"[ffn] caller stream: T={wl.T} E={wl.E} H={wl.H} I={wl.I}", flush=True)
    logits, x, gu, dn, idx_o, w_o, ec, eo, pos, rt = _ffn_setup(wl, std=0.1)
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    xd, gud, dnd, ld = dev(x), dev(gu), dev(dn), dev(logits)
    torch.cuda.synchronize()
    ref = None
    for attempt in range(2):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            idx, w = moe.route(ld, wl.k)
            out = moe.alloc_dispatch(shape, DEV)
            out["send_buf"].view(torch.uint8).fill_(0xA5)  # stale rows would show
            moe.dispatch_index(idx, shape, out)
            moe.dispatch_copy(xd, out["pos"], shape, out["send_buf"])
            eo_gpu = torch.empty_like(out["send_buf"])
            eo_gpu.view(torch.uint8).fill_(0x5A)
            moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                              gud, dnd, expert_out=eo_gpu)
            y = moe.combine(eo_gpu, w, out["pos"], shape)
            got = (eo_gpu.clone(), y.clone())
        s.synchronize()
        # the combine queued behind the FFN on the caller's stream must equal
        # one run after everything has finished
        y_after = moe.combine(got[0], w, out["pos"], shape)
        torch.cuda.synchronize()
        assert torch.equal(got[1].view(torch.uint8), y_after.view(torch.uint8))
        if ref is None:
            ref = got
            nrows = int(ec.sum())
            rows = np.arange(nrows)
            o64, _ = oracle.expert_swiglu_rows(x[rt[rows]], _row_expert(ec, eo, rows), gu, dn)
            _check_rows(host(got[0]), o64, atol=2e-3)
        else:  # a second stream, same results bit for bit
            assert torch.equal(got[0].view(torch.uint8), ref[0].view(torch.uint8))
            assert torch.equal(got[1].view(torch.uint8), ref[1].view(torch.uint8))
