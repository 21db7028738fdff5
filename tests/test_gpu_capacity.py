"""Capacity-factor dispatch (survey section 1.2 eq. (3): overflow dropped in
token order, unused capacity zero-padded) through the C ABI against the oracle,
then the scaled experts and the combine over the padded buffer.

Bars: counts, offsets, positions, row maps and send rows (padding included)
bit-exact; combine stage-isolated bit-exact against the oracle's fp32 fma chain
over the kept picks."""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth
from test_gpu_parity import PARITY, dev, host, shape_of

pytestmark = pytest.mark.gpu

CASES = [("tiny", 1.0), ("tiny", 0.5), ("zipf", 0.5), ("zipf", 1.0), ("zipf", 1.25),
         ("zipf", 4.0), ("dirichlet_waves_T512", 1.0), ("decode_hot", 2.0),
         ("local_layer_T1024_scaled", 0.8)]


def _run(wl, f):
    logits, x = synth.logits(wl), synth.hidden(wl)
    idx_o, w_o = oracle.route(logits, wl.k)
    cap = oracle.expert_capacity(wl.k, f, wl.T, wl.E)
    assert moe.expert_capacity(wl.k, f, wl.T, wl.E) == cap
    ref = oracle.dispatch_capacity(x, idx_o, wl.E, wl.R, wl.W, cap)
    out = moe.dispatch_capacity(dev(x), dev(idx_o), wl.E, wl.R, wl.W, cap)
    torch.cuda.synchronize()
    return logits, x, idx_o, w_o, cap, ref, out


@pytest.mark.parametrize("name,f", CASES)
def test_capacity_dispatch_parity(name, f):
    wl = PARITY[name]
    print(f"[capacity] {name} f={f}: T={wl.T} E={wl.E} k={wl.k} R={wl.R} W={wl.W}", flush=True)
    logits, x, idx_o, w_o, cap, ref, out = _run(wl, f)
    rows = wl.E * cap
    for key in ("kept_counts", "expert_offsets", "rank_counts", "rank_offsets", "wave_offsets",
                "pos"):
        np.testing.assert_array_equal(host(out[key]), ref[key], err_msg=key)
    np.testing.assert_array_equal(host(out["row_token"])[:rows], ref["row_token"])
    np.testing.assert_array_equal(host(out["send_buf"]), ref["send_buf"])

    # scaled experts over the padded buffer, then the combine over the kept picks
    shape = shape_of(wl)
    eo = moe.expert_scale_rows(out["send_buf"], out["expert_offsets"], out["kept_counts"], shape)
    w32 = w_o.astype(np.float32)
    y = moe.combine_rows(eo, dev(w32), out["pos"], shape)
    torch.cuda.synchronize()
    out_o = oracle.expert_scale(ref["send_buf"], ref["expert_offsets"], ref["kept_counts"])
    kept_rows = ref["row_token"] >= 0
    np.testing.assert_array_equal(host(eo)[kept_rows], out_o[kept_rows])
    yq = oracle.combine_f32fma(out_o, w32, ref["pos"], wl.T)
    np.testing.assert_array_equal(host(y), yq)


def test_zero_and_ample_capacity():
    wl = PARITY["zipf"]
    logits, x = synth.logits(wl), synth.hidden(wl)
    idx_o, _ = oracle.route(logits, wl.k)
    # capacity 0: every pick dropped, no rows
    out = moe.dispatch_capacity(dev(x), dev(idx_o), wl.E, wl.R, wl.W, 0)
    torch.cuda.synchronize()
    assert (host(out["pos"]) == -1).all() and (host(out["kept_counts"]) == 0).all()
    assert (host(out["wave_offsets"]) == 0).all()
    # capacity = the largest count: nothing dropped, plain dispatch in padded buckets
    plain = oracle.dispatch(x, idx_o, wl.E, wl.R, wl.W)
    cap = int(plain["expert_counts"].max())
    out = moe.dispatch_capacity(dev(x), dev(idx_o), wl.E, wl.R, wl.W, cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out["kept_counts"]), plain["expert_counts"])
    assert (host(out["pos"]) >= 0).all()
