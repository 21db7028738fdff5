"""Wave-pipelined local layer (irregular AllToAll page, wave-scheduled
pipelining) through the C ABI: per wave a gather dispatch of the wave's rows on
a copy stream and the SwiGLU FFN of the wave's experts on the compute stream.

Bars: the gathered send rows bit-exact against the oracle's dispatch; the
expert rows bit-identical to the unpipelined moe_expert_swiglu on the same send
buffer (same per-element MFMA arithmetic) and within the FFN tolerance of the
oracle's fp64 SwiGLU; the combined tokens bit-identical to the unpipelined
path."""
import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth
from test_gpu_ffn import _check_rows, _row_expert
from test_gpu_parity import DEV, dev, host

pytestmark = pytest.mark.gpu


def _setup(wl, std=0.1):
    logits, x = synth.logits(wl), synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=std)
    idx, w = oracle.route(logits, wl.k)
    return x, gu, dn, idx, w


def _plain(wl, x, gu, dn, idx, w):
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    out = moe.dispatch(dev(x), dev(idx), wl.E, wl.R, wl.W)
    eo = moe.expert_swiglu(out["send_buf"], out["expert_offsets"], out["expert_counts"], shape,
                           dev(gu), dev(dn))
    y = moe.combine(eo, dev(w.astype(np.float32)), out["pos"], shape)
    return shape, out, eo, y


def _waves(wl, x, gu, dn, idx, w, two_streams):
    shape = moe.Shape(wl.T, wl.H, wl.E, wl.k, wl.R, wl.W, torch.bfloat16)
    out = moe.alloc_dispatch(shape, DEV)
    out["send_buf"].fill_(0)
    moe.dispatch_index(dev(idx), shape, out)
    side = torch.cuda.Stream() if two_streams else None
    xd = dev(x)
    eo = moe.swiglu_waves(xd, out, shape, dev(gu), dev(dn), copy_stream=side)
    y = moe.combine(eo, dev(w.astype(np.float32)), out["pos"], shape)
    torch.cuda.synchronize()
    return out, eo, y


# two chains of experts a wave: R1_W1, R1_W2 (one rank), R4_W1 (one wave); the
# others one chain (fewer than eight experts a wave, or a split that is not a
# stride-2 run of expert ids)
CASES = [("R1_W1", 1, 1), ("R1_W2", 1, 2), ("R1_W4", 1, 4), ("R1_W16", 1, 16), ("R2_W2", 2, 2),
         ("R4_W4", 4, 4), ("R4_W1", 4, 1)]


@pytest.mark.parametrize("name,R,W", CASES)
@pytest.mark.parametrize("two_streams", [True, False])
def test_wave_pipeline_matches_plain_and_oracle(name, R, W, two_streams):
    wl = synth.WORKLOADS["local_layer"].with_(T=1024, H=256, I=128, R=R, W=W, seed=11)
    print(f"[waves] {name} two_streams={two_streams}: T={wl.T} H={wl.H} E={wl.E} I={wl.I}",
          flush=True)
    x, gu, dn, idx, w = _setup(wl)
    shape, plain, eo_p, y_p = _plain(wl, x, gu, dn, idx, w)
    out, eo, y = _waves(wl, x, gu, dn, idx, w, two_streams)
    ref = oracle.dispatch(x, idx, wl.E, wl.R, wl.W)
    n = ref["nrows"]
    np.testing.assert_array_equal(host(out["send_buf"])[:n], ref["send_buf"])
    assert torch.equal(eo[:n], eo_p[:n])
    assert torch.equal(y, y_p)
    rows = np.arange(n)
    o64, _ = oracle.expert_swiglu_rows(x[ref["row_token"]], _row_expert(
        ref["expert_counts"], ref["expert_offsets"], rows), gu, dn)
    _check_rows(host(eo)[:n], o64, atol=2e-3)


def test_wave_pipeline_full_size_repeat():
    """The local layer at full size, W = 4 on two streams, twice in a row into
    the same buffers: identical to the unpipelined path both times."""
    wl = synth.WORKLOADS["local_layer"].with_(W=4)
    print(f"[waves full] T={wl.T} H={wl.H} E={wl.E} I={wl.I} W={wl.W}", flush=True)
    x, gu, dn, idx, w = _setup(wl, std=0.02)
    shape, plain, eo_p, y_p = _plain(wl, x, gu, dn, idx, w)
    out = moe.alloc_dispatch(shape, DEV)
    moe.dispatch_index(dev(idx), shape, out)
    side = torch.cuda.Stream()
    xd, gud, dnd = dev(x), dev(gu), dev(dn)
    eo = torch.empty_like(out["send_buf"])
    ws = torch.empty((moe.expert_swiglu_workspace_bytes(shape, wl.I),), dtype=torch.uint8,
                     device=DEV)
    n = int(host(out["expert_counts"]).sum())
    for rep in range(2):
        eo.fill_(0)
        moe.swiglu_waves(xd, out, shape, gud, dnd, expert_out=eo, workspace=ws, copy_stream=side)
        y = moe.combine(eo, dev(w.astype(np.float32)), out["pos"], shape)
        torch.cuda.synchronize()
        assert torch.equal(out["send_buf"][:n], plain["send_buf"][:n]), rep
        assert torch.equal(eo[:n], eo_p[:n]), rep
        assert torch.equal(y, y_p), rep
