"""The FFN rounding bound (tests/ffn_tolerance.py) on the CPU: an fp32 evaluation
of the SwiGLU rows in another summation order (torch's fp32 matmuls, fp32 SiLU,
bf16 rounding of h and of the output) stays inside it, and planted mistakes
(a wrong expert, a dropped K step of the gate/up product, a dropped term of
the down product) fall outside it."""
import numpy as np
import pytest
import torch

import oracle
import synth
from ffn_tolerance import TIGHT_FRACTION, check_rows, round_bf16, swiglu_rows_bound


def _fp32_rows(rows, re, gu, dn, drop_k=0, drop_j=None):
    s = torch.from_numpy(oracle.bf16_to_f64(rows)).float()
    I = dn.shape[2]
    out = np.empty((rows.shape[0], rows.shape[1]), np.uint16)
    for e in np.unique(re):
        sel = np.nonzero(re == e)[0]
        wg = torch.from_numpy(oracle.bf16_to_f64(gu[e])).float()
        wd = torch.from_numpy(oracle.bf16_to_f64(dn[e])).float()
        ss = s[sel].clone()
        if drop_k:
            ss[:, :drop_k] = 0
        a = ss @ wg.T
        g, u = a[:, :I], a[:, I:]
        h = ((g / (1 + torch.exp(-g))) * u).to(torch.bfloat16).float()
        if drop_j is not None:
            h[:, drop_j] = 0
        o = (h @ wd.T).to(torch.bfloat16)
        out[sel] = o.view(torch.int16).numpy().view(np.uint16)
    return out


CASES = [(256, 128, 0.1, 2e-3, 5), (1024, 256, 0.05, 2e-3, 6)]


@pytest.mark.parametrize("H,I,std,atol,seed", CASES)
def test_fp32_evaluation_inside_bound(H, I, std, atol, seed):
    wl = synth.Workload("ffn", T=160, H=H, dtype="bf16", E=4, k=1, R=1, W=1, routing="iid",
                        expert="swiglu", I=I, seed=seed)
    rows = synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=std)
    re = np.arange(wl.T) % wl.E
    o64, _, bound = swiglu_rows_bound(rows, re, gu, dn)
    ratio = check_rows(_fp32_rows(rows, re, gu, dn), o64, bound, atol)
    assert ratio < 1.0


@pytest.mark.parametrize("H,I,std,atol,seed", CASES)
@pytest.mark.parametrize("mistake", ["expert", "k_step", "j_term"])
def test_planted_mistakes_fail(H, I, std, atol, seed, mistake):
    wl = synth.Workload("ffn", T=160, H=H, dtype="bf16", E=4, k=1, R=1, W=1, routing="iid",
                        expert="swiglu", I=I, seed=seed)
    rows = synth.hidden(wl)
    gu, dn = synth.swiglu_weights(wl, std=std)
    re = np.arange(wl.T) % wl.E
    o64, _, bound = swiglu_rows_bound(rows, re, gu, dn)
    if mistake == "expert":
        got = _fp32_rows(rows, (re + 1) % wl.E, gu, dn)
    elif mistake == "k_step":
        got = _fp32_rows(rows, re, gu, dn, drop_k=64)
    else:
        got = _fp32_rows(rows, re, gu, dn, drop_j=I // 3)
    with pytest.raises(AssertionError):
        check_rows(got, o64, bound, atol)


def test_round_bf16_matches_torch():
    v = np.random.default_rng(3).standard_normal(20000) * 10.0 ** np.random.default_rng(4).integers(
        -6, 6, 20000)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()
    # exactly representable in fp32 first, so one rounding on both sides
    assert np.array_equal(round_bf16(v.astype(np.float32).astype(np.float64)), ref)
    assert 0 < TIGHT_FRACTION < 0.01
