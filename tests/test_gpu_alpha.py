"""The GPU Dirichlet alpha fit (digamma series, Newton on ln a) against the
oracle's (exact finite sums, bisection), on the workloads' counts, edge counts
and simulated Dirichlet-multinomial routings.

Bar: within 1e-8 relative (the two roots are found by different arithmetic);
inf / 0 / NaN identical; near-multinomial counts (either side above 1e5) both
above 1e5, since the likelihood is flat there and the inf / finite decision at
the 1e6 end of the search may go either way."""
import math

import numpy as np
import pytest
import torch

import combine_moe_route_03_amd as moe
import oracle
import synth
from test_gpu_parity import DEV, EDGES, PARITY

pytestmark = pytest.mark.gpu


def _check(counts):
    c = np.ascontiguousarray(counts, dtype=np.int32)
    a = moe.dirichlet_alpha(torch.from_numpy(c).to(DEV))
    ref = oracle.dirichlet_alpha(c)
    if ref > 1e5 or a > 1e5:
        assert ref > 1e5 and a > 1e5, (a, ref)
    elif math.isfinite(ref) and ref > 0:
        assert abs(a - ref) <= 1e-8 * ref, (a, ref)
    else:
        assert (math.isnan(a) and math.isnan(ref)) or a == ref, (a, ref)
    return a


@pytest.mark.parametrize("name", list(PARITY) + [f"edge_{n}" for n in EDGES])
def test_alpha_on_workload_counts(name):
    wl = PARITY[name] if name in PARITY else EDGES[name[5:]]
    idx, _ = oracle.route(synth.logits(wl), wl.k)
    _check(np.bincount(idx.ravel(), minlength=wl.E))


@pytest.mark.parametrize("name", ["zipf", "dirichlet_waves", "decode_hot", "local_layer"])
def test_alpha_full_size(name):
    wl = synth.WORKLOADS[name]
    idx, _ = oracle.route(synth.logits(wl), wl.k)
    a = _check(np.bincount(idx.ravel(), minlength=wl.E))
    print(f"[alpha] {name}: {a}", flush=True)


@pytest.mark.parametrize("seed,E,N,alpha", [(0, 256, 131072, 0.3), (1, 1024, 200000, 0.05),
                                            (2, 64, 50000, 5.0), (3, 8, 300, 1.0),
                                            (4, 1024, 5000, 0.5)])
def test_alpha_simulated(seed, E, N, alpha):
    g = np.random.default_rng(seed)
    p = g.dirichlet(np.full(E, alpha))
    _check(np.bincount(g.choice(E, size=N, p=p), minlength=E))


def test_alpha_limits():
    assert math.isnan(_check(np.zeros(16)))
    assert _check(np.array([900] + [0] * 31)) == 0.0
    assert _check(np.full(64, 250)) == math.inf
    assert math.isnan(_check(np.array([5])))
