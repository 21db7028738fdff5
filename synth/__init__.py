"""Seeded synthetic inputs for the MoE routing path.

This module is shared by the tests, the smoke check and the benchmark. It holds
none of the method's arithmetic: it only draws router logits, hidden states and
expert weights with the shapes and value distributions of the five workloads,
and formats them (fp32 -> bf16 bit patterns, round to nearest even).

Every tensor comes from its own numpy PCG64 stream, ``default_rng([seed, id])``,
so one tensor can be regenerated without drawing the others.

The pages measure routing on real corpora and trained models (WikiText, Opus,
Romansh and mock tokens on five MoE models; IMDB/Twitter/WMT traces for Lina).
None of those are available; the skewed bias shapes below stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Stream ids: one independent generator per tensor.
S_LOGIT_NOISE, S_BIAS, S_X, S_HOT_SET, S_HOT_PICK, S_W_GATE_UP, S_W_DOWN, S_PERM = range(1, 9)

# Strength of the Zipf(s=1) log-rank bias of the "zipf" workload. A literal
# s=1 bias over 64 experts makes the hottest expert ~400x the coldest; this
# scale brings hottest/coldest to ~5x (the 4.02x-5.56x hot/cold ratio Lina
# reports for MoE inference), measured on the seed-0 draw and then frozen.
ZIPF_BETA = 0.245
# Logit boost of the experts a "decode_hot" token is steered to.
HOT_BOOST = 8.0


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    dtype: str  # "f32" or "bf16"
    E: int
    k: int
    R: int
    W: int
    routing: str
    expert: str = "scale"  # "scale": expert e is (e+1) * identity; "swiglu": FFN
    I: int = 0  # FFN intermediate size for "swiglu"
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def L(self) -> int:
        return self.E // self.R

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", T=256, H=128, dtype="f32", E=8, k=2, R=4, W=1, routing="iid",
                     note="4 virtual ranks x 2 experts, logits iid N(0,1)"),
    "zipf": Workload("zipf", T=4096, H=2048, dtype="bf16", E=64, k=6, R=8, W=1, routing="zipf1",
                     note="N(0,1) logits + Zipf(s=1) log-rank bias, hottest/coldest ~5x"),
    "dirichlet_waves": Workload("dirichlet_waves", T=16384, H=7168, dtype="bf16", E=256, k=8,
                                R=32, W=8, routing="dirichlet0.3",
                                note="N(0,1) logits + log p, p ~ Dirichlet(0.3), 8 expert waves"),
    "decode_hot": Workload("decode_hot", T=128, H=4096, dtype="bf16", E=128, k=8, R=16, W=1,
                           routing="hot8",
                           note="80% of picks to 8 fixed hot experts, the rest uniform"),
    "local_layer": Workload("local_layer", T=8192, H=4096, dtype="bf16", E=16, k=2, R=1, W=1,
                            routing="zipf0.5", expert="swiglu", I=1408,
                            note="N(0,1) logits + Zipf(s=0.5) bias; SwiGLU FFN I=1408"),
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _zipf_bias(E: int, s: float, scale: float, seed: int) -> np.ndarray:
    """-scale * s * ln(rank_e) with ranks 1..E assigned by a seeded permutation."""
    perm = rng(seed, S_PERM).permutation(E)
    ranks = 1.0 + perm.astype(np.float64)
    return (-scale * s * np.log(ranks)).astype(np.float32)


def _dirichlet_log_bias(E: int, alpha: float, seed: int) -> np.ndarray:
    """ln p, p ~ Dirichlet(alpha * 1_E), drawn in log space so no p underflows:
    ln Gamma(alpha) = ln Gamma(alpha + 1) + ln(U) / alpha (Marsaglia-Tsang boost)."""
    g = rng(seed, S_BIAS)
    lg = np.log(g.standard_gamma(alpha + 1.0, E)) + np.log(g.random(E)) / alpha
    m = lg.max()
    lse = m + np.log(np.exp(lg - m).sum())
    return (lg - lse).astype(np.float32)


def logits(wl: Workload, T: int | None = None) -> np.ndarray:
    """Router logits [T, E] float32 for the workload's routing distribution."""
    T = wl.T if T is None else T
    E = wl.E
    noise = rng(wl.seed, S_LOGIT_NOISE).standard_normal((T, E), dtype=np.float32)
    r = wl.routing
    if r == "iid":
        return noise
    if r == "zipf1":
        return noise + _zipf_bias(E, 1.0, ZIPF_BETA, wl.seed)[None, :]
    if r == "zipf0.5":
        return noise + _zipf_bias(E, 0.5, 1.0, wl.seed)[None, :]
    if r == "dirichlet0.3":
        return noise + _dirichlet_log_bias(E, 0.3, wl.seed)[None, :]
    if r == "hot8":
        return noise + _hot_boost(T, E, wl.k, wl.seed)
    if r == "ties":
        # Integer-valued logits in a narrow range: many exact ties.
        g = rng(wl.seed, S_LOGIT_NOISE)
        return g.integers(-2, 3, size=(T, E)).astype(np.float32)
    raise ValueError(f"unknown routing {r!r}")


def hot_set(E: int, seed: int, n_hot: int = 8) -> np.ndarray:
    return np.sort(rng(seed, S_HOT_SET).choice(E, size=n_hot, replace=False))


def _hot_boost(T: int, E: int, k: int, seed: int, n_hot: int = 8, p_hot: float = 0.8) -> np.ndarray:
    """Per token: h ~ Binomial(k, p_hot) of the hot experts and k - h of the cold
    ones (uniformly, without replacement) get +HOT_BOOST on their logit."""
    hot = hot_set(E, seed, n_hot)
    cold = np.setdiff1d(np.arange(E), hot)
    g = rng(seed, S_HOT_PICK)
    h = np.minimum(g.binomial(k, p_hot, size=T), n_hot)
    h = np.maximum(h, k - cold.size)
    boost = np.zeros((T, E), np.float32)
    # Random subsets via argsort of uniform keys (one draw per row).
    hot_order = np.argsort(g.random((T, n_hot)), axis=1)
    cold_order = np.argsort(g.random((T, cold.size)), axis=1)
    for t in range(T):
        boost[t, hot[hot_order[t, : h[t]]]] = HOT_BOOST
        boost[t, cold[cold_order[t, : k - h[t]]]] = HOT_BOOST
    return boost


def hidden(wl: Workload, T: int | None = None) -> np.ndarray:
    """Token hidden states [T, H] ~ N(0,1): float32, or bf16 bit patterns (uint16)."""
    T = wl.T if T is None else T
    x = rng(wl.seed, S_X).standard_normal((T, wl.H), dtype=np.float32)
    return x if wl.dtype == "f32" else f32_to_bf16_bits(x)


def swiglu_weights(wl: Workload, std: float = 0.02):
    """Expert FFN weights as bf16 bit patterns: w_gate_up [E][2I][H] (gate rows
    0..I-1, up rows I..2I-1) and w_down [E][H][I], entries ~ N(0, std^2)."""
    E, H, I = wl.E, wl.H, wl.I
    gu = rng(wl.seed, S_W_GATE_UP).standard_normal((E, 2 * I, H), dtype=np.float32) * np.float32(std)
    dn = rng(wl.seed, S_W_DOWN).standard_normal((E, H, I), dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(gu), f32_to_bf16_bits(dn)
