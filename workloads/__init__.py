"""Seeded synthetic inputs for the MoE layer share.

This module is shared by the oracle-side tests and the GPU side.  It holds
no arithmetic of the method itself: only random draws, the float32 -> bf16
round-to-nearest-even encoding of the drawn inputs, and the construction of
load skew (a logit bias, a boosted router column), which are properties of
the synthetic workloads, not of the layer.

Workloads (sizes as stated for the benchmark configurations):

* ``tiny``      T=64, d=256, I=128, E=8, top-2, fp32 x and weights, seed 0.
* ``mid``       T=4096, d=4096, I=1024, E=16, top-4, bf16, 4 experts/wave.
* ``v4share``   T=8192, d=7168, I=2048, 32 local of 256 global experts,
                top-8 over all 256, bf16, 8 waves of 4 experts.
* ``decode``    T in {1, 8, 32, 128}, d=7168, I=2048, E=32, top-8,
                Zipf(1.2)-skewed popularity via a logit bias, bf16.
* ``stress``    T in {1, 17, 256, 4096, 16384}, d=4096, I=1536, E=64,
                top-6, one hot expert chosen by about half the tokens,
                256 fixed probe tokens at random positions, dout ~ N(0, 1).

``ungated(wl)`` is the same layer with an ungated expert (one input
projection W1 instead of W1 and W3) at the same expert parameter count:
intermediate size 3I/2, so that d * 3I/2 * 2 = 3 d I, rounded up to a
multiple of 128 (only the tiny layer's 192 moves, to 256).

Random streams: numpy ``SeedSequence(seed).spawn`` in the fixed order
x, Wg, W1, W3, W2, bias/hot-direction, probes, positions, dout.  Values are
drawn as float32 and, for bf16 workloads, rounded to bf16 (RNE).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "ungated", "make_inputs", "bf16_bits", "bf16_value"]


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    I: int
    E_global: int
    E_local: int
    k: int
    G: int = 4
    e_begin: int = 0
    dtype: str = "bf16"          # "f32" (tiny) or "bf16"
    skew: str = "none"           # "none" | "zipf" | "hot"
    T_sweep: tuple = field(default_factory=tuple)
    seed: int = 0

    @property
    def waves(self) -> int:
        return self.E_local // self.G

    def with_T(self, T: int) -> "Workload":
        return replace(self, T=T)


WORKLOADS = {
    "tiny": Workload("tiny", T=64, d=256, I=128, E_global=8, E_local=8, k=2, dtype="f32"),
    "mid": Workload("mid", T=4096, d=4096, I=1024, E_global=16, E_local=16, k=4),
    "v4share": Workload("v4share", T=8192, d=7168, I=2048, E_global=256, E_local=32, k=8),
    "decode": Workload("decode", T=128, d=7168, I=2048, E_global=32, E_local=32, k=8,
                       skew="zipf", T_sweep=(1, 8, 32, 128)),
    "stress": Workload("stress", T=16384, d=4096, I=1536, E_global=64, E_local=64, k=6,
                       skew="hot", T_sweep=(1, 17, 256, 4096, 16384)),
}

N_PROBES = 256
ZIPF_S = 1.2
HOT_SCALE = 100.0


def get(name: str) -> Workload:
    return WORKLOADS[name]


def ungated(wl: Workload | str) -> Workload:
    """The workload's layer with an ungated expert at (about) the same
    parameter count: W1 [d, I'] and W2 [I', d] with I' = 3I/2 rounded up to
    a multiple of 128.  The generator still draws a W3, which such a layer
    does not read."""
    if isinstance(wl, str):
        wl = get(wl)
    I = -(-(3 * wl.I // 2) // 128) * 128
    return replace(wl, name=wl.name + "_ungated", I=I)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, as_bf16: bool, chunk_rows: int = 0):
    """N(0, std^2) draws as float32, optionally rounded to bf16 bits.

    Large tensors are drawn in leading-dimension chunks to bound host memory;
    the chunking never changes the values (one generator, consumed in order).
    """
    shape = tuple(int(s) for s in shape)
    if not as_bf16:
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    out = np.empty(shape, dtype=np.uint16)
    lead = shape[0] if shape else 1
    step = max(1, chunk_rows or lead)
    for s in range(0, lead, step):
        e = min(lead, s + step)
        v = rng.standard_normal((e - s,) + shape[1:], dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:e] = bf16_bits(v)
    return out


def make_inputs(wl: Workload | str, T: int | None = None, need_dout: bool = False,
                weights: bool = True) -> dict:
    """Generate one workload's inputs.

    Returns numpy arrays: ``x`` [T, d], ``Wg`` [d, E_global], ``bias``
    [E_global] float32 or None, ``W1``/``W3`` [E_local, d, I], ``W2``
    [E_local, I, d], optional ``dout`` [T, d] and, for ``stress``,
    ``probe_pos`` (positions of the first min(T, 256) probe tokens).
    bf16 tensors are uint16 bit patterns; fp32 tensors are float32.
    Weights do not depend on T, so every T of a sweep sees the same layer.
    """
    if isinstance(wl, str):
        wl = get(wl)
    T = wl.T if T is None else int(T)
    bf = wl.dtype == "bf16"
    ss = np.random.SeedSequence(wl.seed).spawn(9)
    r_x, r_g, r_w1, r_w3, r_w2, r_b, r_probe, r_pos, r_dout = (np.random.default_rng(s) for s in ss)
    d, I, Eg, El = wl.d, wl.I, wl.E_global, wl.E_local
    out: dict = {"workload": wl, "T": T}

    # Router weights, then the load-skew construction.
    Wg32 = r_g.standard_normal((d, Eg), dtype=np.float32) * np.float32(0.02)
    bias = None
    if wl.skew == "zipf":
        # popularity of expert e proportional to rank_e^-s, via a logit bias
        ranks = r_b.permutation(Eg) + 1
        bias = (-ZIPF_S * np.log(ranks.astype(np.float64))).astype(np.float32)
    elif wl.skew == "hot":
        # one router column along a random unit direction, scaled so that its
        # logit is positive (and dominant) for about half of the tokens
        u = r_b.standard_normal(d).astype(np.float64)
        u /= np.linalg.norm(u)
        hot = int(r_b.integers(Eg))
        Wg32[:, hot] = (HOT_SCALE * u).astype(np.float32)
        out["hot_expert"] = hot
    out["Wg"] = bf16_bits(Wg32) if bf else Wg32
    out["bias"] = bias

    # Token activations.
    if wl.skew == "hot":
        probes = r_probe.standard_normal((N_PROBES, d), dtype=np.float32)
        # positions and fillers depend on T through a T-specific stream
        pos_rng = np.random.default_rng([wl.seed, 7, T])
        fill_rng = np.random.default_rng([wl.seed, 11, T])
        n_p = min(T, N_PROBES)
        pos = np.sort(pos_rng.permutation(T)[:n_p]) if T > 0 else np.zeros(0, np.int64)
        x32 = fill_rng.standard_normal((T, d), dtype=np.float32)
        x32[pos] = probes[:n_p]
        out["probe_pos"] = pos
        out["x"] = bf16_bits(x32)
    else:
        x = _normal(r_x, (T, d), 1.0, bf)
        out["x"] = x

    if weights:
        out["W1"] = _normal(r_w1, (El, d, I), 0.02, bf, chunk_rows=1)
        out["W3"] = _normal(r_w3, (El, d, I), 0.02, bf, chunk_rows=1)
        out["W2"] = _normal(r_w2, (El, I, d), 0.02, bf, chunk_rows=1)
    if need_dout:
        dout_rng = np.random.default_rng([wl.seed, 13, T])
        out["dout"] = _normal(dout_rng, (T, d), 1.0, True)
    return out
