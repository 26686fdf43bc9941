"""Seeded synthetic inputs with the shapes and value distributions of the
workloads the pages describe (GLM-5.2 MoE block: hidden 6144, 256 experts,
top-8, expert intermediate 2048, one shared expert).

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no unpacking, no products, no routing decisions), so both
the CPU oracle's tests and the device tests may use it.

Distributions (one per input kind):
  packed int4 / int2 weight bytes: uniform over 0..255 (uniform nibbles 0..15,
      uniform crumbs 0..3; pad nibbles/crumbs of odd rows are random too,
      which checks that they are never read),
  int8 weights: uniform over -127..127,
  f32 weights: N(0, 1),
  per-row scales: U[0.001, 0.02] fp32,
  activations x: N(0, 1) fp32,
  router weights: N(0, 0.02) fp32, router bias U[-0.1, 0.1] fp32,
  given routing: K distinct experts per token, uniform without replacement,
      weights U(0,1) rescaled to sum to routed_scale,
  skewed routing: expert popularity p_e proportional to rank_e^-alpha over a
      seeded permutation of ranks, K distinct experts per token drawn without
      replacement in proportion to p (Gumbel top-K on log p).
Exact-arithmetic variants draw integer activations and power-of-two scales.
"""
from __future__ import annotations

import numpy as np

F32, I8, I4, I2 = 0, 1, 2, 3
FMT_NAMES = {"f32": F32, "i8": I8, "i4": I4, "i2": I2}


def rng(*seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(seed) if len(seed) > 1 else seed[0]))


def packed_row_bytes(fmt: int, I: int) -> int:
    """Storage size of one row of I elements (layout, not arithmetic)."""
    return {F32: 4 * I, I8: I, I4: (I + 1) // 2, I2: (I + 3) // 4}[fmt]


def weight_bytes(g: np.random.Generator, fmt: int, O: int, I: int) -> np.ndarray:
    """Packed weight matrix [O, packed_row_bytes(fmt, I)] as uint8."""
    rb = packed_row_bytes(fmt, I)
    if fmt == F32:
        return g.standard_normal((O, I), dtype=np.float32).view(np.uint8).reshape(O, rb)
    if fmt == I8:
        return g.integers(-127, 128, size=(O, I), dtype=np.int8).view(np.uint8)
    return np.frombuffer(g.bytes(O * rb), dtype=np.uint8).reshape(O, rb).copy()


def scales(g: np.random.Generator, O: int) -> np.ndarray:
    return g.uniform(0.001, 0.02, size=O).astype(np.float32)


def activations(g: np.random.Generator, S: int, I: int) -> np.ndarray:
    return g.standard_normal((S, I), dtype=np.float32)


def exact_activations(g: np.random.Generator, S: int, I: int, lo: int = -4, hi: int = 4):
    """Small integers, so every partial sum is an exact fp32 value."""
    return g.integers(lo, hi + 1, size=(S, I)).astype(np.float32)


def exact_scales(g: np.random.Generator, O: int, kmax: int = 6) -> np.ndarray:
    """Powers of two 2^-k, k in 0..kmax: multiplying by them is exact."""
    return np.ldexp(np.ones(O, np.float32), -g.integers(0, kmax + 1, size=O)).astype(np.float32)


def router_weights(g: np.random.Generator, E: int, D: int):
    W = (g.standard_normal((E, D), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    b = g.uniform(-0.1, 0.1, size=E).astype(np.float32)
    return W, b


def routing_uniform(g: np.random.Generator, S: int, K: int, E: int,
                    routed_scale: float = 2.5):
    """K distinct experts per token, uniform without replacement; weights
    U(0,1) rescaled to sum to routed_scale."""
    keys = g.random((S, E))
    idx = np.argsort(keys, axis=1)[:, :K].astype(np.int32)
    w = g.uniform(0.0, 1.0, size=(S, K))
    w = (w / w.sum(axis=1, keepdims=True) * routed_scale).astype(np.float32)
    return idx, w


def zipf_popularity(g: np.random.Generator, E: int, alpha: float = 1.1) -> np.ndarray:
    ranks = g.permutation(E) + 1
    p = ranks.astype(np.float64) ** (-alpha)
    return p / p.sum()


def routing_zipf(g: np.random.Generator, S: int, K: int, E: int, alpha: float = 1.1,
                 routed_scale: float = 2.5):
    """K distinct experts per token drawn without replacement in proportion to
    a Zipf(alpha) popularity (Gumbel top-K); weights as in routing_uniform."""
    p = zipf_popularity(g, E, alpha)
    gumbel = -np.log(-np.log(g.random((S, E))))
    keys = np.log(p)[None, :] + gumbel
    idx = np.argsort(-keys, axis=1)[:, :K].astype(np.int32)
    w = g.uniform(0.0, 1.0, size=(S, K))
    w = (w / w.sum(axis=1, keepdims=True) * routed_scale).astype(np.float32)
    return idx, w


def group_scales(g: np.random.Generator, O: int, I: int, gs: int) -> np.ndarray:
    """One scale per gs elements of each of O rows: [O, ceil(I / gs)]."""
    return g.uniform(0.001, 0.02, size=(O, (I + gs - 1) // gs)).astype(np.float32)


def expert_bank(seed: int, fmt: int, E: int, D: int, F: int, experts=None, gs: int = 0):
    """Stacked expert weights; expert e is drawn from its own stream
    (seed, e), so any subset can be regenerated alone.  Returns a dict with
    wg, wu [E,F,rb(D)], wd [E,D,rb(F)], sg, su [E,F], sd [E,D]; with gs > 0
    (grouped-scale int4) sg, su [E,F,ceil(D/gs)], sd [E,D,ceil(F/gs)] and
    gs (the weights are the same as with gs = 0)."""
    rbD, rbF = packed_row_bytes(fmt, D), packed_row_bytes(fmt, F)
    ids = range(E) if experts is None else experts
    n = len(ids)
    sdim = (lambda O, I: (O,)) if gs <= 0 else (lambda O, I: (O, (I + gs - 1) // gs))
    out = dict(fmt=fmt, E=E, D=D, F=F,
               wg=np.empty((n, F, rbD), np.uint8), wu=np.empty((n, F, rbD), np.uint8),
               wd=np.empty((n, D, rbF), np.uint8),
               sg=np.empty((n,) + sdim(F, D), np.float32), su=np.empty((n,) + sdim(F, D), np.float32),
               sd=np.empty((n,) + sdim(D, F), np.float32))
    if gs > 0:
        out["gs"] = gs
    for j, e in enumerate(ids):
        g = rng(seed, int(e))
        out["wg"][j] = weight_bytes(g, fmt, F, D)
        out["wu"][j] = weight_bytes(g, fmt, F, D)
        out["wd"][j] = weight_bytes(g, fmt, D, F)
        if gs > 0:
            out["sg"][j] = group_scales(g, F, D, gs)
            out["su"][j] = group_scales(g, F, D, gs)
            out["sd"][j] = group_scales(g, D, F, gs)
        else:
            out["sg"][j] = scales(g, F)
            out["su"][j] = scales(g, F)
            out["sd"][j] = scales(g, D)
    return out


def shared_mlp(seed: int, fmt: int, D: int, F: int, gs: int = 0):
    g = rng(seed, 1_000_003)
    wg, wu, wd = weight_bytes(g, fmt, F, D), weight_bytes(g, fmt, F, D), weight_bytes(g, fmt, D, F)
    if gs > 0:
        return dict(fmt=fmt, F=F, wg=wg, wu=wu, wd=wd, sg=group_scales(g, F, D, gs),
                    su=group_scales(g, F, D, gs), sd=group_scales(g, D, F, gs), gs=gs)
    return dict(fmt=fmt, F=F, wg=wg, wu=wu, wd=wd, sg=scales(g, F), su=scales(g, F), sd=scales(g, D))
