"""Seeded synthetic inputs for the MoE layer forward.

The same host arrays are handed to the CPU oracle and to the HIP library, so
both sides see identical bits.  This module only draws random numbers and
stores them in the layer's input formats; it performs no step of the layer.

Recipe (every tensor has its own PCG64 stream, keyed by (seed, tensor id,
expert id), so one expert's weights can be regenerated on its own):
  x   [T, d]      N(0, 1); for clustered workloads a seeded subset of
                  floor(frac*T) token positions is replaced by
                  centroid + noise*N(0, 1), centroids ~ N(0, I_d),
                  centroid id uniform.
  Wg  [d, E]      N(0, 1/d)   fp32 (variance 1/fan_in)
  bg  [E]         alpha * ln p(rank e+1), p(r) = r^-s / sum_r' r'^-s (Zipf),
                  plus N(0, gate_bias_std^2) for the parity cases; absent
                  when neither is requested.
  W1  [E, d, d_ff]  N(0, 1/d)
  b1  [E, d_ff]     N(0, bias_std^2) (zero when bias_std == 0)
  W2  [E, d_ff, d]  N(0, 1/d_ff)
  b2  [E, d]        N(0, bias_std^2)
Draws are float32; bf16 tensors are the float32 draws rounded to nearest-even
and kept as raw uint16 bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

from .configs import MoEConfig

_X, _WG, _BG, _W1, _B1, _W2, _B2, _CL = 1, 2, 3, 4, 5, 6, 7, 8


def _rng(seed: int, tensor: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, sub])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs are finite normal draws, so NaN handling is not needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def make_x(cfg: MoEConfig) -> np.ndarray:
    x = _normal(_rng(cfg.seed, _X), (cfg.T, cfg.d), 1.0)
    if cfg.cluster_frac > 0:
        r = _rng(cfg.seed, _CL)
        n = int(math.floor(cfg.cluster_frac * cfg.T))
        pos = r.choice(cfg.T, size=n, replace=False)
        cid = r.integers(0, cfg.n_centroids, size=n)
        cent = _normal(r, (cfg.n_centroids, cfg.d), 1.0)
        noise = _normal(r, (n, cfg.d), cfg.cluster_noise)
        x[pos] = cent[cid] + noise
    return _store(x, cfg.dtype)


def make_gate(cfg: MoEConfig):
    wg = _normal(_rng(cfg.seed, _WG), (cfg.d, cfg.E), 1.0 / math.sqrt(cfg.d))
    bg: Optional[np.ndarray] = None
    if cfg.has_gate_bias:
        b = np.zeros(cfg.E, dtype=np.float64)
        if cfg.zipf_s > 0:
            ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
            p = ranks ** (-cfg.zipf_s)
            p /= p.sum()
            b += cfg.zipf_alpha * np.log(p)
        if cfg.gate_bias_std > 0:
            b += _normal(_rng(cfg.seed, _BG), (cfg.E,), cfg.gate_bias_std).astype(np.float64)
        bg = b.astype(np.float32)
    return wg, bg


def make_expert(cfg: MoEConfig, e: int):
    """(W1[e], b1[e], W2[e], b2[e]) of one expert, in storage formats."""
    w1 = _store(_normal(_rng(cfg.seed, _W1, e), (cfg.d, cfg.d_ff), 1.0 / math.sqrt(cfg.d)), cfg.dtype)
    w2 = _store(_normal(_rng(cfg.seed, _W2, e), (cfg.d_ff, cfg.d), 1.0 / math.sqrt(cfg.d_ff)), cfg.dtype)
    if cfg.bias_std > 0:
        b1 = _normal(_rng(cfg.seed, _B1, e), (cfg.d_ff,), cfg.bias_std)
        b2 = _normal(_rng(cfg.seed, _B2, e), (cfg.d,), cfg.bias_std)
    else:
        b1 = np.zeros(cfg.d_ff, np.float32)
        b2 = np.zeros(cfg.d, np.float32)
    return w1, b1, w2, b2


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_experts(cfg: MoEConfig, experts=None):
    """Stacked expert weights for the given expert ids (default: all)."""
    ids = list(range(cfg.E)) if experts is None else list(experts)
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    W1 = np.empty((len(ids), cfg.d, cfg.d_ff), st)
    W2 = np.empty((len(ids), cfg.d_ff, cfg.d), st)
    b1 = np.empty((len(ids), cfg.d_ff), np.float32)
    b2 = np.empty((len(ids), cfg.d), np.float32)

    def fill(i):
        w1, bb1, w2, bb2 = make_expert(cfg, ids[i])
        W1[i], b1[i], W2[i], b2[i] = w1, bb1, w2, bb2

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(len(ids))))
    return W1, b1, W2, b2


def make_inputs(cfg: MoEConfig) -> Dict[str, Optional[np.ndarray]]:
    """All layer inputs as host arrays: x, Wg, bg (or None), W1, b1, W2, b2."""
    x = make_x(cfg)
    wg, bg = make_gate(cfg)
    W1, b1, W2, b2 = make_experts(cfg)
    return dict(x=x, Wg=wg, bg=bg, W1=W1, b1=b1, W2=W2, b2=b2)
