"""Helpers shared by the GPU parity tests: moving the seeded host inputs to
the device, calling each entry point of the HIP library through its
binding, and the tolerances the comparisons use.

Tolerances (written out here so every test states the same bar):
  gate logits   max|L - Lref|  <= 1e-4 * max|Lref|   (normwise, fp64 Lref)
  weights       max|w - wref|  <= 1e-6               (wref from the fp32 logits under test)
  y, FFN rows   max|y - yref|  <= 1e-2 * max|yref|   bf16 experts
                max|y - yref|  <= 1e-4 * max|yref|   fp32 experts
  aux           |aux - ref|    <= 1e-6 * ref
Integer outputs (indices, counts, offsets, perm, slot) must be identical;
routing is compared with the oracle re-run on the GPU's own fp32 logits.
"""
from __future__ import annotations

import sys

import numpy as np

TOL_LOGITS = 1e-4
TOL_W = 1e-6
TOL_Y = {"bf16": 1e-2, "fp32": 1e-4}
TOL_AUX = 1e-6


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    return t.detach().cpu().numpy()


def dev_inputs(inp):
    return {k: to_dev(v) for k, v in inp.items()}


def make_shape(moe, cfg):
    return moe.shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ff, cfg.capacity_factor, cfg.temperature,
                     cfg.aux_lambda, moe.MOE_BF16 if cfg.dtype == "bf16" else moe.MOE_F32)


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def assert_close_norm(got, ref, rel, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    if scale == 0.0:
        assert err == 0.0, f"{what}: reference is zero, max|got| = {err}"
        return 0.0
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel:g} * {scale:.3e}"
    return err / scale


def sample_tokens(T: int, n: int, seed: int = 1234) -> np.ndarray:
    if T <= n:
        return np.arange(T, dtype=np.int32)
    r = np.random.default_rng(seed)
    pick = r.choice(T, size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], pick])).astype(np.int32)
