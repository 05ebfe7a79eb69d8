"""GPU parity of the sliding-window balance loss (moe_aux_loss_window)
against the oracle, call by call: pbar and aux within 1e-6 relative (fp64
on both sides, stored fp32).  Count sequences: seeded random loads with the
skew of the 64-expert workload, the hand-worked W = 3 sequence, W = 1, and
a window longer than the sequence."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_harness as H

pytestmark = pytest.mark.gpu

TOL = 1e-6


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


def run_sequence(moe, counts_seq, T, k, W, lam):
    import torch
    n, E = counts_seq.shape
    s = moe.shape(T, 64, E, k, 64, 0.0, 1.0, lam)
    state = moe.window_state(E, W)
    # one tensor per call: every pointer must be 16-byte aligned
    cs = [H.to_dev(np.ascontiguousarray(counts_seq[b], np.int32)) for b in range(n)]
    aux = [H.empty(1, torch.float32) for _ in range(n)]
    pbar = [H.empty(E, torch.float32) for _ in range(n)]
    for b in range(n):
        moe.moe_aux_loss_window(s, cs[b], state, W, aux[b], pbar[b])
    torch.cuda.synchronize()
    return np.array([H.to_host(a)[0] for a in aux]), np.stack([H.to_host(p) for p in pbar])


def check(moe, orc, counts_seq, T, k, W, lam):
    aux, pbar = run_sequence(moe, counts_seq, T, k, W, lam)
    raux, rpbar = orc.window_aux(counts_seq, T, k, W, lam)
    assert np.all(np.abs(aux - raux) <= TOL * np.abs(raux) + 1e-30)
    assert np.all(np.abs(pbar - rpbar) <= TOL * np.abs(rpbar) + 1e-30)


def skewed_counts(n, E, T, k, seed):
    r = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=np.float64) ** -0.3
    p /= p.sum()
    return np.stack([r.multinomial(T * k, p) for _ in range(n)]).astype(np.int32)


@pytest.mark.parametrize("E,W,n", [(64, 100, 250), (64, 1, 20), (256, 100, 130), (1024, 7, 30), (8, 500, 40), (1, 3, 10)])
def test_window_loss_sequences(moe, orc, E, W, n):
    H.log(f"[window] E={E} W={W} calls={n}")
    T, k = 8192, min(2, E)
    check(moe, orc, skewed_counts(n, E, T, k, seed=E + W), T, k, W, 0.01)


def test_window_loss_worked_example(moe, orc):
    c = np.array([[10, 0], [0, 10], [5, 5], [10, 0], [10, 0], [10, 0]], np.int32)
    aux, pbar = run_sequence(moe, c, 10, 1, 3, 1.0)
    want = np.array([[1.0, 0.0], [0.5, 0.5], [0.5, 0.5], [0.5, 0.5], [25 / 30, 5 / 30], [1.0, 0.0]])
    assert np.abs(pbar - want).max() <= 1e-7
    assert np.abs(aux - 0.5).max() <= 1e-7
    check(moe, orc, c, 10, 1, 3, 1.0)


def test_window_loss_kept_counts_of_the_layer(moe, orc):
    """Counts from the dispatch of successive batches of a real gate."""
    import torch
    from moe_inputs import get, make_gate
    cfg = get("clustered_small")
    Wg, bg = make_gate(cfg)
    s = H.make_shape(moe, cfg)
    ws = moe.workspace(s)
    seq = []
    for b in range(12):
        x = np.random.default_rng(100 + b).standard_normal((cfg.T, cfg.d)).astype(np.float32)
        from moe_inputs import f32_to_bf16_bits
        xd = H.to_dev(f32_to_bf16_bits(x))
        idx, w = H.empty((cfg.T, cfg.k), torch.int32), H.empty((cfg.T, cfg.k), torch.float32)
        moe.moe_route(s, xd, H.to_dev(Wg), H.to_dev(bg), None, idx, w, ws)
        counts = H.empty(cfg.E, torch.int32)
        offsets = H.empty(cfg.E + 1, torch.int32)
        perm = H.empty(moe.moe_max_rows(s), torch.int32)
        slot = H.empty((cfg.T, cfg.k), torch.int32)
        xp = H.empty((moe.moe_max_rows(s), cfg.d), torch.int16)
        moe.moe_dispatch(s, xd, idx, None, counts, offsets, perm, slot, xp, ws)
        torch.cuda.synchronize()
        seq.append(H.to_host(counts))
    check(moe, orc, np.stack(seq), cfg.T, cfg.k, 5, cfg.aux_lambda)
