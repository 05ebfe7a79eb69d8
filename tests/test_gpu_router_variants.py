"""GPU parity of the router variants and the load-variance loss
(moe_route_logits_ex, moe_aux_loss_ex) against the oracle.

Noisy logits must be bit-identical (both sides round the product and the
sum to fp32 separately, as the page's fp32 code does); indices identical;
weights within 1e-6; the variance loss within 1e-6 relative.  Inputs: logits
with many exact ties and +-0, the gate's own logits of the 64- and 256-expert
workloads, and standard-normal noise draws from a seeded generator."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_harness as H

pytestmark = pytest.mark.gpu

TOL_AUX_REL = 1e-6


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


def tie_logits(T, E, seed):
    r = np.random.default_rng(seed)
    L = r.integers(-3, 4, (T, E)).astype(np.float32)
    L[r.random((T, E)) < 0.1] = -0.0
    L[::4] = r.standard_normal((len(L[::4]), E)).astype(np.float32)
    L[1] = 0.25                                    # all tied
    return L


def run_variant(moe, L, k, mode, tau, noise=None, scale=0.0):
    import torch
    T, E = L.shape
    s = moe.shape(T, 64, E, k, 64, 0.0, tau)
    idx = H.empty((T, k), torch.int32)
    w = H.empty((T, k), torch.float32)
    noisy = H.empty((T, E), torch.float32) if noise is not None else None
    moe.moe_route_logits_ex(s, mode, H.to_dev(L), idx, w, noise=H.to_dev(noise), noise_scale=scale,
                            noisy_logits=noisy)
    torch.cuda.synchronize()
    return H.to_host(idx), H.to_host(w), (H.to_host(noisy) if noisy is not None else None)


@pytest.mark.parametrize("E,tau", [(8, 1.0), (64, 1.0), (100, 0.2), (128, 0.7), (256, 1.0), (1000, 1.5), (1024, 1.0)])
def test_top1_full_softmax(moe, orc, E, tau):
    H.log(f"[top1] E={E} tau={tau}")
    L = tie_logits(777, E, seed=E)
    idx, w, _ = run_variant(moe, L, 1, moe.MOE_ROUTER_TOP1_FULL, tau)
    ridx, rw = orc.route_top1_full(L, tau)
    assert np.array_equal(idx, ridx)
    assert np.abs(w - rw).max() <= H.TOL_W


@pytest.mark.parametrize("E,k,mode", [(64, 1, 1), (64, 2, 0), (256, 1, 1), (128, 8, 0), (1024, 32, 0), (16, 1, 1)])
def test_noisy_routing(moe, orc, E, k, mode):
    H.log(f"[noisy] E={E} k={k} mode={mode}")
    r = np.random.default_rng(E * 7 + k)
    T = 3001
    L = (r.standard_normal((T, E)) * 2).astype(np.float32)
    noise = r.standard_normal((T, E)).astype(np.float32)
    idx, w, noisy = run_variant(moe, L, k, mode, 0.5 if k > 1 else 1.0, noise, 0.1)
    ref_noisy = orc.noisy_logits(L, noise, 0.1)
    assert np.array_equal(noisy.view(np.uint32), ref_noisy.view(np.uint32))
    if mode == moe.MOE_ROUTER_TOP1_FULL:
        ridx, rw = orc.route_top1_full(ref_noisy, 1.0)
    else:
        ridx, rw = orc.route(ref_noisy, k, 0.5)
    assert np.array_equal(idx, ridx)
    assert np.abs(w - rw).max() <= H.TOL_W


def test_topk_mode_equals_route_logits(moe):
    import torch
    L = tie_logits(999, 64, seed=5)
    idx, w, _ = run_variant(moe, L, 2, moe.MOE_ROUTER_TOPK, 1.0)
    s = moe.shape(999, 64, 64, 2, 64)
    i2, w2 = H.empty((999, 2), torch.int32), H.empty((999, 2), torch.float32)
    moe.moe_route_logits(s, H.to_dev(L), i2, w2)
    torch.cuda.synchronize()
    assert np.array_equal(idx, H.to_host(i2)) and np.array_equal(w, H.to_host(w2))


@pytest.mark.parametrize("name", ["skewed_e64", "large_e256"])
def test_stable_layer_routing_full_size(moe, orc, name):
    """The stable layer's routing on the gate's own logits at full size:
    noisy top-1 over the full softmax, then the variance loss of the top-1
    loads."""
    import torch
    from moe_inputs import get, make_gate, make_x
    cfg = get(name)
    H.log(f"[stable] {name}: T={cfg.T} E={cfg.E}")
    Wg, bg = make_gate(cfg)
    inp = {"x": make_x(cfg), "Wg": Wg, "bg": bg}
    T, E = cfg.T, cfg.E
    s = H.make_shape(moe, cfg)
    logits = H.empty((T, E), torch.float32)
    i0, w0 = H.empty((T, cfg.k), torch.int32), H.empty((T, cfg.k), torch.float32)
    moe.moe_route(s, H.to_dev(inp["x"]), H.to_dev(inp["Wg"]), H.to_dev(inp["bg"]), logits, i0, w0,
                  moe.workspace(s))
    noise = np.random.default_rng(11).standard_normal((T, E)).astype(np.float32)
    s1 = moe.shape(T, cfg.d, E, 1, cfg.d_ff, 0.0, 1.0, 0.01)
    idx, w = H.empty((T, 1), torch.int32), H.empty((T, 1), torch.float32)
    noisy = H.empty((T, E), torch.float32)
    moe.moe_route_logits_ex(s1, moe.MOE_ROUTER_TOP1_FULL, logits, idx, w, noise=H.to_dev(noise), noise_scale=0.1,
                            noisy_logits=noisy)
    Hm, routed = H.empty((E, E), torch.int32), H.empty(E, torch.int32)
    moe.moe_coactivation(s1, idx, Hm, routed)
    aux = H.empty(1, torch.float32)
    moe.moe_aux_loss_ex(s1, moe.MOE_LOSS_VARIANCE, routed, aux)
    torch.cuda.synchronize()
    L = H.to_host(logits)
    ref_noisy = orc.noisy_logits(L, noise, 0.1)
    assert np.array_equal(H.to_host(noisy).view(np.uint32), ref_noisy.view(np.uint32))
    ridx, rw = orc.route_top1_full(ref_noisy, 1.0)
    assert np.array_equal(H.to_host(idx), ridx)
    assert np.abs(H.to_host(w) - rw).max() <= H.TOL_W
    _, rr = orc.coactivation(ridx, E)
    assert np.array_equal(H.to_host(routed).astype(np.int64), rr)
    ref_aux = orc.aux_variance(rr, 0.01)
    assert abs(float(H.to_host(aux)[0]) - ref_aux) <= TOL_AUX_REL * ref_aux


@pytest.mark.parametrize("E", [1, 8, 64, 256, 1024])
def test_aux_loss_variants(moe, orc, E):
    import torch
    r = np.random.default_rng(E)
    load = r.integers(0, 5000, E).astype(np.int32)
    s = moe.shape(4096, 64, E, 1, 64, 0.0, 1.0, 0.01)
    a_var, a_share, a_ref = (H.empty(1, torch.float32) for _ in range(3))
    ld = H.to_dev(load)
    moe.moe_aux_loss_ex(s, moe.MOE_LOSS_VARIANCE, ld, a_var)
    moe.moe_aux_loss_ex(s, moe.MOE_LOSS_SHARE, ld, a_share)
    moe.moe_aux_loss(s, ld, a_ref)
    torch.cuda.synchronize()
    want = orc.aux_variance(load.astype(np.int64), 0.01)
    got = float(H.to_host(a_var)[0])
    assert abs(got - want) <= TOL_AUX_REL * max(want, 1e-30) or (want == 0.0 and got == 0.0)
    assert H.to_host(a_share)[0] == H.to_host(a_ref)[0]
