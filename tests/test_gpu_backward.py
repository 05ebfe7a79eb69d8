"""GPU parity of the layer backward (moe_layer_backward) against the oracle.

The forward runs on the GPU (moe_layer_forward); its routing outputs and
workspace regions feed the backward.  The oracle recomputes everything from
the inputs, routing on the GPU's fp32 logits (the same reading as the
forward parity).  Bars, normwise per gradient tensor:
max|g - g_ref| <= 1e-4 max|g_ref| for fp32 layers and 1e-2 max|g_ref| for
bf16 layers (h is stored in bf16 by the forward and recomputed so here; the
oracle keeps it unrounded).  Small cases and two mid-size cases (several
work items per workgroup at K = 1536; long row segments, where the weight
gradients take the pipelined form) compare every gradient in full; at full
size the gate gradients dWg and dbg in full (the oracle's expert outputs of
every kept row give the routing-weight gradients), the weight gradients of
the two busiest and the two least busy experts, dx of 256 seeded tokens,
idle experts' zeros, and the sums that hold at any size (per-token gate
gradients sum to zero)."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_harness as H
from moe_inputs import get, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 1e-2}
SMALL = ["tiny_fp32", "tiny_fp32_bias", "ragged_fp32", "ragged_bf16", "medium_bf16", "hybrid_small",
         "clustered_small", "single_token", "one_expert", "k_equals_e", "cap_one", "soft_k64_e64", "k100_e200", "k40_fp32",
         "k50_e300"]
# every gradient in full: several items per workgroup at K = 1536; long row
# segments (the weight gradients' pipelined form); segments whose
# weight-gradient operands span 2 GiB (past that form's 32-bit offsets)
MID = ["multi_item", "bw_long_rows", "wgrad_2g"]


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


def forward_backward(moe, cfg, inp, dy, xperm_from_dispatch=False):
    import torch
    dv = H.dev_inputs(inp)
    s = H.make_shape(moe, cfg)
    T, E, k, d, F = cfg.T, cfg.E, cfg.k, cfg.d, cfg.d_ff
    i32, f32 = torch.int32, torch.float32
    ws = moe.workspace(s)
    y, counts, aux = H.empty((T, d), f32), H.empty(E, i32), H.empty(1, f32)
    idx, w, logits = H.empty((T, k), i32), H.empty((T, k), f32), H.empty((T, E), f32)
    moe.moe_layer_forward(s, dv["x"], dv["Wg"], dv["bg"], dv["W1"], dv["b1"], dv["W2"], dv["b2"], y, counts, aux, ws,
                          topk_idx=idx, topk_w=w, logits=logits)
    R = moe.moe_max_rows(s)
    esz = 2 if cfg.dtype == "bf16" else 4

    def region(which, dtype, shape):
        off = moe.moe_workspace_offset(s, which)
        n = int(np.prod(shape)) * (4 if dtype in (i32, f32) else 2)
        return ws[off:off + n].view(dtype).view(*shape)

    slot = region(moe.MOE_WS_SLOT, i32, (T, k))
    offsets = region(moe.MOE_WS_OFFSETS, i32, (E + 1,))
    # a bf16 forward keeps x_perm only in the tile layout: the backward then
    # copies the rows of x itself (x_perm = None); or x_perm from
    # moe_dispatch on the forward's routing (its own workspace)
    xperm = region(moe.MOE_WS_XPERM, f32, (R, d)) if esz == 4 else None
    if xperm_from_dispatch:
        xperm = H.empty((R, d), torch.int16 if esz == 2 else f32)
        moe.moe_dispatch(s, dv["x"], idx, H.empty(E, i32), H.empty(E, i32), H.empty(E + 1, i32), H.empty(R, i32),
                         H.empty((T, k), i32), xperm, moe.workspace(s))
    out = region(moe.MOE_WS_OUT, f32, (R, d))
    bws = moe.backward_workspace(s)
    g = dict(dx=H.empty((T, d), f32), dWg=H.empty((d, E), f32), dbg=H.empty(E, f32), dW1=H.empty((E, d, F), f32),
             db1=H.empty((E, F), f32), dW2=H.empty((E, F, d), f32), db2=H.empty((E, d), f32))
    moe.moe_layer_backward(s, dv["x"], dv["Wg"], dv["W1"], dv["b1"], dv["W2"], H.to_dev(dy), idx, w, slot, offsets,
                           xperm, out, g["dx"], g["dWg"], g["dbg"], g["dW1"], g["db1"], g["dW2"], g["db2"], bws)
    torch.cuda.synchronize()
    return ({n: H.to_host(v) for n, v in g.items()}, H.to_host(logits), H.to_host(counts), H.to_host(offsets))


def dy_of(cfg, seed=77):
    return np.random.default_rng(seed).standard_normal((cfg.T, cfg.d)).astype(np.float32)


@pytest.mark.parametrize("name", SMALL + MID)
def test_backward_every_gradient(moe, orc, name):
    cfg = get(name)
    H.log(f"[backward] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff} {cfg.dtype}")
    inp = make_inputs(cfg)
    dy = dy_of(cfg)
    got, L, _, _ = forward_backward(moe, cfg, inp, dy)
    ref = orc.layer_backward(inp["x"], inp["Wg"], inp["W1"], inp["b1"], inp["W2"], inp["b2"], L, cfg.k,
                             cfg.capacity_factor, cfg.temperature, dy)
    tol = TOL[cfg.dtype]
    for n in ("dx", "dWg", "dbg", "dW1", "db1", "dW2", "db2"):
        H.assert_close_norm(got[n], ref[n], tol, f"{name} {n}")


@pytest.mark.parametrize("name", ["ragged_bf16", "medium_bf16", "ragged_fp32"])
def test_backward_xperm_given_or_copied(moe, name):
    """x_perm passed in (moe_dispatch's row-major rows) and x_perm = None
    (the backward copies the kept rows of x by slot) give the same gradients,
    bit for bit."""
    cfg = get(name)
    inp = make_inputs(cfg)
    dy = dy_of(cfg)
    a, La, _, _ = forward_backward(moe, cfg, inp, dy)
    b, Lb, _, _ = forward_backward(moe, cfg, inp, dy, xperm_from_dispatch=True)
    assert np.array_equal(La, Lb)
    for n in a:
        assert np.array_equal(a[n], b[n]), f"{name} {n}: x_perm given vs copied"


@pytest.mark.parametrize("name", ["skewed_e64", "skewed_e64_literal", "dense_soft_e16"])
def test_backward_full_size(moe, orc, name):
    cfg = get(name)
    H.log(f"[backward-full] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff}")
    inp = make_inputs(cfg)
    dy = dy_of(cfg)
    got, L, counts, offsets = forward_backward(moe, cfg, inp, dy)
    tol = TOL[cfg.dtype]
    idx, w = orc.route(L, cfg.k, cfg.temperature)
    dsp = orc.dispatch(idx, cfg.E, orc.capacity(cfg.T, cfg.E, cfg.k, cfg.capacity_factor))
    assert np.array_equal(dsp["offsets"], offsets)
    slot = dsp["slot"]
    # idle experts: exact zeros
    for e in np.nonzero(counts == 0)[0]:
        for n in ("dW1", "db1", "dW2", "db2"):
            assert not got[n][e].any(), (n, e)
    # weight gradients of the two busiest and two least busy active experts, over all their rows
    act = np.nonzero(counts > 0)[0]
    order = act[np.argsort(counts[act], kind="stable")]
    for e in sorted(set(order[:2].tolist() + order[-2:].tolist())):
        tt, jj = np.nonzero((slot >= 0) & (idx == e))
        _, _, dW1, db1, dW2, db2 = orc.ffn_backward_rows(tt.astype(np.int32), idx[tt, jj], w[tt, jj], inp["x"],
                                                         inp["W1"], inp["b1"], inp["W2"], inp["b2"], dy, cfg.E)
        for n, ref in (("dW1", dW1), ("db1", db1), ("dW2", dW2), ("db2", db2)):
            H.assert_close_norm(got[n][e], ref[e], tol, f"{name} {n}[{e}]")
    # gate gradients in full: the routing-weight gradient of every kept slot
    # is dy[t] . o[row] with the oracle's expert output o of that row
    # (dropped slots: 0)
    kt, kj = np.nonzero(slot >= 0)
    rows = slot[kt, kj]
    o = orc.ffn_rows(kt.astype(np.int32), idx[kt, kj], inp["x"], inp["W1"], inp["b1"], inp["W2"], inp["b2"])
    dw_all = np.zeros((cfg.T, cfg.k))
    dw_all[kt, kj] = np.einsum("nd,nd->n", dy[kt].astype(np.float64), o)
    _, dWg_ref, dbg_ref, dxg_all = orc.route_backward(inp["x"], inp["Wg"], idx, w, dw_all, cfg.temperature)
    H.assert_close_norm(got["dWg"], dWg_ref, tol, f"{name} dWg (full)")
    H.assert_close_norm(got["dbg"], dbg_ref, tol, f"{name} dbg (full)")
    del o, rows
    # dx of sampled tokens: expert path plus gate path of those tokens
    toks = H.sample_tokens(cfg.T, 256, seed=5)
    sel = slot[toks] >= 0
    tt, jj = np.nonzero(sel)
    dw = np.zeros((len(toks), cfg.k))
    dwr, dxp, *_ = orc.ffn_backward_rows(toks[tt].astype(np.int32), idx[toks[tt], jj], w[toks[tt], jj], inp["x"],
                                         inp["W1"], inp["b1"], inp["W2"], inp["b2"], dy, cfg.E)
    dw[tt, jj] = dwr
    dx_ref = np.zeros((len(toks), cfg.d))
    np.add.at(dx_ref, tt, dxp)
    assert np.allclose(dw, dw_all[toks], rtol=1e-9, atol=1e-12)
    H.assert_close_norm(got["dx"][toks], dx_ref + dxg_all[toks], tol, f"{name} dx (sampled)")
    # per-token gate gradients sum to zero over the experts: so do dbg and every row of dWg
    scale = np.abs(got["dbg"]).max() + 1e-30
    assert abs(got["dbg"].sum()) <= 1e-3 * scale * np.sqrt(cfg.E)
    rs = np.abs(got["dWg"].sum(axis=1)).max()
    assert rs <= 1e-3 * (np.abs(got["dWg"]).max() + 1e-30) * np.sqrt(cfg.E)


def test_backward_long_segments(moe, orc):
    """Idle, one-row and long expert segments in one batch: exact zeros for
    the idle experts, full weight gradients of the five least busy active
    experts and of the two whose row counts are nearest 400, sampled dx and
    the gate sums."""
    cfg = get("long_segments")
    H.log(f"[backward-long] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff}")
    inp = make_inputs(cfg)
    dy = dy_of(cfg)
    got, L, counts, offsets = forward_backward(moe, cfg, inp, dy)
    tol = TOL[cfg.dtype]
    idx, w = orc.route(L, cfg.k, cfg.temperature)
    dsp = orc.dispatch(idx, cfg.E, orc.capacity(cfg.T, cfg.E, cfg.k, cfg.capacity_factor))
    assert np.array_equal(dsp["offsets"], offsets)
    slot = dsp["slot"]
    idle = np.nonzero(counts == 0)[0]
    assert len(idle) > 0
    for e in idle:
        for n in ("dW1", "db1", "dW2", "db2"):
            assert not got[n][e].any(), (n, e)
    act = np.nonzero(counts > 0)[0]
    order = act[np.argsort(counts[act], kind="stable")]
    mid = act[np.argsort(np.abs(counts[act] - 400), kind="stable")[:2]]
    for e in sorted(set(order[:5].tolist() + mid.tolist())):
        tt, jj = np.nonzero((slot >= 0) & (idx == e))
        _, _, dW1, db1, dW2, db2 = orc.ffn_backward_rows(tt.astype(np.int32), idx[tt, jj], w[tt, jj], inp["x"],
                                                         inp["W1"], inp["b1"], inp["W2"], inp["b2"], dy, cfg.E)
        for n, ref in (("dW1", dW1), ("db1", db1), ("dW2", dW2), ("db2", db2)):
            H.assert_close_norm(got[n][e], ref[e], tol, f"long_segments {n}[{e}] ({counts[e]} rows)")
    toks = H.sample_tokens(cfg.T, 64, seed=9)
    tt, jj = np.nonzero(slot[toks] >= 0)
    dw = np.zeros((len(toks), cfg.k))
    dwr, dxp, *_ = orc.ffn_backward_rows(toks[tt].astype(np.int32), idx[toks[tt], jj], w[toks[tt], jj], inp["x"],
                                         inp["W1"], inp["b1"], inp["W2"], inp["b2"], dy, cfg.E)
    dw[tt, jj] = dwr
    dx_ref = np.zeros((len(toks), cfg.d))
    np.add.at(dx_ref, tt, dxp)
    _, _, _, dxg = orc.route_backward(inp["x"][toks], inp["Wg"], idx[toks], w[toks], dw, cfg.temperature)
    H.assert_close_norm(got["dx"][toks], dx_ref + dxg, tol, "long_segments dx (sampled)")
    scale = np.abs(got["dbg"]).max() + 1e-30
    assert abs(got["dbg"].sum()) <= 1e-3 * scale * np.sqrt(cfg.E)


def test_backward_repeatable(moe):
    cfg = get("medium_bf16")
    inp = make_inputs(cfg)
    dy = dy_of(cfg)
    a, *_ = forward_backward(moe, cfg, inp, dy)
    b, *_ = forward_backward(moe, cfg, inp, dy)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_backward_soft_e128(moe, orc):
    """The naive soft layer over all 128 experts (k = E = 128, 131072 rows,
    1024 per expert) at full size: the weight and bias gradients of the first
    and last expert over all their rows, dx of 8 seeded tokens (every one of
    their 128 slots) and the gate sums.  The oracle takes each expert's
    weights alone (an expert's gradients depend on its own rows only)."""
    cfg = get("dense_soft_e128")
    H.log(f"[backward-soft128] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff}")
    inp = make_inputs(cfg)
    dy = dy_of(cfg)
    got, L, counts, offsets = forward_backward(moe, cfg, inp, dy)
    tol = TOL[cfg.dtype]
    idx, w = orc.route(L, cfg.k, cfg.temperature)
    assert (counts == cfg.T).all()
    slot = orc.dispatch(idx, cfg.E, orc.capacity(cfg.T, cfg.E, cfg.k, cfg.capacity_factor))["slot"]

    def expert_rows(e, tt, jj):
        sl = lambda a: np.ascontiguousarray(a[e:e + 1])
        return orc.ffn_backward_rows(tt.astype(np.int32), np.zeros(len(tt), np.int32), w[tt, jj], inp["x"],
                                     sl(inp["W1"]), sl(inp["b1"]), sl(inp["W2"]), sl(inp["b2"]), dy, 1)

    for e in (0, cfg.E - 1):
        tt, jj = np.nonzero(idx == e)
        _, _, dW1, db1, dW2, db2 = expert_rows(e, tt, jj)
        for n, ref in (("dW1", dW1), ("db1", db1), ("dW2", dW2), ("db2", db2)):
            H.assert_close_norm(got[n][e], ref[0], tol, f"soft128 {n}[{e}]")
    toks = H.sample_tokens(cfg.T, 8, seed=21)
    dw = np.zeros((len(toks), cfg.k))
    dx_ref = np.zeros((len(toks), cfg.d))
    for e in range(cfg.E):
        ti, jj = np.nonzero(idx[toks] == e)
        dwr, dxp, *_ = expert_rows(e, toks[ti], jj)
        dw[ti, jj] = dwr
        np.add.at(dx_ref, ti, dxp)
    assert (slot[toks] >= 0).all()
    _, _, _, dxg = orc.route_backward(inp["x"][toks], inp["Wg"], idx[toks], w[toks], dw, cfg.temperature)
    H.assert_close_norm(got["dx"][toks], dx_ref + dxg, tol, "soft128 dx (sampled)")
    scale = np.abs(got["dbg"]).max() + 1e-30
    assert abs(got["dbg"].sum()) <= 1e-3 * scale * np.sqrt(cfg.E)
    rs = np.abs(got["dWg"].sum(axis=1)).max()
    assert rs <= 1e-3 * (np.abs(got["dWg"]).max() + 1e-30) * np.sqrt(cfg.E)
