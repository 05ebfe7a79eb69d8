"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

For every case the fused entry point moe_layer_forward and the separate
entry points (moe_route, moe_dispatch, moe_grouped_ffn, moe_combine,
moe_aux_loss) run on the same seeded inputs as the oracle.  Integer outputs
are compared bit for bit, with the routing re-derived by the oracle from
the GPU's own fp32 logits; floating-point outputs within the tolerances of
gpu_harness.  Small cases, the 16-expert workload and the multi-item case
compare every output element.  The other full-size workloads compare every
integer output in full; of the expert outputs (out_perm) the first and last
row of every 64-row block of every expert segment (so the first and last row
of every grouped-GEMM work item, whatever its row tile), every row of the two
busiest and the two least busy active experts, and the rows of 1024 seeded
tokens, whose y is compared too.
"""
from __future__ import annotations

import numpy as np
import pytest

import gpu_harness as H
from moe_inputs import get, make_inputs

pytestmark = pytest.mark.gpu

SMALL = ["tiny_fp32", "tiny_fp32_bias", "ragged_bf16", "ragged_fp32", "medium_bf16",
         "hybrid_small", "clustered_small", "single_token", "one_expert", "k_equals_e",
         "cap_one", "max_experts", "max_k", "soft_k_equals_e12", "k16_e40", "e100_k5",
         "e200_t33001", "soft_k64_e64", "k100_e200", "k40_fp32", "k50_e300"]
FULL = ["bf16_e16", "multi_item", "skewed_e64", "skewed_e64_literal", "hybrid_e128", "large_e256", "dense_soft_e16",
        "dense_soft_e128", "ragged_large", "ragged_large_even", "wide_d"]
FULL_Y = {"bf16_e16", "multi_item", "wide_d"}   # the oracle over every token still takes seconds
SAMPLE = 1024                  # tokens whose y is checked on the other full-size cases
SAMPLE_OF = {"dense_soft_e128": 128}   # 128 experts per token: 16384 oracle rows
BLOCK = 64                     # row blocks of an expert segment whose first and last rows are checked


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


def _expert_of_rows(offsets, rows):
    return (np.searchsorted(offsets, rows, side="right") - 1).astype(np.int32)


def item_rows(offsets, block=BLOCK):
    """First and last row of every `block`-row block of every expert segment
    (a superset of the first and last rows of the GEMMs' work items for any
    row tile that is a multiple of `block`)."""
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for m0 in range(lo, hi, block):
            rows += [m0, min(m0 + block, hi) - 1]
    return np.unique(np.asarray(rows, np.int64))


def hot_cold_rows(counts, offsets, n=2):
    """Every row of the n busiest and the n least busy active experts."""
    act = np.nonzero(counts > 0)[0]
    order = act[np.argsort(counts[act], kind="stable")]
    pick = sorted(set(order[:n].tolist()) | set(order[-n:].tolist()))
    if not pick:
        return np.zeros(0, np.int64)
    return np.concatenate([np.arange(offsets[e], offsets[e + 1], dtype=np.int64) for e in pick])


def _check_tiled_copy(moe, s, wsh, cfg, dsp, x, name):
    """The fused bf16 forward's tiled copy of x_perm (MOE_WS_XPT): kept row r
    of expert e sits at padded row p = r - offsets[e] + P[e] (P: earlier
    experts' counts rounded up to 16), element (p, c) at ((p / 16) KT + c / 32)
    512 + (p % 16) 32 + c % 32; every kept row equals x[perm[r]] with zeros in
    columns d .. 32 KT - 1 (padding rows are undefined).  Byte copy: bit-exact."""
    d = cfg.d
    KT = (d + 31) // 32
    offs = dsp["offsets"].astype(np.int64)
    S = int(offs[-1])
    poff = np.concatenate([[0], np.cumsum((np.diff(offs) + 15) // 16 * 16)])
    rows = np.arange(S, dtype=np.int64)
    e = _expert_of_rows(dsp["offsets"], rows)
    p = rows - offs[e] + poff[e]
    nrow = int(poff[-1])
    off = moe.moe_workspace_offset(s, moe.MOE_WS_XPT)
    xpt = wsh[off:off + 2 * nrow * KT * 32].view(np.uint16).reshape(nrow // 16, KT, 16, 32)
    got = xpt[p // 16, :, p % 16, :].reshape(S, KT * 32)
    want = np.zeros((S, KT * 32), np.uint16)
    want[:, :d] = x.view(np.uint16)[dsp["perm"][:S]]
    assert np.array_equal(got, want), f"{name}: tiled x_perm rows"


def _check_case(moe, orc, name):
    import torch
    cfg = get(name)
    H.log(f"[parity] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff} {cfg.dtype}")
    inp = make_inputs(cfg)
    dv = H.dev_inputs(inp)
    s = H.make_shape(moe, cfg)
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    tol_y = H.TOL_Y[cfg.dtype]
    i32, f32 = torch.int32, torch.float32
    ws = moe.workspace(s)
    cap = orc.capacity(T, E, k, cfg.capacity_factor)
    assert moe.moe_capacity(s) == cap
    smax = moe.moe_max_rows(s)

    # ---------------- fused layer forward ----------------
    y = H.empty((T, d), f32)
    counts = H.empty(E, i32)
    routed = H.empty(E, i32)
    aux = H.empty(1, f32)
    idx = H.empty((T, k), i32)
    w = H.empty((T, k), f32)
    logits = H.empty((T, E), f32)
    moe.moe_layer_forward(s, dv["x"], dv["Wg"], dv["bg"], dv["W1"], dv["b1"], dv["W2"], dv["b2"],
                          y, counts, aux, ws, routed=routed, topk_idx=idx, topk_w=w, logits=logits)
    torch.cuda.synchronize()
    L = H.to_host(logits)
    Lref = orc.gate(inp["x"], inp["Wg"], inp["bg"])
    gerr = H.assert_close_norm(L, Lref, H.TOL_LOGITS, f"{name} gate logits")

    idx_ref, w_ref = orc.route(L, k, cfg.temperature)
    assert np.array_equal(H.to_host(idx), idx_ref), f"{name}: top-k indices differ"
    werr = float(np.abs(H.to_host(w) - w_ref).max())
    assert werr <= H.TOL_W, f"{name}: routing weights err {werr:.3e}"
    dsp = orc.dispatch(idx_ref, E, cap)
    assert np.array_equal(H.to_host(routed), dsp["routed"]), f"{name}: routed counts"
    assert np.array_equal(H.to_host(counts), dsp["counts"]), f"{name}: kept counts"
    wsh = H.to_host(ws)
    def ws_i32(which, n):
        off = moe.moe_workspace_offset(s, which)
        return wsh[off:off + 4 * n].view(np.int32)
    assert np.array_equal(ws_i32(moe.MOE_WS_OFFSETS, E + 1), dsp["offsets"]), f"{name}: offsets"
    assert np.array_equal(ws_i32(moe.MOE_WS_PERM, smax), dsp["perm"]), f"{name}: perm"
    assert np.array_equal(ws_i32(moe.MOE_WS_SLOT, T * k).reshape(T, k), dsp["slot"]), f"{name}: slot"
    aux_ref = orc.aux(dsp["counts"], T, k, cfg.aux_lambda)
    assert abs(float(H.to_host(aux)[0]) - aux_ref) <= H.TOL_AUX * abs(aux_ref) + 1e-12

    toks = np.arange(T, dtype=np.int32) if (name in SMALL or name in FULL_Y) else H.sample_tokens(T, SAMPLE_OF.get(name, SAMPLE))
    yref = orc.layer_tokens(toks, inp["x"], inp["W1"], inp["b1"], inp["W2"], inp["b2"], idx_ref,
                            dsp["slot"], w_ref)
    yh = H.to_host(y)
    yerr = H.assert_close_norm(yh[toks], yref, tol_y, f"{name} fused y")

    # ---------------- separate entry points ----------------
    idx2 = H.empty((T, k), i32)
    w2 = H.empty((T, k), f32)
    logits2 = H.empty((T, E), f32)
    moe.moe_route(s, dv["x"], dv["Wg"], dv["bg"], logits2, idx2, w2, ws)
    counts2 = H.empty(E, i32)
    routed2 = H.empty(E, i32)
    offsets2 = H.empty(E + 1, i32)
    perm2 = H.empty(smax, i32)
    slot2 = H.empty((T, k), i32)
    xperm = torch.zeros((smax, d), dtype=dv["x"].dtype, device="cuda")
    moe.moe_dispatch(s, dv["x"], idx2, routed2, counts2, offsets2, perm2, slot2, xperm, ws)
    out_perm = torch.zeros((smax, d), dtype=f32, device="cuda")
    moe.moe_grouped_ffn(s, xperm, offsets2, dv["W1"], dv["b1"], dv["W2"], dv["b2"], out_perm, ws)
    y2 = H.empty((T, d), f32)
    moe.moe_combine(s, out_perm, slot2, w2, y2)
    aux2 = H.empty(1, f32)
    moe.moe_aux_loss(s, counts2, aux2)
    torch.cuda.synchronize()
    assert np.array_equal(H.to_host(logits2), L), f"{name}: moe_route logits differ from fused"
    assert np.array_equal(H.to_host(idx2), idx_ref)
    for key, t in (("routed", routed2), ("counts", counts2), ("offsets", offsets2), ("perm", perm2),
                   ("slot", slot2)):
        assert np.array_equal(H.to_host(t), dsp[key]), f"{name}: moe_dispatch {key}"
    S = int(dsp["offsets"][-1])
    xp = H.to_host(xperm)
    assert np.array_equal(xp[:S], inp["x"].view(xp.dtype)[dsp["perm"][:S]]), f"{name}: x_perm rows"
    if cfg.dtype == "bf16":
        _check_tiled_copy(moe, s, wsh, cfg, dsp, inp["x"], name)
    # FFN rows: all of them for the small cases and FULL_Y; otherwise the
    # first and last row of every work item, the busiest and least busy
    # experts in full and the rows of the sampled tokens
    if name in SMALL or name in FULL_Y:
        rows = np.arange(S, dtype=np.int64)
    else:
        sl = dsp["slot"][toks]
        rows = np.unique(np.concatenate([sl[sl >= 0].astype(np.int64), item_rows(dsp["offsets"]),
                                         hot_cold_rows(dsp["counts"], dsp["offsets"])]))
    oref = orc.ffn_rows(dsp["perm"][rows], _expert_of_rows(dsp["offsets"], rows), inp["x"],
                        inp["W1"], inp["b1"], inp["W2"], inp["b2"])
    H.assert_close_norm(H.to_host(out_perm)[rows], oref, tol_y, f"{name} grouped FFN rows")
    # the fused forward's expert outputs (its first GEMM reads the tiled copy of x_perm)
    off_out = moe.moe_workspace_offset(s, moe.MOE_WS_OUT)
    out_fused = wsh[off_out:off_out + 4 * smax * d].view(np.float32).reshape(smax, d)
    assert np.array_equal(out_fused[:S], H.to_host(out_perm)[:S]), f"{name}: fused and unfused expert outputs"
    H.assert_close_norm(H.to_host(y2)[toks], yref, tol_y, f"{name} unfused y")
    # the fused entry point runs the same kernels as the separate ones
    assert np.array_equal(H.to_host(y2), yh), f"{name}: fused and unfused y differ"
    assert abs(float(H.to_host(aux2)[0]) - aux_ref) <= H.TOL_AUX * abs(aux_ref) + 1e-12
    if k > 32:
        # the selection by rank on logits the workspace keeps (no caller buffer)
        y3 = H.empty((T, d), f32)
        idx3 = H.empty((T, k), i32)
        w3 = H.empty((T, k), f32)
        moe.moe_layer_forward(s, dv["x"], dv["Wg"], dv["bg"], dv["W1"], dv["b1"], dv["W2"], dv["b2"],
                              y3, H.empty(E, i32), H.empty(1, f32), ws, topk_idx=idx3, topk_w=w3)
        idx4 = H.empty((T, k), i32)
        w4 = H.empty((T, k), f32)
        moe.moe_route_logits(s, logits, idx4, w4)
        torch.cuda.synchronize()
        assert np.array_equal(H.to_host(y3), yh), f"{name}: y with the logits in the workspace"
        for got, want, what in ((idx3, idx, "indices"), (w3, w, "weights"), (idx4, idx, "moe_route_logits indices"),
                                (w4, w, "moe_route_logits weights")):
            assert np.array_equal(H.to_host(got), H.to_host(want)), f"{name}: {what} (logits in the workspace)"
    H.log(f"[parity] {name}: ok  logits {gerr:.2e}  w {werr:.2e}  y {yerr:.2e}  S={S}/{T * k}  "
          f"rows checked {len(rows)}  tokens {len(toks)}")
    del dv, ws, xperm, out_perm
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", SMALL)
def test_parity_small(moe, orc, name):
    _check_case(moe, orc, name)


@pytest.mark.parametrize("name", FULL)
def test_parity_full_size(moe, orc, name):
    _check_case(moe, orc, name)
