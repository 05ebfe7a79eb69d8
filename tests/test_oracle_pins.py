"""Pins of the CPU oracle against things other than itself: textbook
routines, closed forms, invariants, brute force on tiny inputs and a
hand-derived worked example.  CPU only."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import bruteforce as bf
from moe_inputs import f32_to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(s):
    return np.random.default_rng(s)


def _np_gelu(a):
    return 0.5 * a * (1.0 + np.vectorize(math.erf)(a / math.sqrt(2.0)))


def _as_f64(a):
    return bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


# ---------------------------------------------------------------- gate -----
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_gate_matches_numpy_matmul(orc, dtype):
    r = _rng(1)
    T, d, E = 37, 24, 11
    x = r.standard_normal((T, d)).astype(np.float32)
    if dtype == "bf16":
        x = f32_to_bf16_bits(x)
    Wg = r.standard_normal((d, E)).astype(np.float32)
    bg = r.standard_normal(E).astype(np.float32)
    ref = _as_f64(x) @ Wg.astype(np.float64) + bg.astype(np.float64)
    got = orc.gate(x, Wg, bg)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    ref0 = _as_f64(x) @ Wg.astype(np.float64)
    np.testing.assert_allclose(orc.gate(x, Wg, None), ref0, rtol=1e-13, atol=1e-13)


def test_gate_exact_on_integers(orc):
    r = _rng(2)
    x = r.integers(-3, 4, (9, 5)).astype(np.float32)
    Wg = r.integers(-3, 4, (5, 7)).astype(np.float32)
    assert np.array_equal(orc.gate(x, Wg), x.astype(np.int64) @ Wg.astype(np.int64))


# --------------------------------------------------------------- route -----
@pytest.mark.parametrize("seed,E,k", [(0, 8, 2), (1, 5, 1), (2, 6, 6), (3, 8, 8), (4, 16, 3)])
def test_route_selection_bruteforce(orc, seed, E, k):
    r = _rng(seed)
    T = 40
    # few distinct values so that ties are frequent, plus -0.0/+0.0 pairs
    L = r.integers(-2, 3, (T, E)).astype(np.float32)
    L[r.random((T, E)) < 0.2] = -0.0
    L[:5] = r.standard_normal((5, E)).astype(np.float32)
    idx, w = orc.route(L, k)
    for t in range(T):
        assert list(idx[t]) == bf.select([float(v) for v in L[t]], k)


def test_route_all_tied_picks_lowest(orc):
    L = np.full((3, 10), 0.25, np.float32)
    L[1] = -0.0
    L[2, ::2] = 0.0
    L[2, 1::2] = -0.0
    idx, w = orc.route(L, 4)
    assert (idx == np.arange(4)).all()
    np.testing.assert_allclose(w, 0.25, rtol=0, atol=1e-15)


def test_route_weight_closed_forms(orc):
    # k = 1 -> weight exactly 1
    L = _rng(5).standard_normal((7, 9)).astype(np.float32)
    _, w1 = orc.route(L, 1)
    assert (w1 == 1.0).all()
    # a logit gap of tau*ln 3 gives weights (3/4, 1/4), for two temperatures
    for tau in (1.0, 0.2):
        gap = np.float32(tau * math.log(3.0))
        L2 = np.array([[0.5, 0.5 - gap, -9.0]], np.float32)
        g = float(np.float32(0.5)) - float(np.float32(np.float32(0.5) - gap))
        idx, w = orc.route(L2, 2, tau)
        assert list(idx[0]) == [0, 1]
        expect = 1.0 / (1.0 + math.exp(-g / tau))
        assert abs(w[0, 0] - expect) < 1e-15 and abs(w[0, 0] - 0.75) < 1e-6
        assert abs(w[0, 1] - (1 - expect)) < 1e-15


def test_route_invariants(orc):
    L = _rng(6).standard_normal((200, 64)).astype(np.float32)
    for k, tau in ((2, 1.0), (8, 0.2)):
        idx, w = orc.route(L, k, tau)
        assert all(len(set(row)) == k for row in idx.tolist())
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
        assert (np.diff(w, axis=1) <= 0).all()
        sel = np.take_along_axis(L, idx, 1)
        assert (np.diff(sel, axis=1) <= 0).all()
        # every unselected logit is <= the smallest selected one
        mask = np.ones_like(L, bool)
        np.put_along_axis(mask, idx, False, 1)
        assert (np.where(mask, L, -np.inf).max(1) <= sel[:, -1]).all()


# ------------------------------------------------------------ capacity -----
@pytest.mark.parametrize("T,E,k,cf,cap", [
    (4096, 16, 2, 1.25, 640), (8192, 64, 2, 2.0, 512), (32768, 256, 2, 1.25, 320),
    (8192, 128, 8, 0.0, 8192), (256, 8, 2, 0.0, 256), (256, 8, 2, -1.0, 256),
    (200, 8, 2, 0.02, 1), (10, 1, 1, 5.0, 10), (100, 3, 1, 0.75, 25), (100, 3, 1, 0.5, 17),
    (5, 3, 2, 0.5, 2), (1000, 12, 3, 1.0, 250)])
def test_capacity_closed_forms(orc, T, E, k, cf, cap):
    assert orc.capacity(T, E, k, cf) == cap


# ------------------------------------------------------------ dispatch -----
@pytest.mark.parametrize("seed,T,E,k,cap", [(0, 30, 4, 2, 9), (1, 25, 5, 3, 4), (2, 40, 3, 1, 40),
                                            (3, 17, 6, 2, 1), (4, 1, 4, 2, 1), (5, 33, 8, 8, 20)])
def test_dispatch_bruteforce_and_invariants(orc, seed, T, E, k, cap):
    r = _rng(seed)
    L = r.standard_normal((T, E)).astype(np.float32)
    L[:, 0] += 1.0  # skew toward expert 0 so that drops happen
    idx, _ = orc.route(L, k)
    got = orc.dispatch(idx, E, cap)
    ref = bf.dispatch(idx.tolist(), E, cap)
    for key in ("routed", "counts", "offsets", "perm", "slot"):
        assert np.array_equal(np.asarray(got[key]), np.asarray(ref[key])), key
    counts, offsets, perm, slot = got["counts"], got["offsets"], got["perm"], got["slot"]
    S = int(offsets[-1])
    drops = int((slot < 0).sum())
    assert counts.sum() == T * k - drops and (counts <= cap).all()
    assert (got["routed"] >= counts).all() and got["routed"].sum() == T * k
    # bijection between kept slots and rows [0, S)
    rows = np.sort(slot[slot >= 0])
    assert np.array_equal(rows, np.arange(S))
    for t in range(T):
        for j in range(k):
            if slot[t, j] >= 0:
                assert perm[slot[t, j]] == t
                e = idx[t, j]
                assert offsets[e] <= slot[t, j] < offsets[e + 1]
            else:
                e = idx[t, j]
                seg = perm[offsets[e]:offsets[e + 1]]
                assert len(seg) == cap and (seg < t).all()
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()
    assert (perm[S:] == -1).all()


def test_dispatch_two_expert_closed_form(orc):
    T, c = 50, 13
    L = np.full((T, 6), -1.0, np.float32)
    L[:, 0] = 2.0
    L[:, 1] = 1.0
    idx, _ = orc.route(L, 2)
    got = orc.dispatch(idx, 6, c)
    assert int((got["slot"] < 0).sum()) == 2 * (T - c)
    assert np.array_equal(got["perm"][:c], np.arange(c))
    assert np.array_equal(got["perm"][c:2 * c], np.arange(c))
    assert (got["slot"][:c] >= 0).all() and (got["slot"][c:] < 0).all()


def test_dispatch_worked_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "dispatch_worked_example.json")))
    L = np.array(g["logits"], np.float32)
    L[4, 0] = -0.0
    assert orc.capacity(g["T"], g["E"], g["k"], g["capacity_factor"]) == g["cap"]
    idx, w = orc.route(L, g["k"], g["temperature"])
    assert idx.tolist() == g["idx"]
    np.testing.assert_allclose(w, np.array(g["w"]), rtol=0, atol=1e-15)
    got = orc.dispatch(idx, g["E"], g["cap"])
    for key in ("routed", "counts", "offsets", "perm", "slot"):
        assert np.asarray(got[key]).tolist() == g[key], key
    assert abs(orc.aux(got["counts"], g["T"], g["k"], g["aux_lambda"]) - g["aux"]) < 1e-18


# ---------------------------------------------------------------- GELU -----
def test_gelu_textbook_values(orc):
    # Phi(1) and Phi(-1) of the standard normal distribution
    assert abs(orc.gelu(1.0) - 0.8413447460685429) < 1e-15
    assert abs(orc.gelu(-1.0) + 0.15865525393145707) < 1e-15
    assert orc.gelu(0.0) == 0.0
    # Phi(2) = 0.9772498680518208
    assert abs(orc.gelu(2.0) - 2 * 0.9772498680518208) < 1e-15
    for u in (0.3, 1.7, 4.2, 11.0):
        assert abs((orc.gelu(u) - orc.gelu(-u)) - u) <= 4e-16 * max(1.0, u)
    assert abs(orc.gelu(40.0) - 40.0) < 1e-12 and abs(orc.gelu(-40.0)) < 1e-12


# ----------------------------------------------------------------- FFN -----
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_one_expert_dense_ffn_matches_numpy(orc, dtype):
    r = _rng(7)
    T, d, dff = 23, 12, 20
    x = r.standard_normal((T, d)).astype(np.float32)
    W1 = (r.standard_normal((1, d, dff)) / math.sqrt(d)).astype(np.float32)
    W2 = (r.standard_normal((1, dff, d)) / math.sqrt(dff)).astype(np.float32)
    b1 = r.standard_normal((1, dff)).astype(np.float32)
    b2 = r.standard_normal((1, d)).astype(np.float32)
    Wg = r.standard_normal((d, 1)).astype(np.float32)
    if dtype == "bf16":
        x, W1, W2 = f32_to_bf16_bits(x), f32_to_bf16_bits(W1), f32_to_bf16_bits(W2)
    out = orc.layer_forward(x, Wg, None, W1, b1, W2, b2, k=1, cf=0.0)
    ref = _np_gelu(_as_f64(x) @ _as_f64(W1)[0] + b1[0]) @ _as_f64(W2)[0] + b2[0]
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    assert (out["w"] == 1.0).all() and out["counts"].tolist() == [T]


def _identity_experts(E, d, dff, dtype):
    assert dff >= 2 * d
    W1 = np.zeros((E, d, dff), np.float32)
    W2 = np.zeros((E, dff, d), np.float32)
    I = np.eye(d, dtype=np.float32)
    W1[:, :, :d] = I
    W1[:, :, d:2 * d] = -I
    W2[:, :d, :] = I
    W2[:, d:2 * d, :] = -I
    if dtype == "bf16":
        W1, W2 = f32_to_bf16_bits(W1), f32_to_bf16_bits(W2)
    return W1, np.zeros((E, dff), np.float32), W2, np.zeros((E, d), np.float32)


@pytest.mark.parametrize("dtype,cf", [("fp32", 0.0), ("bf16", 0.0), ("bf16", 0.6)])
def test_identity_experts_reproduce_x(orc, dtype, cf):
    r = _rng(8)
    T, d, dff, E, k = 60, 8, 24, 5, 2
    x = r.standard_normal((T, d)).astype(np.float32)
    if dtype == "bf16":
        x = f32_to_bf16_bits(x)
    Wg = r.standard_normal((d, E)).astype(np.float32)
    W1, b1, W2, b2 = _identity_experts(E, d, dff, dtype)
    out = orc.layer_forward(x, Wg, None, W1, b1, W2, b2, k=k, cf=cf)
    kept_w = np.where(out["slot"] >= 0, out["w"], 0.0).sum(1)
    np.testing.assert_allclose(out["y"], kept_w[:, None] * _as_f64(x), rtol=1e-14, atol=1e-14)
    if cf == 0.0:
        np.testing.assert_allclose(out["y"], _as_f64(x), rtol=1e-14, atol=1e-14)
    else:
        assert (out["slot"] < 0).any()


def test_k_equals_e_is_dense_soft_moe(orc):
    r = _rng(9)
    T, d, dff, E, tau = 31, 10, 14, 4, 0.5
    x = r.standard_normal((T, d)).astype(np.float32)
    Wg = r.standard_normal((d, E)).astype(np.float32)
    W1 = r.standard_normal((E, d, dff)).astype(np.float32) / 3
    W2 = r.standard_normal((E, dff, d)).astype(np.float32) / 3
    b1 = r.standard_normal((E, dff)).astype(np.float32)
    b2 = r.standard_normal((E, d)).astype(np.float32)
    out = orc.layer_forward(x, Wg, None, W1, b1, W2, b2, k=E, cf=0.0, tau=tau)
    L = out["logits32"].astype(np.float64) / tau
    g = np.exp(L - L.max(1, keepdims=True))
    g /= g.sum(1, keepdims=True)
    ref = np.zeros((T, d))
    for e in range(E):
        fe = _np_gelu(x.astype(np.float64) @ W1[e] + b1[e]) @ W2[e].astype(np.float64) + b2[e]
        ref += g[:, e:e + 1] * fe
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def test_token_permutation_equivariance(orc):
    r = _rng(10)
    T, d, dff, E, k = 50, 16, 32, 6, 2
    x = f32_to_bf16_bits(r.standard_normal((T, d)).astype(np.float32))
    Wg = r.standard_normal((d, E)).astype(np.float32)
    W1 = f32_to_bf16_bits(r.standard_normal((E, d, dff)).astype(np.float32) / 4)
    W2 = f32_to_bf16_bits(r.standard_normal((E, dff, d)).astype(np.float32) / 4)
    b1 = r.standard_normal((E, dff)).astype(np.float32)
    b2 = r.standard_normal((E, d)).astype(np.float32)
    p = r.permutation(T)
    a = orc.layer_forward(x, Wg, None, W1, b1, W2, b2, k=k)
    b = orc.layer_forward(x[p], Wg, None, W1, b1, W2, b2, k=k)
    assert np.array_equal(a["y"][p], b["y"])
    assert np.array_equal(a["idx"][p], b["idx"])


# ----------------------------------------------------------------- aux -----
def test_aux_closed_form(orc):
    T, E, k = 40, 8, 2
    L = _rng(11).standard_normal((T, E)).astype(np.float32)
    L[:, 3] += 3
    idx, _ = orc.route(L, k)
    for cap in (T, 6):
        got = orc.dispatch(idx, E, cap)
        drops = int((got["slot"] < 0).sum())
        expect = 0.01 * (T * k - drops) / (T * k * E)
        assert abs(orc.aux(got["counts"], T, k, 0.01) - expect) <= 1e-17
    assert abs(orc.aux(orc.dispatch(idx, E, T)["counts"], T, k, 0.01) - 0.01 / E) < 1e-17


# ------------------------------------------------------ composed layer -----
def test_layer_forward_equals_its_parts(orc):
    from moe_inputs import get, make_inputs
    c = get("ragged_bf16").scaled(T=120)
    inp = make_inputs(c)
    out = orc.layer_forward(inp["x"], inp["Wg"], inp["bg"], inp["W1"], inp["b1"], inp["W2"],
                            inp["b2"], k=c.k, cf=c.capacity_factor, tau=c.temperature)
    L = orc.gate(inp["x"], inp["Wg"], inp["bg"])
    assert np.array_equal(L, out["logits"])
    idx, w = orc.route(L.astype(np.float32), c.k, c.temperature)
    cap = orc.capacity(c.T, c.E, c.k, c.capacity_factor)
    dsp = orc.dispatch(idx, c.E, cap)
    y = orc.layer_tokens(np.arange(c.T), inp["x"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                         idx, dsp["slot"], w)
    assert np.array_equal(idx, out["idx"]) and np.array_equal(w, out["w"])
    for key in ("routed", "counts", "offsets", "perm", "slot"):
        assert np.array_equal(dsp[key], out[key])
    assert np.array_equal(y, out["y"])
    assert (dsp["slot"] < 0).any(), "this case is meant to drop slots"


# ---- routing heat map and load telemetry ([EP] 3.2 step 1, 2.1; [PyTorchMoE] 3.3) ----

def _distinct_rows(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("seed,T,E,k", [(0, 40, 6, 3), (1, 25, 5, 5), (2, 30, 7, 1), (3, 60, 4, 2)])
def test_coactivation_bruteforce(orc, seed, T, E, k):
    idx = _distinct_rows(_rng(seed), T, E, k)
    H, routed = orc.coactivation(idx, E)
    Hb, rb = bf.coactivation(idx.tolist(), E)
    assert H.tolist() == Hb
    assert routed.tolist() == rb


def test_coactivation_invariants(orc):
    rng = _rng(7)
    T, E, k = 500, 16, 4
    idx = _distinct_rows(rng, T, E, k)
    H, routed = orc.coactivation(idx, E)
    assert H.sum() == T * k * (k - 1) // 2
    assert np.all(np.diag(H) == 0)
    assert routed.sum() == T * k
    # every token that chose e pairs it with its k - 1 other experts
    assert np.array_equal((H + H.T).sum(axis=1), routed * (k - 1))


def test_coactivation_order_closed_forms(orc):
    T, E = 33, 5
    H, routed = orc.coactivation(np.tile(np.array([[0, 1]], np.int32), (T, 1)), E)
    ref = np.zeros((E, E), np.int64)
    ref[0, 1] = T
    assert np.array_equal(H, ref)
    H2, _ = orc.coactivation(np.tile(np.array([[1, 0]], np.int32), (T, 1)), E)
    assert np.array_equal(H2, ref.T)
    assert routed.tolist() == [T, T, 0, 0, 0]
    # k = E: every token chose every expert, so H + H^T = T (J - I)
    idx = _distinct_rows(_rng(3), T, E, E)
    H3, r3 = orc.coactivation(idx, E)
    assert np.array_equal(H3 + H3.T, T * (np.ones((E, E), np.int64) - np.eye(E, dtype=np.int64)))
    assert np.all(r3 == T)
    # k = 1: no pairs
    H4, _ = orc.coactivation(idx[:, :1], E)
    assert not H4.any()


def test_load_stats_closed_forms(orc):
    import statistics
    E, T = 8, 1000
    s = orc.load_stats(np.full(E, 250, np.int64))
    assert s["mean"] == 250 and s["var"] == 0 and s["cv"] == 0
    one = np.zeros(E, np.int64)
    one[0] = T   # k = 1, every token on expert 0
    s = orc.load_stats(one)
    assert math.isclose(s["var"], T * T * (E - 1) / E ** 2, rel_tol=1e-15)
    assert math.isclose(s["cv"], math.sqrt(E - 1), rel_tol=1e-15)
    load = _rng(5).integers(0, 900, 64).astype(np.int64)
    s = orc.load_stats(load)
    assert math.isclose(s["var"], statistics.pvariance(load.tolist()), rel_tol=1e-12)
    assert math.isclose(s["cv"], statistics.pstdev(load.tolist()) / statistics.fmean(load.tolist()),
                        rel_tol=1e-12)


# ---- router variants ([PyTorchMoE] 2.3, 3.3 item 1, 4.3) ----

@pytest.mark.parametrize("seed,T,E,tau", [(0, 30, 5, 1.0), (1, 20, 16, 0.2), (2, 25, 3, 2.5)])
def test_top1_full_softmax_matches_library(orc, seed, T, E, tau):
    from scipy.special import softmax
    r = _rng(seed)
    L = r.integers(-4, 5, (T, E)).astype(np.float32)          # ties
    L[::3] = r.standard_normal((len(L[::3]), E)).astype(np.float32)
    idx, w = orc.route_top1_full(L, tau)
    for t in range(T):
        row = L[t].astype(np.float64)
        best = max(range(E), key=lambda e: (row[e], -e))       # largest, then lowest index
        assert idx[t, 0] == best
        assert math.isclose(w[t, 0], softmax(row / tau)[best], rel_tol=1e-12)


def test_top1_full_softmax_closed_forms(orc):
    E = 6
    L = np.zeros((3, E), np.float32)
    L[1, 4] = np.float32(math.log(3.0))      # tau = 1: weight 3 / (3 + E - 1)
    L[2] = -0.0
    L[2, 3] = 0.0                            # -0 == +0: index 0 wins
    idx, w = orc.route_top1_full(L, 1.0)
    assert idx[:, 0].tolist() == [0, 4, 0]
    assert math.isclose(w[0, 0], 1.0 / E, rel_tol=1e-15)
    assert math.isclose(w[1, 0], 3.0 / (E + 2), rel_tol=1e-7)   # log 3 rounded to fp32
    assert math.isclose(w[2, 0], 1.0 / E, rel_tol=1e-15)
    # top-1 of the full softmax picks what top-k with k = 1 picks
    L = _rng(9).standard_normal((200, 11)).astype(np.float32)
    idx1, _ = orc.route_top1_full(L, 0.5)
    idxk, wk = orc.route(L, 1, 0.5)
    assert np.array_equal(idx1, idxk) and np.all(wk == 1.0)


def test_noisy_logits_fp32_steps(orc):
    """Each fp32 step rounded once from its exact rational value."""
    from fractions import Fraction
    r = _rng(4)
    L = (r.standard_normal(300) * np.exp2(r.integers(-30, 30, 300))).astype(np.float32)
    n = r.standard_normal(300).astype(np.float32)
    out = orc.noisy_logits(L, n, 0.1)
    s32 = Fraction(float(np.float32(0.1)))
    for i in range(300):
        p = np.float32(float(s32 * Fraction(float(n[i]))))
        want = np.float32(float(Fraction(float(L[i])) + Fraction(float(p))))
        assert out[i] == want, i
    assert np.array_equal(orc.noisy_logits(L, n, 0.0), L)
    assert np.array_equal(orc.noisy_logits(L, np.zeros_like(n), 0.1), L)


def test_aux_variance_closed_forms(orc):
    import statistics
    E, T, lam = 8, 1000, 0.01
    one = np.zeros(E, np.int64)
    one[2] = T
    assert math.isclose(orc.aux_variance(one, lam), lam * T * T * (E - 1) / E ** 2, rel_tol=1e-15)
    assert orc.aux_variance(np.full(E, 7, np.int64), lam) == 0.0
    load = _rng(6).integers(0, 500, 33).astype(np.int64)
    assert math.isclose(orc.aux_variance(load, 0.5), 0.5 * statistics.pvariance(load.tolist()), rel_tol=1e-12)


# ---- sliding-window balance loss ([EP] 2.3) and the dense soft workload ----

def test_window_aux_worked_example(orc):
    """T = 10, k = 1, E = 2, W = 3; counts per batch (10,0), (0,10), (5,5),
    (10,0), (10,0), (10,0): the window means worked out by hand."""
    c = np.array([[10, 0], [0, 10], [5, 5], [10, 0], [10, 0], [10, 0]], np.int32)
    aux, pbar = orc.window_aux(c, T=10, k=1, W=3, lam=1.0)
    want = [[1.0, 0.0], [0.5, 0.5], [0.5, 0.5], [0.5, 0.5], [25 / 30, 5 / 30], [1.0, 0.0]]
    assert np.allclose(pbar, want, rtol=0, atol=1e-15)
    # the shares of every window sum to 1 here, so aux = lambda / E throughout
    assert np.allclose(aux, 0.5, rtol=0, atol=1e-15)


def test_window_aux_reduces_to_the_per_batch_loss(orc):
    r = _rng(12)
    E, T, k, lam = 16, 4096, 2, 0.01
    c = r.integers(0, 600, (30, E)).astype(np.int32)
    aux1, pbar1 = orc.window_aux(c, T, k, 1, lam)            # W = 1: each batch alone
    for b in range(30):
        assert math.isclose(aux1[b], orc.aux(c[b], T, k, lam), rel_tol=1e-13)
        assert np.allclose(pbar1[b], c[b] / (T * k), rtol=1e-15, atol=0)
    same = np.tile(c[:1], (250, 1))                          # constant batches: any W
    auxw, _ = orc.window_aux(same, T, k, 100, lam)
    assert np.allclose(auxw, orc.aux(c[0], T, k, lam), rtol=1e-13, atol=0)
    auxw, pbarw = orc.window_aux(c, T, k, 7, lam)            # a window mean of batch shares
    assert np.allclose(pbarw[20], c[14:21].mean(axis=0) / (T * k), rtol=1e-13, atol=0)


# ---- backward ([EP] 4.3: gradients for the active experts only) ----

def _fd_setup(seed=21, T=7, d=8, E=5, k=2, dff=12, cf=0.6, tau=0.7):
    """Small fp32 layer with biases, one drop-inducing capacity and expert 4
    made inactive by a very negative gate bias; no near-ties in the routing."""
    r = _rng(seed)
    while True:
        x = r.standard_normal((T, d)).astype(np.float32)
        Wg = (r.standard_normal((d, E)) / math.sqrt(d)).astype(np.float32)
        bg = np.array([0.3, -0.2, 0.1, 0.0, -50.0], np.float32)[:E]
        L = x.astype(np.float64) @ Wg.astype(np.float64) + bg
        srt = np.sort(L, axis=1)[:, ::-1]
        if np.min(srt[:, k - 1] - srt[:, k]) > 0.05:
            break
    W1 = (r.standard_normal((E, d, dff)) / math.sqrt(d)).astype(np.float32)
    b1 = (0.1 * r.standard_normal((E, dff))).astype(np.float32)
    W2 = (r.standard_normal((E, dff, d)) / math.sqrt(dff)).astype(np.float32)
    b2 = (0.1 * r.standard_normal((E, d))).astype(np.float32)
    dy = r.standard_normal((T, d)).astype(np.float32)
    return dict(x=x, Wg=Wg, bg=bg, W1=W1, b1=b1, W2=W2, b2=b2, dy=dy, k=k, cf=cf, tau=tau)


def _fd_loss(orc, p, idx, slot):
    """sum(dy * y) with the routing decisions fixed and w from fp64 logits."""
    L = orc.gate(p["x"], p["Wg"], p["bg"])
    sel = np.take_along_axis(L, idx, 1) / p["tau"]
    sel -= sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    w /= w.sum(axis=1, keepdims=True)
    tt, jj = np.nonzero(slot >= 0)
    o = orc.ffn_rows(tt.astype(np.int32), idx[tt, jj], p["x"], p["W1"], p["b1"], p["W2"], p["b2"])
    y = np.zeros(p["x"].shape, np.float64)
    np.add.at(y, tt, w[tt, jj][:, None] * o)
    return float((p["dy"].astype(np.float64) * y).sum())


def test_layer_backward_matches_finite_differences(orc):
    p = _fd_setup()
    L32 = orc.gate(p["x"], p["Wg"], p["bg"]).astype(np.float32)
    g = orc.layer_backward(p["x"], p["Wg"], p["W1"], p["b1"], p["W2"], p["b2"], L32, p["k"], p["cf"], p["tau"],
                           p["dy"])
    assert (g["slot"] < 0).any(), "the capacity should drop a slot"
    # the gate bias gradient is the column sum of dl (the bias adds into every logit)
    g["dbg_check"] = g["dl"].sum(axis=0)
    assert np.allclose(g["dbg"], g["dbg_check"], rtol=1e-12, atol=1e-15)
    r = _rng(5)
    names = {"x": "dx", "Wg": "dWg", "bg": "dbg", "W1": "dW1", "b1": "db1", "W2": "dW2", "b2": "db2"}
    for name, gname in names.items():
        arr = p[name]
        for _ in range(6):
            i = tuple(int(r.integers(0, s)) for s in arr.shape)
            if name in ("W1", "b1", "W2", "b2") and i[0] == 4:
                i = (int(r.integers(0, 4)),) + i[1:]
            v = arr[i]
            hi, lo = np.float32(v + np.float32(1e-3)), np.float32(v - np.float32(1e-3))
            arr[i] = hi
            f_hi = _fd_loss(orc, p, g["idx"], g["slot"])
            arr[i] = lo
            f_lo = _fd_loss(orc, p, g["idx"], g["slot"])
            arr[i] = v
            fd = (f_hi - f_lo) / (float(hi) - float(lo))
            assert abs(fd - g[gname][i]) <= 2e-6 * max(1.0, abs(fd)), (name, i, fd, g[gname][i])


def test_backward_inactive_expert_and_dropped_slots(orc):
    p = _fd_setup()
    L32 = orc.gate(p["x"], p["Wg"], p["bg"]).astype(np.float32)
    g = orc.layer_backward(p["x"], p["Wg"], p["W1"], p["b1"], p["W2"], p["b2"], L32, p["k"], p["cf"], p["tau"],
                           p["dy"])
    assert not (g["idx"] == 4).any()
    for name in ("dW1", "db1", "dW2", "db2"):
        assert not g[name][4].any(), name          # expert-grained: no gradient for an idle expert
    assert np.all(g["dw"][g["slot"] < 0] == 0.0)   # a dropped slot's output does not depend on its weight
    # softmax over the selected logits: its gradient sums to zero over each token's choices
    assert np.allclose(g["dl"].sum(axis=1), 0.0, atol=1e-13)


def test_gelu_derivative_closed_forms(orc):
    # GELU'(0) = 1/2; GELU'(u) + GELU'(-u) = 1 (Phi(u) + Phi(-u) = 1, the u phi terms cancel)
    d, dff = 1, 1
    x = np.array([[0.0], [1.3], [-1.3]], np.float32)
    W1 = np.ones((1, d, dff), np.float32)
    W2 = np.ones((1, dff, d), np.float32)
    b = np.zeros((1, 1), np.float32)
    dy = np.ones((3, 1), np.float32)
    _, dxp, _, _, _, _ = orc.ffn_backward_rows(np.arange(3, dtype=np.int32), np.zeros(3, np.int32),
                                               np.ones(3), x, W1, b, W2, b, dy, 1)
    assert math.isclose(dxp[0, 0], 0.5, rel_tol=1e-15)
    assert math.isclose(dxp[1, 0] + dxp[2, 0], 1.0, rel_tol=1e-14)
    # against the normal CDF and density from the statistics module
    from statistics import NormalDist
    nd = NormalDist()
    u = float(x[1, 0])
    assert math.isclose(dxp[1, 0], nd.cdf(u) + u * nd.pdf(u), rel_tol=1e-12)
