"""ctypes front end of the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke entry point and the
benchmark's cpu_baseline leg are the only users.  The product path (the HIP
library and its binding) never imports this package.

All functions take and return numpy arrays.  bf16 tensors are uint16 bit
patterns, fp32 tensors float32.  Results are float64 unless they are indices.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
SRC_PATH = os.path.join(_HERE, "moe_oracle.c")

_lib = None

_P = C.c_void_p
_I64 = C.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, -O2, OpenMP)."""
    from .build import build_oracle
    return build_oracle(force=force)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        L.oracle_threads.restype = C.c_int
        L.oracle_gelu.restype = C.c_double
        L.oracle_gelu.argtypes = [C.c_double]
        L.oracle_gate.argtypes = [_I64, _I64, _I64, C.c_int, _P, _P, _P, _P]
        L.oracle_route.argtypes = [_I64, _I64, _I64, C.c_double, _P, _P, _P]
        L.oracle_capacity.restype = _I64
        L.oracle_capacity.argtypes = [_I64, _I64, _I64, C.c_float]
        L.oracle_dispatch.argtypes = [_I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P]
        L.oracle_ffn_rows.argtypes = [_I64, _P, _P, _I64, _I64, C.c_int, _P, _P, _P, _P, _P, _P]
        L.oracle_layer_tokens.argtypes = [_I64, _P, _I64, _I64, _I64, C.c_int, _P, _P, _P,
                                          _P, _P, _P, _P, _P, _P]
        L.oracle_aux.restype = C.c_double
        L.oracle_aux.argtypes = [_I64, _I64, _I64, _P, C.c_double]
        L.oracle_coactivation.argtypes = [_I64, _I64, _I64, _P, _P, _P]
        L.oracle_noisy_logits.argtypes = [_I64, _P, _P, C.c_float, _P]
        L.oracle_route_top1_full.argtypes = [_I64, _I64, C.c_double, _P, _P, _P]
        L.oracle_window_aux.argtypes = [_I64] * 5 + [_P, C.c_double, _P, _P]
        L.oracle_ffn_backward_rows.argtypes = [_I64, _P, _P, _P, _I64, _I64, C.c_int] + [_P] * 12
        L.oracle_route_backward.argtypes = [_I64, _I64, _I64, _I64, C.c_double, C.c_int] + [_P] * 9
        L.oracle_aux_variance.restype = C.c_double
        L.oracle_aux_variance.argtypes = [_I64, _P, C.c_double]
        L.oracle_load_stats.argtypes = [_I64, _P, _P, _P, _P]
        L.oracle_layer_forward.argtypes = ([_I64] * 5 + [C.c_int, C.c_float, C.c_double, C.c_double]
                                           + [_P] * 18)
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError(f"oracle inputs are float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a, dt=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def threads() -> int:
    return lib().oracle_threads()


def gelu(u: float) -> float:
    return lib().oracle_gelu(float(u))


def gate(x, Wg, bg=None) -> np.ndarray:
    x = _c(x)
    Wg = _c(Wg, np.float32)
    bg = _c(bg, np.float32)
    T, d = x.shape
    E = Wg.shape[1]
    L = np.empty((T, E), np.float64)
    lib().oracle_gate(T, d, E, _dtype_code(x), _p(x), _p(Wg), _p(bg), _p(L))
    return L


def route(logits32, k: int, tau: float = 1.0):
    L = _c(logits32, np.float32)
    T, E = L.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().oracle_route(T, E, k, float(tau), _p(L), _p(idx), _p(w))
    return idx, w


def capacity(T: int, E: int, k: int, cf: float) -> int:
    return int(lib().oracle_capacity(T, E, k, float(np.float32(cf))))


def dispatch(idx, E: int, cap: int):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    smax = min(T * k, E * cap)
    routed = np.empty(E, np.int32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(smax, 1), np.int32)[:smax]
    slot = np.empty((T, k), np.int32)
    lib().oracle_dispatch(T, E, k, cap, _p(idx), _p(routed), _p(counts), _p(offsets),
                          _p(perm), _p(slot))
    return dict(routed=routed, counts=counts, offsets=offsets, perm=perm, slot=slot)


def ffn_rows(tok, exp_id, x, W1, b1, W2, b2) -> np.ndarray:
    tok = _c(tok, np.int32)
    exp_id = _c(exp_id, np.int32)
    x, W1, W2 = _c(x), _c(W1), _c(W2)
    b1, b2 = _c(b1, np.float32), _c(b2, np.float32)
    d = x.shape[1]
    dff = W1.shape[2]
    out = np.empty((len(tok), d), np.float64)
    lib().oracle_ffn_rows(len(tok), _p(tok), _p(exp_id), d, dff, _dtype_code(x), _p(x),
                          _p(W1), _p(b1), _p(W2), _p(b2), _p(out))
    return out


def layer_tokens(toks, x, W1, b1, W2, b2, idx, slot, w) -> np.ndarray:
    toks = _c(toks, np.int32)
    x, W1, W2 = _c(x), _c(W1), _c(W2)
    b1, b2 = _c(b1, np.float32), _c(b2, np.float32)
    idx, slot, w = _c(idx, np.int32), _c(slot, np.int32), _c(w, np.float64)
    d = x.shape[1]
    dff = W1.shape[2]
    k = idx.shape[1]
    y = np.empty((len(toks), d), np.float64)
    lib().oracle_layer_tokens(len(toks), _p(toks), d, dff, k, _dtype_code(x), _p(x), _p(W1),
                              _p(b1), _p(W2), _p(b2), _p(idx), _p(slot), _p(w), _p(y))
    return y


def aux(counts, T: int, k: int, lam: float) -> float:
    counts = _c(counts, np.int32)
    return float(lib().oracle_aux(len(counts), T, k, _p(counts), float(lam)))


def coactivation(idx, E: int):
    """Ordered co-selection counts H [E, E] int64 (H[i, j]: tokens that list
    expert i before expert j) and per-expert loads routed [E] int64."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    H = np.empty((E, E), np.int64)
    routed = np.empty(E, np.int64)
    lib().oracle_coactivation(T, E, k, _p(idx), _p(H), _p(routed))
    return H, routed


def load_stats(load) -> dict:
    """mean, population variance and CV of per-expert loads (float64)."""
    load = _c(load, np.int64)
    m, v, c = C.c_double(), C.c_double(), C.c_double()
    lib().oracle_load_stats(len(load), _p(load), C.byref(m), C.byref(v), C.byref(c))
    return dict(mean=m.value, var=v.value, cv=c.value)


def noisy_logits(L, noise, scale: float) -> np.ndarray:
    """fp32(L + fp32(scale * noise)), scale taken as float32 (the stable
    layer's exploration noise, in the page's fp32 arithmetic)."""
    L, noise = _c(L, np.float32), _c(noise, np.float32)
    out = np.empty(L.shape, np.float32)
    lib().oracle_noisy_logits(L.size, _p(L), _p(noise), float(np.float32(scale)), _p(out))
    return out


def route_top1_full(logits32, tau: float = 1.0):
    """Top-1 over all E with the full-softmax probability as weight:
    (idx [T,1] int32, w [T,1] float64)."""
    L = _c(logits32, np.float32)
    T, E = L.shape
    idx = np.empty((T, 1), np.int32)
    w = np.empty((T, 1), np.float64)
    lib().oracle_route_top1_full(T, E, float(tau), _p(L), _p(idx), _p(w))
    return idx, w


def window_aux(counts_seq, T: int, k: int, W: int, lam: float):
    """Sliding-window balance loss after each of n batches: (aux [n], pbar
    [n, E]) in float64, from the per-batch counts [n, E]."""
    c = _c(counts_seq, np.int32)
    n, E = c.shape
    aux = np.empty(n, np.float64)
    pbar = np.empty((n, E), np.float64)
    lib().oracle_window_aux(n, E, T, k, W, _p(c), float(lam), _p(aux), _p(pbar))
    return aux, pbar


def ffn_backward_rows(tok, exp_id, wt, x, W1, b1, W2, b2, dy, E: int):
    """Backward of the expert FFN over listed kept rows (token, expert,
    routing weight): (dw [n], dxp [n,d], dW1, db1, dW2, db2), float64, the
    weight gradients summed over the listed rows only."""
    tok, exp_id = _c(tok, np.int32), _c(exp_id, np.int32)
    wt = _c(wt, np.float64)
    x, W1, W2 = _c(x), _c(W1), _c(W2)
    b1, b2, dy = _c(b1, np.float32), _c(b2, np.float32), _c(dy, np.float32)
    d, dff = x.shape[1], W1.shape[2]
    n = len(tok)
    dw = np.zeros(n, np.float64)
    dxp = np.zeros((n, d), np.float64)
    dW1 = np.zeros((E, d, dff), np.float64)
    db1 = np.zeros((E, dff), np.float64)
    dW2 = np.zeros((E, dff, d), np.float64)
    db2 = np.zeros((E, d), np.float64)
    lib().oracle_ffn_backward_rows(n, _p(tok), _p(exp_id), _p(wt), d, dff, _dtype_code(x), _p(x), _p(W1),
                                   _p(b1), _p(W2), _p(b2), _p(dy), _p(dw), _p(dxp), _p(dW1), _p(db1),
                                   _p(dW2), _p(db2))
    return dw, dxp, dW1, db1, dW2, db2


def route_backward(x, Wg, idx, w, dw, tau: float):
    """Gate backward from the routing-weight gradients dw [T,k]: (dl [T,E],
    dWg [d,E], dbg [E], dxg [T,d]), float64."""
    x, Wg = _c(x), _c(Wg, np.float32)
    idx, w, dw = _c(idx, np.int32), _c(w, np.float64), _c(dw, np.float64)
    T, d = x.shape
    E = Wg.shape[1]
    k = idx.shape[1]
    dl = np.empty((T, E), np.float64)
    dWg = np.empty((d, E), np.float64)
    dbg = np.empty(E, np.float64)
    dxg = np.empty((T, d), np.float64)
    lib().oracle_route_backward(T, d, E, k, float(tau), _dtype_code(x), _p(x), _p(Wg), _p(idx), _p(w), _p(dw),
                                _p(dl), _p(dWg), _p(dbg), _p(dxg))
    return dl, dWg, dbg, dxg


def layer_backward(x, Wg, W1, b1, W2, b2, logits32, k: int, cf: float, tau: float, dy):
    """Gradients of sum(dy * y) for the layer routed on the fp32 logits
    `logits32`: the selection, capacity and drops are fixed by them; the
    routing weights, expert FFNs and the gate are differentiated.  Returns a
    dict of float64 arrays: dx, dWg, dbg, dW1, db1, dW2, db2, plus dw, dl."""
    T, d = np.asarray(x).shape
    E = np.asarray(Wg).shape[1]
    idx, w = route(logits32, k, tau)
    dsp = dispatch(idx, E, capacity(T, E, k, cf))
    slot = dsp["slot"]
    tt, jj = np.nonzero(slot >= 0)
    dw = np.zeros((T, k), np.float64)
    dwr, dxp, dW1, db1, dW2, db2 = ffn_backward_rows(tt.astype(np.int32), idx[tt, jj], w[tt, jj], x, W1, b1, W2,
                                                     b2, dy, E)
    dw[tt, jj] = dwr
    dx = np.zeros((T, d), np.float64)
    np.add.at(dx, tt, dxp)
    dl, dWg, dbg, dxg = route_backward(x, Wg, idx, w, dw, tau)
    return dict(dx=dx + dxg, dWg=dWg, dbg=dbg, dW1=dW1, db1=db1, dW2=dW2, db2=db2, dw=dw, dl=dl,
                idx=idx, slot=slot)


def aux_variance(load, lam: float) -> float:
    load = _c(load, np.int64)
    return float(lib().oracle_aux_variance(len(load), _p(load), float(lam)))


def layer_forward(x, Wg, bg, W1, b1, W2, b2, k: int, cf: float = 0.0, tau: float = 1.0,
                  lam: float = 0.01) -> dict:
    """Whole layer in oracle-only mode (routing on the oracle's own logits
    rounded to float32)."""
    x = _c(x)
    Wg, bg = _c(Wg, np.float32), _c(bg, np.float32)
    W1, W2 = _c(W1), _c(W2)
    b1, b2 = _c(b1, np.float32), _c(b2, np.float32)
    T, d = x.shape
    E = Wg.shape[1]
    dff = W1.shape[2]
    cap = capacity(T, E, k, cf)
    smax = min(T * k, E * cap)
    out = dict(
        logits=np.empty((T, E), np.float64), logits32=np.empty((T, E), np.float32),
        idx=np.empty((T, k), np.int32), w=np.empty((T, k), np.float64),
        routed=np.empty(E, np.int32), counts=np.empty(E, np.int32),
        offsets=np.empty(E + 1, np.int32), perm=np.empty(max(smax, 1), np.int32),
        slot=np.empty((T, k), np.int32), y=np.empty((T, d), np.float64),
        aux=np.empty(1, np.float64))
    lib().oracle_layer_forward(
        T, d, E, k, dff, _dtype_code(x), float(np.float32(cf)), float(tau), float(lam),
        _p(x), _p(Wg), _p(bg), _p(W1), _p(b1), _p(W2), _p(b2),
        _p(out["logits"]), _p(out["logits32"]), _p(out["idx"]), _p(out["w"]),
        _p(out["routed"]), _p(out["counts"]), _p(out["offsets"]), _p(out["perm"]),
        _p(out["slot"]), _p(out["y"]), _p(out["aux"]))
    out["perm"] = out["perm"][:smax]
    out["aux"] = float(out["aux"][0])
    out["cap"] = cap
    return out
