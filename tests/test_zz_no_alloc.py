"""moe_dispatch_noalloc (the dispatch with its per-block histogram in a
static device array instead of a workspace) against moe_dispatch on the same
inputs, through the C ABI: two calls in a row, the second on a smaller
batch, each compared bit for bit -- routed, counts, offsets, perm, slot and
the x_perm rows -- and against the oracle's dispatch of the same top-k
lists.  The first case's histogram leaves larger contents in the shared
array than the second case writes, so a stale entry would show."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_harness as H
from moe_inputs import get
from moe_inputs.gen import make_gate, make_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


def _dispatch_both(moe, orc, name):
    import torch
    cfg = get(name)
    H.log(f"[no-alloc] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k}")
    wg, bg = make_gate(cfg)
    inp = dict(x=make_x(cfg), Wg=wg, bg=bg)   # the dispatch needs no expert weights
    dv = H.dev_inputs(inp)
    s = H.make_shape(moe, cfg)
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    R = moe.moe_max_rows(s)
    i32 = torch.int32
    ws = moe.workspace(s)
    idx, w, logits = H.empty((T, k), i32), H.empty((T, k), torch.float32), H.empty((T, E), torch.float32)
    moe.moe_route(s, dv["x"], dv["Wg"], dv["bg"], logits, idx, w, ws)
    xdt = dv["x"].dtype
    outs = []
    for noalloc in (False, True):
        o = dict(routed=H.empty(E, i32), counts=H.empty(E, i32), offsets=H.empty(E + 1, i32),
                 perm=H.empty(R, i32), slot=H.empty((T, k), i32),
                 x_perm=torch.zeros((R, d), dtype=xdt, device="cuda"))
        if noalloc:
            moe.moe_dispatch_noalloc(s, dv["x"], idx, o["routed"], o["counts"], o["offsets"], o["perm"],
                                     o["slot"], o["x_perm"])
        else:
            moe.moe_dispatch(s, dv["x"], idx, o["routed"], o["counts"], o["offsets"], o["perm"], o["slot"],
                             o["x_perm"], ws)
        torch.cuda.synchronize()
        outs.append({n: H.to_host(v) for n, v in o.items()})
    ref, got = outs
    for n in ref:
        assert np.array_equal(got[n], ref[n]), f"{name}: moe_dispatch_noalloc {n} differs from moe_dispatch"
    # the integer outputs against the oracle's dispatch of the same top-k lists
    cap = orc.capacity(T, E, k, cfg.capacity_factor)
    dsp = orc.dispatch(H.to_host(idx), E, cap)
    for n in ("routed", "counts", "offsets", "perm", "slot"):
        assert np.array_equal(got[n], dsp[n]), f"{name}: {n} differs from the oracle"
    S = int(dsp["offsets"][-1])
    assert np.array_equal(got["x_perm"][:S], inp["x"].view(got["x_perm"].dtype)[dsp["perm"][:S]])
    H.log(f"[no-alloc] {name}: ok, S={S}")


def test_dispatch_noalloc_matches_dispatch_twice(moe, orc):
    # a large batch first (64 experts, 8 token blocks), then a smaller one
    # (12 experts, ragged blocks): the second call reuses the same array
    _dispatch_both(moe, orc, "skewed_e64")
    _dispatch_both(moe, orc, "ragged_bf16")


def test_dispatch_noalloc_rejects_oversized(moe):
    import torch
    s = moe.shape(1 << 20, 64, 1024, 2, 64, 1.0)
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoEError, match="static scratch"):
        moe.moe_dispatch_noalloc(s, t, t, None, t, t, t, t, t)
