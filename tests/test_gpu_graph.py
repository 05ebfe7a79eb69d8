"""moe_layer_forward inside a captured HIP graph: the call allocates nothing,
synchronises nothing and records no memset, so a serving loop can capture it
once and replay it.  Each replay (with eager work on the same buffers in
between) must reproduce the eager call bit for bit."""
import numpy as np
import pytest

import gpu_harness as H
from moe_inputs import get, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


# bf16_e16: both GEMMs on the 256 x 256 tiles with the experts' tails on 128-row tiles
@pytest.mark.parametrize("name", ["medium_bf16", "ragged_fp32", "soft_k64_e64", "bf16_e16"])
def test_forward_graph_replays_match_eager(moe, name):
    import torch
    cfg = get(name)
    H.log(f"[graph] {name}: T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} d_ff={cfg.d_ff} {cfg.dtype}")
    inp = make_inputs(cfg)
    dv = H.dev_inputs(inp)
    s = H.make_shape(moe, cfg)
    T, E, d, k = cfg.T, cfg.E, cfg.d, cfg.k
    f32, i32 = torch.float32, torch.int32
    ws = moe.workspace(s)
    out = dict(y=H.empty((T, d), f32), counts=H.empty(E, i32), aux=H.empty(1, f32), idx=H.empty((T, k), i32),
               w=H.empty((T, k), f32))

    def forward(stream=None):
        moe.moe_layer_forward(s, dv["x"], dv["Wg"], dv["bg"], dv["W1"], dv["b1"], dv["W2"], dv["b2"], out["y"],
                              out["counts"], out["aux"], ws, topk_idx=out["idx"], topk_w=out["w"], stream=stream)

    forward()
    torch.cuda.synchronize()
    ref = {n: H.to_host(t).copy() for n, t in out.items()}

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            forward(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        for t in out.values():
            t.fill_(-1)          # eager work on the outputs between replays
        ws.fill_(0xA5)           # and on the workspace
        g.replay()
        torch.cuda.synchronize()
        for n, t in out.items():
            assert np.array_equal(H.to_host(t), ref[n]), f"{name}: replay {r} differs in {n}"
    del g
