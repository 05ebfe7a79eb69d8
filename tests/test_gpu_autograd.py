"""The autograd wrapper (mixture_experts_layer_26_amd.layer) against direct
calls of moe_layer_forward / moe_layer_backward on the same inputs: y, aux
and every gradient identical (the wrapper only marshals arguments; bf16
weights and x receive the round-to-nearest-even of the fp32 gradients)."""
import numpy as np
import pytest

import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


@pytest.mark.parametrize("dtype_name,T,d,E,k,d_ff,cf", [("bf16", 777, 136, 12, 3, 200, 1.1),
                                                        ("fp32", 300, 64, 8, 2, 128, 0.75),
                                                        ("bf16", 256, 64, 40, 36, 64, 0.0)])
def test_autograd_matches_direct_calls(moe, dtype_name, T, d, E, k, d_ff, cf):
    import torch
    from mixture_experts_layer_26_amd.layer import MoELayer
    H.log(f"[autograd] {dtype_name} T={T} d={d} E={E} k={k} d_ff={d_ff} cf={cf}")
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    g = torch.Generator().manual_seed(T + E)
    layer = MoELayer(d, d_ff, E, k=k, capacity_factor=cf, temperature=0.7, gate_bias=True, dtype=dt,
                     device="cuda", generator=g)
    with torch.no_grad():
        layer.bg.copy_(torch.randn(E, generator=g) * 0.3)
        layer.b1.copy_(torch.randn(E, d_ff, generator=g) * 0.1)
        layer.b2.copy_(torch.randn(E, d, generator=g) * 0.1)
    x = torch.randn(T, d, generator=g).to(dt).cuda().requires_grad_(True)
    dy = torch.randn(T, d, generator=g).cuda()
    y, aux = layer(x)
    assert not aux.requires_grad
    (y * dy).sum().backward()

    # the same through the entry points
    s = moe.shape(T, d, E, k, d_ff, cf, 0.7, 0.01, moe.MOE_BF16 if dtype_name == "bf16" else moe.MOE_F32)
    ws = moe.workspace(s)
    f32, i32 = torch.float32, torch.int32
    y2, counts, aux2 = H.empty((T, d), f32), H.empty(E, i32), H.empty(1, f32)
    idx, w = H.empty((T, k), i32), H.empty((T, k), f32)
    xd = x.detach().contiguous()
    moe.moe_layer_forward(s, xd, layer.Wg.detach(), layer.bg.detach(), layer.W1.detach(), layer.b1.detach(),
                          layer.W2.detach(), layer.b2.detach(), y2, counts, aux2, ws, topk_idx=idx, topk_w=w)
    R = moe.moe_max_rows(s)

    def region(which, dtype, shp):
        off = moe.moe_workspace_offset(s, which)
        n = int(np.prod(shp)) * 4
        return ws[off:off + n].view(dtype).view(*shp)

    xperm = region(moe.MOE_WS_XPERM, f32, (R, d)) if dtype_name == "fp32" else None
    gr = dict(dx=H.empty((T, d), f32), dWg=H.empty((d, E), f32), dbg=H.empty(E, f32),
              dW1=H.empty((E, d, d_ff), f32), db1=H.empty((E, d_ff), f32), dW2=H.empty((E, d_ff, d), f32),
              db2=H.empty((E, d), f32))
    moe.moe_layer_backward(s, xd, layer.Wg.detach(), layer.W1.detach(), layer.b1.detach(), layer.W2.detach(), dy,
                           idx, w, region(moe.MOE_WS_SLOT, i32, (T, k)), region(moe.MOE_WS_OFFSETS, i32, (E + 1,)),
                           xperm, region(moe.MOE_WS_OUT, f32, (R, d)), gr["dx"], gr["dWg"], gr["dbg"], gr["dW1"],
                           gr["db1"], gr["dW2"], gr["db2"], moe.backward_workspace(s))
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2) and torch.equal(aux, aux2)
    pairs = [(x.grad, gr["dx"].to(dt)), (layer.Wg.grad, gr["dWg"]), (layer.bg.grad, gr["dbg"]),
             (layer.W1.grad, gr["dW1"].to(dt)), (layer.b1.grad, gr["db1"]), (layer.W2.grad, gr["dW2"].to(dt)),
             (layer.b2.grad, gr["db2"])]
    for i, (got, want) in enumerate(pairs):
        assert got is not None and got.dtype == want.dtype, i
        assert torch.equal(got, want), f"gradient {i} differs from the direct call"
    # the gradients are not trivially zero
    assert float(layer.W1.grad.float().abs().max()) > 0 and float(layer.Wg.grad.abs().max()) > 0
