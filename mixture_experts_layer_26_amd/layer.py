"""torch.autograd / nn.Module wrapper of the C ABI: the MoE layer of the
"PithTrain" page, section 4.1 (linear gate, top-k, softmax over the selected
logits, Linear(d, d_ff) -> GELU -> Linear(d_ff, d) experts, weighted sum),
returning (y, aux) as the stable layer of the "PyTorchMoE" page, section 4.3.

Argument marshalling only: the forward is one moe_layer_forward call, the
backward one moe_layer_backward call on the routing the forward saved
(topk_idx, topk_w and the slot / offsets / expert-output regions of its
workspace).  The balance loss depends on integer counts only and carries no
gradient.  Gradients come out of the library in fp32 and are cast to each
input's dtype (bf16 weights and x get the round-to-nearest-even of them).
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import (MOE_BF16, MOE_F32, MOE_WS_OFFSETS, MOE_WS_OUT, MOE_WS_SLOT, MOE_WS_XPERM, backward_workspace,
               moe_layer_backward, moe_layer_forward, moe_max_rows, moe_workspace_offset, shape, workspace)


def _region(ws: torch.Tensor, s, which: int, dtype: torch.dtype, shp) -> torch.Tensor:
    off = moe_workspace_offset(s, which)
    n = int(math.prod(shp)) * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + n].view(dtype).view(*shp)


class MoEFunction(torch.autograd.Function):
    """y, aux = MoEFunction.apply(x, Wg, bg, W1, b1, W2, b2, k, capacity_factor, temperature, aux_lambda).

    x [T, d] and W1 [E, d, d_ff], W2 [E, d_ff, d] in one dtype (torch.bfloat16
    or torch.float32); Wg [d, E], bg [E] (or None), b1 [E, d_ff], b2 [E, d]
    in fp32.  y [T, d] fp32; aux [1] fp32 (no gradient)."""

    @staticmethod
    def forward(ctx, x, Wg, bg, W1, b1, W2, b2, k: int, capacity_factor: float, temperature: float,
                aux_lambda: float):
        if x.dtype not in (torch.bfloat16, torch.float32) or W1.dtype != x.dtype or W2.dtype != x.dtype:
            raise ValueError("x, W1 and W2 must share one dtype, torch.bfloat16 or torch.float32")
        if any(t is not None and t.dtype != torch.float32 for t in (Wg, bg, b1, b2)):
            raise ValueError("Wg, bg, b1 and b2 must be torch.float32")
        T, d = x.shape
        E, d_ff = Wg.shape[1], W1.shape[2]
        dt = MOE_F32 if x.dtype == torch.float32 else MOE_BF16
        s = shape(T, d, E, k, d_ff, capacity_factor, temperature, aux_lambda, dt)
        dev = x.device
        ws = workspace(s, dev)
        y = torch.empty((T, d), dtype=torch.float32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        aux = torch.empty(1, dtype=torch.float32, device=dev)
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        moe_layer_forward(s, x, Wg, bg, W1, b1, W2, b2, y, counts, aux, ws, topk_idx=idx, topk_w=w)
        ctx.s = s
        ctx.has_bg = bg is not None
        ctx.save_for_backward(x, Wg, W1, b1, W2, idx, w, ws)
        ctx.mark_non_differentiable(aux)
        return y, aux

    @staticmethod
    def backward(ctx, dy, _daux):
        x, Wg, W1, b1, W2, idx, w, ws = ctx.saved_tensors
        s = ctx.s
        T, d, E, k, d_ff = s.T, s.d, s.E, s.k, s.d_ff
        R = moe_max_rows(s)
        dev = x.device
        f32 = torch.float32
        slot = _region(ws, s, MOE_WS_SLOT, torch.int32, (T, k))
        offsets = _region(ws, s, MOE_WS_OFFSETS, torch.int32, (E + 1,))
        out = _region(ws, s, MOE_WS_OUT, f32, (R, d))
        # fp32 layers keep x_perm row-major in the workspace; bf16 layers keep
        # only its tile layout, and the backward copies the kept rows itself
        xperm = _region(ws, s, MOE_WS_XPERM, f32, (R, d)) if s.dtype == MOE_F32 else None
        dx = torch.empty((T, d), dtype=f32, device=dev)
        dWg = torch.empty((d, E), dtype=f32, device=dev)
        dbg = torch.empty(E, dtype=f32, device=dev)
        dW1 = torch.empty((E, d, d_ff), dtype=f32, device=dev)
        db1 = torch.empty((E, d_ff), dtype=f32, device=dev)
        dW2 = torch.empty((E, d_ff, d), dtype=f32, device=dev)
        db2 = torch.empty((E, d), dtype=f32, device=dev)
        moe_layer_backward(s, x, Wg, W1, b1, W2, dy.to(f32).contiguous(), idx, w, slot, offsets, xperm, out,
                           dx, dWg, dbg, dW1, db1, dW2, db2, backward_workspace(s, dev))
        return (dx.to(x.dtype), dWg, dbg if ctx.has_bg else None, dW1.to(W1.dtype), db1, dW2.to(W2.dtype), db2,
                None, None, None, None)


class MoELayer(torch.nn.Module):
    """The MoE layer as a module: forward(x) -> (y, aux).

    dtype torch.bfloat16 (x and the expert weights in bf16, the gate, the
    biases and the outputs in fp32) or torch.float32.  Parameters are
    random-initialised: Wg, W1, W2 ~ N(0, 1/fan_in), biases zero."""

    def __init__(self, d: int, d_ff: int, num_experts: int, k: int = 2, capacity_factor: float = 0.0,
                 temperature: float = 1.0, aux_lambda: float = 0.01, gate_bias: bool = False,
                 dtype: torch.dtype = torch.bfloat16, device: Optional[torch.device] = None,
                 generator: Optional[torch.Generator] = None):
        super().__init__()
        if dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("dtype must be torch.bfloat16 or torch.float32")
        self.k, self.capacity_factor, self.temperature, self.aux_lambda = k, capacity_factor, temperature, aux_lambda
        E = num_experts

        def normal(shp, fan_in, dt):
            t = torch.randn(shp, generator=generator, dtype=torch.float32) / math.sqrt(fan_in)
            return torch.nn.Parameter(t.to(dtype=dt, device=device))

        self.Wg = normal((d, E), d, torch.float32)
        self.bg = torch.nn.Parameter(torch.zeros(E, device=device)) if gate_bias else None
        self.W1 = normal((E, d, d_ff), d, dtype)
        self.b1 = torch.nn.Parameter(torch.zeros((E, d_ff), device=device))
        self.W2 = normal((E, d_ff, d), d_ff, dtype)
        self.b2 = torch.nn.Parameter(torch.zeros((E, d), device=device))

    def forward(self, x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        return MoEFunction.apply(x.contiguous(), self.Wg, self.bg, self.W1, self.b1, self.W2, self.b2, self.k,
                                 self.capacity_factor, self.temperature, self.aux_lambda)
