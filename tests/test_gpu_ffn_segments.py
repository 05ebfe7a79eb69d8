"""The grouped expert FFN on chosen row segments (moe_grouped_ffn with given
offsets and x_perm): expert row counts at every boundary the tile split uses
(whole 256-row blocks, remainders of 1..128 rows on 128-row tiles, remainders
above 128 on 256-row tiles) and empty experts, every row compared with the
oracle's FFN of that row.  With a wide d_ff the first GEMM has enough items for
the split launch (tails on 128-row tiles); with a wide d the second GEMM runs
on the 256 x 256 pipelined tiles, and d_ff = 200 gives it an odd K-step count
(one all-zero step per item)."""
import numpy as np
import pytest

import gpu_harness as H
from moe_inputs import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 127, 128, 129, 255, 256, 257, 384, 385, 511, 512, 0, 640, 100, 200]


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import mixture_experts_layer_26_amd as m
    return m


# >= 128 items of 256 columns: the split launch (GEMM1, d_ff wide) or the pipelined one (GEMM2, d wide)
@pytest.mark.parametrize("d,d_ff", [(256, 2048), (200, 1992), (2048, 512), (1992, 200)])
def test_segments_at_tile_boundaries(moe, orc, d, d_ff):
    import torch
    E = len(SIZES)
    S = int(sum(SIZES))
    H.log(f"[segments] E={E} S={S} d={d} d_ff={d_ff} sizes={SIZES}")
    r = np.random.default_rng(d + d_ff)
    x = f32_to_bf16_bits(r.standard_normal((S, d)).astype(np.float32))
    W1 = f32_to_bf16_bits((r.standard_normal((E, d, d_ff)) / np.sqrt(d)).astype(np.float32))
    W2 = f32_to_bf16_bits((r.standard_normal((E, d_ff, d)) / np.sqrt(d_ff)).astype(np.float32))
    b1 = (0.1 * r.standard_normal((E, d_ff))).astype(np.float32)
    b2 = (0.1 * r.standard_normal((E, d))).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(SIZES)]).astype(np.int32)
    # one choice per token, no capacity limit: max_rows = T = S
    s = moe.shape(S, d, E, 1, d_ff, 0.0, 1.0, 0.01, moe.MOE_BF16)
    assert moe.moe_max_rows(s) == S
    ws = moe.workspace(s)
    out = torch.zeros((S, d), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(s, H.to_dev(x), H.to_dev(offsets), H.to_dev(W1), H.to_dev(b1), H.to_dev(W2),
                        H.to_dev(b2), out, ws)
    torch.cuda.synchronize()
    rows = np.arange(S, dtype=np.int32)
    exp_id = (np.searchsorted(offsets, rows, side="right") - 1).astype(np.int32)
    ref = orc.ffn_rows(rows, exp_id, x, W1, b1, W2, b2)
    got = H.to_host(out)
    # per expert, so that a wrong tail or block names its segment
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            H.assert_close_norm(got[lo:hi], ref[lo:hi], H.TOL_Y["bf16"], f"expert {e} ({hi - lo} rows)")
