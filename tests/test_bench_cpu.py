"""bench.py's host-side logic on the CPU: the refusal of more than one GPU,
the kernel-name -> stage map its counter records rely on (names as
rocprofv3 prints them for the current kernels: the forward's GEMMs map to
their stage, the backward's instantiations of the same kernels to none),
and the algorithmic bytes of the headline's first GEMM from its definition
(the weights of every active expert once, the kept rows in, h out, b1)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "exactly one GPU" in line["error"]


TILE = "moe::(anonymous namespace)::TileCfg<256, 256, 2, 4, 32>"
NAMES = {
    # forward: GEMM1 (tiled or row-major x_perm), GEMM2, on the split and the pipelined kernels
    "void moe::ffn_gemm_bf16_split_kernel<4, 0, true, false>(moe::GemmArgs)": "ffn1",
    "void moe::ffn_gemm_bf16_split_kernel<4, 0, false, false>(moe::GemmArgs)": "ffn1",
    f"void moe::ffn_gemm_bf16_pipe_kernel<{TILE}, 4, 1024, 2, 0, true, false, false>(moe::GemmArgs)": "ffn1",
    "void moe::ffn_gemm_bf16_split_kernel<4, 1, true, false>(moe::GemmArgs)": "ffn2",
    f"void moe::ffn_gemm_bf16_pipe_kernel<{TILE}, 4, 1024, 2, 1, true, false, false>(moe::GemmArgs)": "ffn2",
    # backward: recompute, dh, dx_perm, weight gradients
    "void moe::ffn_gemm_bf16_split_kernel<4, 2, false, false>(moe::GemmArgs)": None,
    "void moe::ffn_gemm_bf16_split_kernel<4, 3, false, true>(moe::GemmArgs)": None,
    "void moe::ffn_gemm_bf16_split_kernel<4, 1, false, true>(moe::GemmArgs)": None,
    f"void moe::ffn_gemm_bf16_pipe_kernel<{TILE}, 4, 1024, 2, 4, false, false, true>(moe::GemmArgs)": None,
    # routing, dispatch and combine
    "void moe::route_mfma_kernel<64, 32, 4, 2, 8, false>(moe::RouteArgs, unsigned short const*)": "route",
    "void moe::route_variant_kernel<1>(moe::RouteArgs, int, float const*, float, float*)": None,
    "moe::hist_kernel(moe::DispatchArgs)": "hist",
    "moe::scatter_kernel(moe::DispatchArgs)": "scatter",
    "moe::gather_tiled_kernel(moe::DispatchArgs, unsigned short*, int)": "gather",
    "moe::gather_slots_kernel(long, int, long, long, void const*, int const*, void*)": None,
    "moe::combine_kernel(long, int, int, float const*, int const*, float const*, float*)": "combine",
}


def test_kernel_names_map_to_their_stage():
    for name, stage in NAMES.items():
        assert bench._stage_of(name) == stage, name


def test_first_gemm_algorithmic_bytes():
    from moe_inputs import get
    cfg = get("skewed_e64")
    S, active = 14789, 64          # the seeded routing's kept slots and active experts
    nblk = (cfg.T + bench.dispatch_block_tokens(cfg.T, cfg.E, cfg.k) - 1) // bench.dispatch_block_tokens(
        cfg.T, cfg.E, cfg.k)
    bf = bench.stage_bytes_flops(cfg, S, active, 2, nblk)
    d, f = cfg.d, cfg.d_ff
    assert bf["ffn1"][0] == active * d * f * 2 + S * d * 2 + S * f * 2 + active * f * 4 == 2452459520
    assert bf["ffn1"][1] == 2 * S * d * f
