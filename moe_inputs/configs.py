"""Workload table for the MoE layer forward.

Each entry fixes the shapes, the routing hyper-parameters and the recipe of the
seeded synthetic inputs.  Nothing here computes any step of the layer: the
capacity, the routing and the expert FFN are defined by the oracle and the HIP
library, never by this table.

Sources of the shapes and distributions:
  * top-k gate followed by a softmax over the selected logits, expert FFN
    Linear(d, 4d) -> GELU -> Linear(4d, d): "PithTrain" page, section 4.1
    (the PithTrainMoELayer sketch).
  * capacity factor: "PithTrain" page, section 4.3 item 1.
  * temperature softmax over a coarse top-8 ("Hybrid Soft MoE"):
    "Expert Parallelism: Scaling Mixture-of-Experts Models" page, section 2.2.
  * skewed load with a coefficient of variation near 0.8: same page,
    section 2.1 (first flaw, load imbalance).
  * co-activation hot spots: same page, section 3.2 (routing heat-map).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                      # tokens in the batch
    d: int                      # model width
    E: int                      # number of experts
    k: int                      # experts per token
    d_ff: int                   # expert hidden width
    dtype: str = "bf16"         # "bf16" or "fp32": dtype of x, W1, W2 and h
    capacity_factor: float = 0.0  # <= 0 means no capacity limit
    temperature: float = 1.0
    aux_lambda: float = 0.01
    # input recipe
    seed: int = 0
    zipf_s: float = 0.0         # > 0: gate bias b_e = zipf_alpha * ln p(rank e+1)
    zipf_alpha: float = 1.0
    cluster_frac: float = 0.0   # fraction of tokens drawn around shared centroids
    n_centroids: int = 16
    cluster_noise: float = 0.1
    bias_std: float = 0.0       # std of b1, b2 (0 = zero biases)
    gate_bias_std: float = 0.0  # extra N(0, std^2) gate bias (parity cases only)
    note: str = ""

    @property
    def has_gate_bias(self) -> bool:
        return self.zipf_s > 0 or self.gate_bias_std > 0

    def scaled(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


# Gate-bias strength for the skewed E=64 workload.  The workload asks for a
# Zipf(s=1.2) rank bias "so that the load CV is about 0.8".  Taken literally
# (alpha = 1) the bias spans 1.2*ln(64) ~ 5 nats against unit-variance logits
# and the routed load CV is ~3.7 with most slots dropped; alpha scales the
# log-probabilities so that the stated CV is met on seed 0 (measured by the
# calibration recorded with the workload recipe).  The literal reading is kept
# as its own parity case.
SKEW_ALPHA = 0.24

CONFIGS: Dict[str, MoEConfig] = {}


def _add(c: MoEConfig) -> None:
    CONFIGS[c.name] = c


# --- the five workloads --------------------------------------------------
_add(MoEConfig("tiny_fp32", T=256, d=64, E=8, k=2, d_ff=256, dtype="fp32",
               capacity_factor=0.0,
               note="fp32 everything, exact-erf GELU, no capacity limit"))
_add(MoEConfig("bf16_e16", T=4096, d=1024, E=16, k=2, d_ff=4096,
               capacity_factor=1.25))
_add(MoEConfig("skewed_e64", T=8192, d=2048, E=64, k=2, d_ff=8192,
               capacity_factor=2.0, zipf_s=1.2, zipf_alpha=SKEW_ALPHA,
               note="Zipf(1.2) rank bias on the gate, scaled to load CV ~0.8"))
_add(MoEConfig("hybrid_e128", T=8192, d=1024, E=128, k=8, d_ff=4096,
               capacity_factor=0.0, temperature=0.2,
               note="coarse top-8 then softmax(logits/0.2) over the 8"))
_add(MoEConfig("large_e256", T=32768, d=2048, E=256, k=2, d_ff=8192,
               capacity_factor=1.25, cluster_frac=0.3,
               note="30% of tokens around 16 centroids"))

# --- extra parity cases ----------------------------------------------------
_add(CONFIGS["skewed_e64"].scaled(name="skewed_e64_literal", zipf_alpha=1.0,
                                  note="Zipf bias taken literally (alpha=1)"))
_add(CONFIGS["tiny_fp32"].scaled(name="tiny_fp32_bias", bias_std=0.1,
                                 gate_bias_std=0.1, capacity_factor=0.75))
# several tiles in every GEMM dimension plus ragged tails, drops, k=3, biases
_add(MoEConfig("ragged_bf16", T=1000, d=200, E=12, k=3, d_ff=328,
               capacity_factor=1.0, temperature=0.7, bias_std=0.1,
               gate_bias_std=0.5))
_add(MoEConfig("ragged_fp32", T=777, d=136, E=6, k=2, d_ff=200, dtype="fp32",
               capacity_factor=1.1, temperature=1.3, bias_std=0.1,
               gate_bias_std=0.3))
# medium bf16 case: spans many 128x128 tiles per expert, realistic widths
_add(MoEConfig("medium_bf16", T=2048, d=512, E=16, k=2, d_ff=2048,
               capacity_factor=1.25, bias_std=0.1))
_add(MoEConfig("hybrid_small", T=1024, d=256, E=32, k=8, d_ff=1024,
               capacity_factor=0.0, temperature=0.2))
_add(MoEConfig("clustered_small", T=2048, d=256, E=64, k=2, d_ff=512,
               capacity_factor=1.25, cluster_frac=0.3))
_add(MoEConfig("single_token", T=1, d=64, E=4, k=2, d_ff=64,
               capacity_factor=1.0, bias_std=0.1))
_add(MoEConfig("one_expert", T=300, d=96, E=1, k=1, d_ff=160,
               capacity_factor=0.0, bias_std=0.1))
_add(MoEConfig("k_equals_e", T=300, d=64, E=4, k=4, d_ff=128,
               capacity_factor=0.0, temperature=0.5, bias_std=0.1))
# the matrix-core router with up to 16 winners per token: k = E on 12
# experts (every expert, ragged d) and k = 16 of 40 experts (4 logits per lane)
_add(MoEConfig("soft_k_equals_e12", T=1000, d=200, E=12, k=12, d_ff=136,
               capacity_factor=0.0, temperature=0.2, bias_std=0.1,
               gate_bias_std=0.3))
_add(MoEConfig("k16_e40", T=777, d=136, E=40, k=16, d_ff=200,
               capacity_factor=1.5, temperature=0.7, bias_std=0.1))
# the router's eight-wave expert split: 100 experts (padded to 128), and
# 200 experts (padded to 256) over enough tokens for its 128-token tiles,
# with a ragged last tile
_add(MoEConfig("e100_k5", T=1500, d=256, E=100, k=5, d_ff=200,
               capacity_factor=1.3, temperature=0.8, bias_std=0.1,
               gate_bias_std=0.3))
_add(MoEConfig("e200_t33001", T=33001, d=64, E=200, k=2, d_ff=64,
               capacity_factor=1.1, bias_std=0.1, gate_bias_std=0.3))
# the fused forward's token-by-token gather in two passes per row (d > 4096
# columns: 576 chunks of 16 bytes against 512 per pass), with a K tail
# (4608 = 144 x 32) and a gate over K = 4608
_add(MoEConfig("wide_d", T=2048, d=4608, E=8, k=2, d_ff=64,
               capacity_factor=0.0, bias_std=0.1, gate_bias_std=0.3,
               note="x 18 MiB and S = 2T: the gather takes the token way"))
_add(MoEConfig("cap_one", T=200, d=64, E=8, k=2, d_ff=64,
               capacity_factor=0.02, bias_std=0.1,
               note="capacity clips to 1 slot per expert"))

# the 256 x 256 tile path with ragged tails: d and d_ff are multiples of
# neither the 32-wide K step nor the 256-wide N tile, uneven expert loads
_add(MoEConfig("ragged_large", T=16384, d=1800, E=8, k=2, d_ff=2000,
               capacity_factor=1.1, bias_std=0.1, gate_bias_std=0.5,
               note="odd K-step counts (57, 63): one all-zero step per item"))
_add(MoEConfig("ragged_large_even", T=32768, d=1000, E=8, k=2, d_ff=1976,
               capacity_factor=1.1, bias_std=0.1, gate_bias_std=0.5,
               note="even K-step counts (32, 62) with a partial last step"))

# dense soft MoE ([EP] section 2.2): every token weighted over all experts
# by softmax(logits / 0.2); k = E with no capacity limit, 4096 rows per
# expert, so the grouped GEMMs run in their matrix-core-bound regime
_add(MoEConfig("dense_soft_e16", T=4096, d=1024, E=16, k=16, d_ff=4096,
               capacity_factor=0.0, temperature=0.2,
               note="k = E: the soft MoE of every expert, 4096 rows each"))
# the page's naive soft MoE over all 128 experts ([EP] section 2.2): k = E =
# 128 selects past the register router's 32 winners (the selection by rank),
# 1024 rows per expert, 131072 rows through each grouped GEMM
_add(MoEConfig("dense_soft_e128", T=1024, d=1024, E=128, k=128, d_ff=4096,
               capacity_factor=0.0, temperature=0.2,
               note="k = E = 128: every token through every expert"))

# several grouped-GEMM work items per workgroup at long K, compared in full:
# K = 1536 (48 K-steps) in both GEMMs, 6 column tiles of 256 and skewed
# expert loads (1-10 row tiles of 256 per expert) give about 970 items
# per GEMM for 256 workgroups; the oracle still finishes every row
_add(MoEConfig("multi_item", T=16384, d=1536, E=64, k=2, d_ff=1536,
               capacity_factor=0.0, zipf_s=1.2, zipf_alpha=SKEW_ALPHA, bias_std=0.1,
               note="3+ work items per workgroup at K = 1536, every row compared"))
# the backward's weight-gradient GEMM in its pipelined form (2048 rows per
# expert on average) with every gradient compared in full
_add(MoEConfig("bw_long_rows", T=16384, d=512, E=16, k=2, d_ff=1024,
               capacity_factor=0.0, bias_std=0.1, gate_bias_std=0.3,
               note="long row segments: the weight gradients' pipelined form, full gradients"))

# expert segments of 65536 rows at d_ff = 16384: a weight-gradient GEMM over
# one segment spans 2 GiB of bf16 operand bytes, past the 32-bit offsets of
# the pipelined weight-gradient form (the 128 x 128 kernel takes it instead)
_add(MoEConfig("wgrad_2g", T=65536, d=16, E=2, k=2, d_ff=16384,
               capacity_factor=0.0, bias_std=0.1,
               note="weight-gradient segments of 2 GiB of operand bytes"))

# long expert segments next to idle and one-row experts: the literal Zipf(1.2)
# gate bias without a capacity limit gives 3 idle experts, several with 1-2
# rows and the busiest with ~25k (the backward's weight-gradient GEMM runs
# its pipelined form from 1024 rows per expert on average)
_add(MoEConfig("long_segments", T=32768, d=1024, E=64, k=2, d_ff=1024,
               capacity_factor=0.0, zipf_s=1.2, zipf_alpha=1.0,
               note="idle, one-row and ~25k-row experts in one batch"))

# limits of the library: E = 1024 experts, k = 32 choices per token
_add(MoEConfig("max_experts", T=2048, d=64, E=1024, k=4, d_ff=64,
               capacity_factor=1.0, bias_std=0.1))
_add(MoEConfig("max_k", T=256, d=64, E=48, k=32, d_ff=64,
               capacity_factor=0.0, temperature=2.0, bias_std=0.1))
# the selection by rank (k above 32): every expert of 64, compared in full;
# 100 of 200 experts with a capacity limit (drops) and ragged d
_add(MoEConfig("soft_k64_e64", T=384, d=128, E=64, k=64, d_ff=256,
               capacity_factor=0.0, temperature=0.2, bias_std=0.1,
               gate_bias_std=0.3))
_add(MoEConfig("k100_e200", T=300, d=72, E=200, k=100, d_ff=96,
               capacity_factor=0.9, temperature=0.7, bias_std=0.1))
# the selection by rank after the vector-ALU gate: an fp32 layer, and a bf16
# layer of more than 256 experts
_add(MoEConfig("k40_fp32", T=200, d=64, E=48, k=40, d_ff=64, dtype="fp32",
               capacity_factor=1.2, temperature=0.5, bias_std=0.1))
_add(MoEConfig("k50_e300", T=257, d=96, E=300, k=50, d_ff=64,
               capacity_factor=0.0, temperature=1.0, bias_std=0.1, gate_bias_std=0.3))

# The workload the throughput metric is quoted on (E=64, top-2, d=2048).
HEADLINE = "skewed_e64"
# The five workloads in their published order.
WORKLOADS = ["tiny_fp32", "bf16_e16", "skewed_e64", "hybrid_e128", "large_e256"]


def get(name: str) -> MoEConfig:
    return CONFIGS[name]
