"""Seeded synthetic inputs and the workload table, shared by the oracle-side
tests and the HIP-side tests and benchmark.  Holds no step of the layer."""
from .configs import CONFIGS, HEADLINE, WORKLOADS, MoEConfig, get  # noqa: F401
from .gen import (bf16_bits_to_f32, f32_to_bf16_bits, make_experts,  # noqa: F401
                  make_gate, make_inputs, make_x)
