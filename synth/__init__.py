"""Seeded synthetic inputs shared by the CPU oracle checks and the GPU path.

This package holds no attention, softmax, GEMM, scatter or Burst-Gap arithmetic. It draws
random numbers, casts them to bf16 bit patterns, and builds structured probe patterns.
Both sides of every parity test consume the exact bytes produced here.
"""

from .moe import MOE_WORKLOADS, MoeWorkload, moe_routing, moe_tensors  # noqa: F401
from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    f32_to_bf16_bits,
    make_inputs,
    make_placement_probe,
    make_placement_probe_torch,
    workload,
)
