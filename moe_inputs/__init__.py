"""Workload descriptors and seeded synthetic inputs for the MoE expert layer.

Shared by the CPU oracle and the GPU tests and bench; it holds no step of the
layer itself.
"""
from .configs import CONFIGS, ALIASES, MoEConfig, get  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits, bf16_to_f32, make_inputs, make_routing, quantise_weight_int8, weight_f32, x_f32,
)
