"""Seeded synthetic inputs for the MoE layer (shared by the oracle's tests,
the GPU parity tests and the benchmark).

This package draws random numbers and converts storage formats. It holds none
of the layer's arithmetic: no schedule, no expert FFN, no combine.
"""
from .moe_inputs import (  # noqa: F401
    Problem, CONFIGS, problem, bf16_round, bf16_to_f32, f32_to_bf16_bits,
    make_x, make_routing, router_weights, make_expert, make_all_experts, make_dy,
)
