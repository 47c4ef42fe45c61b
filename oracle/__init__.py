"""CPU fp64 oracle for the deterministic MoE layer.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import it. The product path (the HIP library and
its Python binding) never imports, calls or falls back to anything here.
"""
from .moe_oracle import (  # noqa: F401
    schedule, ring_row, minibatch_count,
    silu, swiglu, expert_ffn,
    forward, forward_tokens,
    backward, backward_tokens, backward_expert_weights,
    e4m3_decode, e4m3_encode, mxfp8_quantize, mxfp8_dequantize, mxfp8_roundtrip,
    forward_mxfp8, forward_mxfp8_tokens, backward_mxfp8, backward_mxfp8_expert_weights,
    backward_mxfp8_tokens, bf16_round,
    router_forward, router_backward,
    STATUS_BAD_EXPERT_ID,
)
