"""Seeded synthetic inputs for the grouped NVFP4 MoE expert projection.

This package only draws random inputs (bytes, bf16 activations, routing).
It holds none of the projection's arithmetic, so both the fp64 oracle and
the HIP path can consume exactly the same bytes.
"""
from .moe_inputs import (  # noqa: F401
    CONFIGS,
    MoeShape,
    PROJ_DOWN,
    PROJ_GATE,
    PROJ_UP,
    SCALE2_F32,
    SCALE2_MX_F32,
    config,
    expert_bytes,
    gen_expert,
    gen_expert_mx,
    gen_logits,
    gen_routing,
    gen_x,
    proj_dims,
)
