"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .moe_oracle import (  # noqa: F401
    E2M1,
    E4M3FN,
    bf16_bits_to_f64,
    blend,
    dequant,
    down_rows,
    e2m1_value,
    e4m3fn_value,
    expert_weights,
    gate_up_silu_rows,
    moe_layer,
    route_topk,
    silu,
    sort_routes,
    transpose_u8,
)
