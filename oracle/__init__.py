"""Float64 CPU oracle (test infrastructure only; see oracle.oracle)."""

from .oracle import (  # noqa: F401
    BLOCK,
    E4M3_MAX,
    SAFETY,
    h_drift,
    bf16_to_f64,
    block_scales,
    dequant_expert,
    e4m3_encode,
    e4m3_lut,
    e4m3_midpoint_distance,
    e4m3_value,
    forward,
    forward_dense,
    gathered_count,
    quantize_rows,
    route,
    routed_experts,
    silu,
    sort_pairs,
)
