"""CPU oracle for the routed mixture-of-experts FFN layer of DeepSeek-V4.1-Flash.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from it.

Everything is computed in float64 from the exact values of the inputs (bf16
activations and weights, fp32 router weights, MXFP4 expert weights decoded
exactly), directly from the definitions, with no tiling, fusion or reordering.
"""

from .moe_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    rmsnorm,
    e2m1_value,
    e2m1_table,
    e8m0_value,
    decode_mxfp4,
    mxfp4_packed_bytes,
    e4m3_value,
    e4m3_table,
    decode_mxfp8,
    EXPERT_FORMATS,
    softplus,
    sqrtsoftplus,
    silu,
    clamped_swiglu,
    router_logits,
    route,
    route_with_selection,
    valid_selections,
    permute,
    expert_mlp,
    shared_expert,
    combine,
    layer_forward,
    routed_expert_weights,
)
