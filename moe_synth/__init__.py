"""Seeded synthetic inputs for the routed MoE FFN layer.

Shared by the oracle-side tests and the HIP-side tests and benchmark; it holds
none of the layer's arithmetic (no routing, no expert math, no MXFP4
decoding).  It draws random tensors and encodes the synthetic fp32 expert
weights into the MXFP4 (or MXFP8) byte layout the layer consumes.
"""

from .configs import CONFIGS, LayerConfig  # noqa: F401
from .gen import (  # noqa: F401
    ExpertTensor,
    LayerInputs,
    make_inputs,
    make_router_inputs,
    mxfp4_encode,
    mxfp8_encode,
    pack_nibbles,
    f32_to_bf16_bits,
    derive_seed,
)
