"""MI355X (gfx950) HIP implementation of the DeepSeek-V4.1-Flash routed MoE FFN layer.

The layer runs in libmoe_ffn.so (hand-written HIP kernels behind the C ABI
declared in include/moe_ffn.h); this package only builds and binds it.
"""

from ._lib import (  # noqa: F401
    MoeConfig,
    MoeError,
    MoeWeights,
    config_from,
    header_functions,
    load,
    make_config,
    make_weights,
    moe_combine,
    moe_expert_ffn,
    moe_layer_forward,
    moe_layer_forward_noalloc,
    moe_layer_forward_timed,
    moe_permute,
    moe_rmsnorm,
    moe_route,
    moe_workspace_bytes,
    weights_from,
    workspace,
)
