"""CPU oracle (test infrastructure only; see moe_ref's header)."""
from .moe_ref import (  # noqa: F401
    bf16_to_f64,
    expert_block_backward,
    expert_offsets,
    gmm,
    gmm_bwd_input,
    gmm_bwd_weight,
    gmm_swiglu,
    moe_layer_backward,
    moe_layer_forward,
    permute,
    permute_bwd,
    permute_maps,
    round_bf16,
    sigmoid,
    swiglu,
    swiglu_bwd,
    to_bf16_bits,
    tokens_per_expert,
    unpermute,
    unpermute_bwd,
)
from . import mx_ref  # noqa: F401,E402
