"""MI355X (gfx950) kernelized linear attention.

The compute path is the HIP library ``liblinattn.so`` (C ABI in
``include/linattn.h``); this package is its thin Python binding.  PyTorch is
used only for device memory and the current stream.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LA_BF16,
    LA_F32,
    LA_OP_BWD_CAUSAL,
    LA_OP_BWD_NONCAUSAL,
    LA_OP_FWD_CAUSAL,
    LA_OP_FWD_NONCAUSAL,
    LIB_PATH,
    LinAttnError,
    causal_linear_attention,
    la_backward_causal,
    la_backward_causal_state,
    la_backward_noncausal,
    la_decode_step,
    la_decode_steps,
    la_decode_steps_features,
    la_forward_causal_features,
    la_forward_noncausal_features,
    favor_features,
    favor_features_blocks,
    features_workspace_size,
    la_forward_causal_features_blocks,
    la_forward_noncausal_features_blocks,
    la_decode_steps_features_blocks,
    la_backward_causal_features,
    la_backward_causal_features_blocks,
    la_backward_noncausal_features_blocks,
    favor_features_blocks_backward,
    la_backward_noncausal_features,
    favor_features_backward,
    favor_attention,
    la_forward_causal,
    la_forward_causal_grouped,
    la_forward_noncausal,
    linear_attention,
    load_library,
    new_saved_state,
    profile_enable,
    profile_entries,
    saved_state_size,
    backward_wait_failures,
    set_wait_limit,
    wait_limit,
    workspace_size,
)

__version__ = "0.1.0"
