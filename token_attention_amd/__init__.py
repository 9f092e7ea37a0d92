"""token_attention_amd: Multi-Token Attention layer (forward and gradients) on AMD MI355X (gfx950).

The compute lives in ``libmta.so`` (hand-written HIP, C ABI in ``include/mta.h``);
this package only marshals torch device tensors into it.
"""
from .mta import (  # noqa: F401
    FP32, GN, KQ_POST, KQ_PRE, MIX_POST, MIX_PRE, MTAError, attention_plain, backward_fused,
    backward_fused_workspace_bytes, backward_materialized, backward_workspace_bytes, check_args, forward,
    forward_materialized, forward_rows, forward_rows_split, forward_rows_split_noalloc, forward_train,
    last_error, lib, library_path, materialized_workspace_bytes, mta_layer, placement_flags, rows_split_plan,
    rows_split_workspace_bytes,
)
