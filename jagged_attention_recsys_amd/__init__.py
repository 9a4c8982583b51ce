"""MI355X (gfx950) jagged attention: JFA softmax and GDPA SiLU/GELU forward and backward,
including the block-diagonal BlockAttention form.

The computation runs in ``libjagged_attn.so`` (hand-written HIP kernels behind the C
ABI of ``include/jagged_attn.h``); this package only marshals torch tensors into it.
"""
from .ops import (  # noqa: F401
    block_attn_workspace_size,
    bwd_workspace_size,
    fwd_schedule,
    fwd_tile_shape,
    fwd_workspace_size,
    jagged_attn_bwd,
    jagged_attn_fwd,
    jagged_attn_fwd_noalloc,
    jagged_block_attn_bwd,
    jagged_block_attn_fwd,
    jagged_attn_fwd_mxfp8,
    mxfp8_quantize,
    validate_offsets,
)

__all__ = [
    "jagged_attn_fwd",
    "jagged_attn_fwd_noalloc",
    "jagged_attn_bwd",
    "jagged_block_attn_fwd",
    "jagged_block_attn_bwd",
    "jagged_attn_fwd_mxfp8",
    "mxfp8_quantize",
    "fwd_workspace_size",
    "bwd_workspace_size",
    "block_attn_workspace_size",
    "fwd_schedule",
    "fwd_tile_shape",
    "validate_offsets",
]
