"""Packed variable-length ("thd") attention for AMD Instinct MI355X (gfx950).

The compute path is libthdattn.so (hand-written HIP kernels behind the C ABI
of include/thd_attn.h); this package is its thin torch binding.
"""
from .attention import (  # noqa: F401
    MASK_CAUSAL,
    MASK_CAUSAL_BOTTOM_RIGHT,
    MASK_PADDING,
    attn_bwd,
    attn_fwd,
    bwd_workspace_size,
    fwd_workspace_size,
    padding_mask,
    padding_masks,
    thd_attention,
)
from .metrics import valid_pairs, attention_flops  # noqa: F401

__version__ = "0.1.0"
