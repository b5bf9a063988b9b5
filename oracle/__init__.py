"""fp64 CPU oracle for packed-thd attention and its padding mask.

Test infrastructure only: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the library itself.
"""
from .thd_oracle import (  # noqa: F401
    attn_bwd,
    attn_bwd_key_range,
    attn_fwd,
    attn_rows,
    padding_mask,
    padding_mask_loop,
    round_to_storage,
    sequence_rows,
    valid_pairs,
    visible_keys,
)
