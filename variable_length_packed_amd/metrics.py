"""Host-side work accounting for packed-thd attention (no device access).

Valid pairs are the (query, key) pairs the attention actually computes: for a
sequence with lq queries and lk keys, lq*lk under the ``padding`` mask type,
sum_i min(i+1, lk) under top-left ``padding_causal`` and
sum_i clamp(i+1+lk-lq, 0, lk) under ``padding_causal_bottom_right``.  FLOPs count two per
multiply-add of each matrix product: forward 2 products (QK^T, PV) = 4*d per
pair; backward 5 products (S recompute, dP, dV, dK, dQ) = 10*d per pair, the
convention the throughput metric is quoted in.  The two passes of the backward
for head dims up to 128 form S and dP once each: the dq pass does 3 products
(S, dP, dQ: 6*d per pair), the dk/dv pass 4 (S, dP, dV, dK: 8*d per pair).
"""
import numpy as np


def pairs_per_sequence(lens_q, lens_kv, mask_type):
    """Per-sequence pair counts; mask_type 1 = top-left causal, 2 = bottom-right
    causal, anything else = padding (a boolean causal flag is types 0 / 1)."""
    lq = np.asarray(lens_q, dtype=np.int64)
    lk = np.asarray(lens_kv, dtype=np.int64)
    mt = np.asarray(mask_type).astype(np.int64)
    full = lq * lk
    # sum_{i<lq} min(i+1, lk): the first min(lq, lk) rows see i+1 keys, the rest lk
    m = np.minimum(lq, lk)
    top_left = m * (m + 1) // 2 + (lq - m) * lk
    # sum_{i<lq} clamp(i+1+lk-lq, 0, lk): lk >= lq gives lq(lq+1)/2 + lq(lk-lq);
    # lk < lq leaves the first lq-lk rows empty and the rest see 1..lk keys
    bottom_right = np.where(lk >= lq, lq * (lq + 1) // 2 + lq * (lk - lq), lk * (lk + 1) // 2)
    return np.where(mt == 1, top_left, np.where(mt == 2, bottom_right, full))


def valid_pairs(lens_q, lens_kv, causal, h_q=1):
    """Total valid (query, key) pairs over all sequences and query heads."""
    return int(pairs_per_sequence(lens_q, lens_kv, causal).sum()) * int(h_q)


def attention_flops(pairs, d, part="fwd+bwd"):
    per = {"fwd": 4, "bwd": 10, "fwd+bwd": 14, "bwd_dq_pass": 6, "bwd_dkdv_pass": 8}[part]
    return per * int(d) * int(pairs)
