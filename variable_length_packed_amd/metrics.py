"""Host-side work accounting for packed-thd attention (no device access).

Valid pairs are the (query, key) pairs the attention actually computes: for a
sequence with lq queries and lk keys, lq*lk under the ``padding`` policy and
sum_i min(i+1, lk) under top-left ``padding_causal``.  FLOPs count two per
multiply-add of each matrix product: forward 2 products (QK^T, PV) = 4*d per
pair; backward 5 products (S recompute, dP, dV, dK, dQ) = 10*d per pair.
"""
import numpy as np


def pairs_per_sequence(lens_q, lens_kv, causal):
    lq = np.asarray(lens_q, dtype=np.int64)
    lk = np.asarray(lens_kv, dtype=np.int64)
    c = np.asarray(causal).astype(bool)
    full = lq * lk
    # sum_{i<lq} min(i+1, lk): the first min(lq, lk) rows see i+1 keys, the rest lk
    m = np.minimum(lq, lk)
    causal_pairs = m * (m + 1) // 2 + (lq - m) * lk
    return np.where(c, causal_pairs, full)


def valid_pairs(lens_q, lens_kv, causal, h_q=1):
    """Total valid (query, key) pairs over all sequences and query heads."""
    return int(pairs_per_sequence(lens_q, lens_kv, causal).sum()) * int(h_q)


def attention_flops(pairs, d, part="fwd+bwd"):
    per = {"fwd": 4, "bwd": 10, "fwd+bwd": 14}[part]
    return per * int(d) * int(pairs)
