"""Plain fp64 CPU oracle for packed variable-length ("thd") attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, tables or
constants with the HIP library; it sees the same seeded inputs (upcast to
float64) and nothing else.

Sources (the three web pages the method is defined by):

* Megatron-LM issue "How to pad sequences that cannot be evenly split in
  context parallelism (CP)?" -- the question (packed ``thd`` q/k/v, int32
  ``cu_seqlens``, ``max_seqlen``, the ``padding`` mask type, pad tokens that
  carry garbage) and the printed reference output of the full attention.
* TransformerEngine PR "Add per-sequence causal policy to packed THD
  attention" -- Description (one causal flag per packed sequence), Changes,
  and the maintainer's two-call example with ``cu_seqlens_padded`` (slot
  starts; pad positions of each call's output are zeros, so the two outputs
  can be summed).
* TransformerEngine PR "[PyTorch] Build the attention padding mask without
  host syncs" -- Description (the mask is ``positions >= seqlens``; the older
  per-sequence list construction), Changes (buffers longer than batch+1),
  Equivalence (the exhaustive case spaces; invalid lengths).

Where the pages are silent the plainest reading is taken; every such reading
is listed with the design notes of the repository.  In particular:

* softmax scale defaults to 1/sqrt(head_dim) (the only scale that reproduces
  the issue's printed reference output);
* ``padding_causal`` is top-left aligned: query i of a sequence sees key j
  iff j <= i; ``padding_causal_bottom_right`` (the third mask type of the
  maintainer's ``attn_mask_type_per_seq`` proposal in the per-sequence causal
  PR) aligns the diagonal with the last key: j <= i + (lk - lq);
* sequence b occupies rows [start_b, start_b + len_b) where start_b is
  ``cu_seqlens_padded[b]`` when given, else ``cu_seqlens[b]``; every other
  row is pad and every output written for it is 0;
* a query row with no visible key (kv length 0) gets output 0 and
  log-sum-exp -inf, and contributes no gradient;
* GQA: query head hq reads key/value head hq // (h_q // h_kv).
"""

import math

import numpy as np

__all__ = [
    "MASK_PADDING",
    "MASK_CAUSAL",
    "MASK_CAUSAL_BOTTOM_RIGHT",
    "padding_mask",
    "padding_mask_loop",
    "sequence_rows",
    "visible_keys",
    "valid_pairs",
    "attn_fwd",
    "attn_bwd",
    "attn_rows",
    "attn_bwd_key_range",
    "round_to_storage",
]


# Per-sequence mask types ("Add per-sequence causal policy to packed THD
# attention", maintainer review: a per-sequence mask type naming "padding",
# "padding_causal" and "padding_causal_bottom_right").  A boolean causal flag
# is the special case 0 / 1.
MASK_PADDING = 0
MASK_CAUSAL = 1
MASK_CAUSAL_BOTTOM_RIGHT = 2


def _mask_type(mask_type, b):
    return int(mask_type[b]) if mask_type is not None else MASK_PADDING


# ---------------------------------------------------------------------------
# Padding mask
# ---------------------------------------------------------------------------

def padding_mask(cu_seqlens, batch_size, max_seqlen):
    """Definitional padding mask, True = pad.

    Follows "[PyTorch] Build the attention padding mask without host syncs",
    Description: seqlens are the first ``batch_size`` differences of the
    cumulative buffer (entries past batch_size+1 are ignored, Changes), and
    position s of row b is pad iff s >= seqlens[b].  Shape [B, 1, 1, max].

    The differences are taken in int32, as the int32 ``cu_seqlens`` tensor
    of the page does (two's-complement wrap on overflow); positions are
    compared as int64.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int32)
    if batch_size < 0 or max_seqlen < 0:
        raise ValueError("batch_size and max_seqlen must be >= 0")
    if cu.shape[0] < batch_size + 1 and batch_size > 0:
        raise ValueError("cu_seqlens needs at least batch_size + 1 entries")
    with np.errstate(over="ignore"):
        seqlens = (cu[1:batch_size + 1] - cu[:batch_size]).astype(np.int64)
    positions = np.arange(max_seqlen, dtype=np.int64)
    mask = positions[None, :] >= seqlens[:, None]
    return mask.reshape(batch_size, 1, 1, max_seqlen)


def padding_mask_loop(cu_seqlens, batch_size, max_seqlen):
    """The older per-sequence construction of the same mask, True = pad.

    Follows the loop quoted in the Description of "[PyTorch] Build the
    attention padding mask without host syncs": for each of the first
    ``batch_size`` sequences a host list of ``len`` False then
    ``max_seqlen - len`` True, rows stacked.  A row whose length is not
    ``max_seqlen`` (a sequence longer than max_seqlen, Equivalence) cannot be
    stacked and raises, as the concatenation on the page does.
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    rows = []
    for i in range(batch_size):
        n = cu[i + 1] - cu[i]
        row = [False] * n + [True] * (max_seqlen - n)
        if len(row) != max_seqlen:
            raise ValueError(f"sequence {i}: row of length {len(row)} cannot be "
                             f"stacked with rows of length {max_seqlen}")
        rows.append(row)
    out = np.array(rows, dtype=bool).reshape(batch_size, max_seqlen)
    return out.reshape(batch_size, 1, 1, max_seqlen)


# ---------------------------------------------------------------------------
# Sequence placement and the attention mask
# ---------------------------------------------------------------------------

def sequence_rows(cu_seqlens, batch_size, cu_seqlens_padded=None):
    """(start_row, length) of each packed sequence.

    Lengths come from ``cu_seqlens`` (the issue's ``cu_seqlens_q = [0, 7]``);
    starts come from ``cu_seqlens_padded`` when it is given (slot starts in
    the maintainer's two-call example, which need not begin at 0), else from
    ``cu_seqlens`` itself.
    """
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    starts = cu if cu_seqlens_padded is None else \
        [int(x) for x in np.asarray(cu_seqlens_padded).reshape(-1)]
    return [(starts[b], cu[b + 1] - cu[b]) for b in range(batch_size)]


def visible_keys(lq, lk, mask_type):
    """Boolean [lq, lk]: True where query i may attend key j.

    ``padding`` (0): every valid key.  ``padding_causal`` (1, the per-sequence
    flag of "Add per-sequence causal policy to packed THD attention"):
    top-left aligned, j <= i.  ``padding_causal_bottom_right`` (2, named in
    that PR's maintainer review): the diagonal ends at the last key,
    j <= i + (lk - lq); when lq > lk the first lq - lk queries see no key.
    Any other value is taken as ``padding``.
    """
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    allowed = np.ones((lq, lk), dtype=bool)
    mt = int(mask_type)
    if mt == MASK_CAUSAL:
        allowed &= j <= i
    elif mt == MASK_CAUSAL_BOTTOM_RIGHT:
        allowed &= j <= i + (lk - lq)
    return allowed


def valid_pairs(cu_q, cu_kv, batch_size, mask_type=None):
    """Number of (query, key) pairs that attention actually computes, per head."""
    total = 0
    for b in range(batch_size):
        lq = int(cu_q[b + 1]) - int(cu_q[b])
        lk = int(cu_kv[b + 1]) - int(cu_kv[b])
        total += int(visible_keys(lq, lk, _mask_type(mask_type, b)).sum())
    return total


def _default_scale(d, scale):
    if scale is None or not (scale > 0):
        return 1.0 / math.sqrt(d)
    return float(scale)


def _check_shapes(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [T, h, d]")
    if k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("k and v must match, head_dim must agree")
    if q.shape[1] % k.shape[1] != 0:
        raise ValueError("h_q must be a multiple of h_kv")


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------

def attn_fwd(q, k, v, cu_q, cu_kv, batch_size, mask_type=None,
             cu_q_padded=None, cu_kv_padded=None, scale=None):
    """softmax(scale * Q K^T + mask) V, one sequence at a time.

    q: [T_q, h_q, d]; k, v: [T_kv, h_kv, d] (float64 upcasts of the device
    inputs).  Returns (out [T_q, h_q, d], lse [h_q, T_q]).  Rows outside every
    sequence are 0 in ``out`` and -inf in ``lse``; a query row that sees no
    key is 0 / -inf too.

    This is the attention of the issue's full reference call, restricted to
    each sequence's valid tokens, with the per-sequence mask type
    (``visible_keys``) and the padded placement of the two-call example.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _check_shapes(q, k, v)
    T_q, h_q, d = q.shape
    h_kv = k.shape[1]
    group = h_q // h_kv
    scale = _default_scale(d, scale)

    out = np.zeros_like(q)
    lse = np.full((h_q, T_q), -np.inf)
    rows_q = sequence_rows(cu_q, batch_size, cu_q_padded)
    rows_k = sequence_rows(cu_kv, batch_size, cu_kv_padded)
    for b in range(batch_size):
        oq, lq = rows_q[b]
        ok, lk = rows_k[b]
        if lq <= 0:
            continue
        allowed = visible_keys(lq, lk, _mask_type(mask_type, b))
        for hq in range(h_q):
            hk = hq // group
            Q = q[oq:oq + lq, hq, :]
            K = k[ok:ok + lk, hk, :]
            V = v[ok:ok + lk, hk, :]
            S = scale * (Q @ K.T)
            S = np.where(allowed, S, -np.inf)
            has_key = allowed.any(axis=1)
            m = np.where(has_key, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.where(allowed, np.exp(S - m[:, None]), 0.0)
            denom = E.sum(axis=1)
            P = np.divide(E, denom[:, None], out=np.zeros_like(E),
                          where=has_key[:, None])
            out[oq:oq + lq, hq, :] = P @ V
            with np.errstate(divide="ignore"):
                lse[hq, oq:oq + lq] = np.where(has_key, m + np.log(denom), -np.inf)
    return out, lse


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def attn_bwd(q, k, v, dout, cu_q, cu_kv, batch_size, mask_type=None,
             cu_q_padded=None, cu_kv_padded=None, scale=None, out=None):
    """Gradients (dq, dk, dv) of sum(out * dout) for ``attn_fwd``.

    Textbook softmax-attention backward, per sequence and query head, with the
    probabilities recomputed from scratch:
    dV = P^T dO;  dP = dO V^T;  dS = P * (dP - D),  D = rowsum(P * dP);
    dQ = scale dS K;  dK = scale dS^T Q.
    Key/value gradients of a GQA group are summed over its query heads.
    ``dout`` at pad rows is ignored and every pad row of dq/dk/dv is 0.

    ``out``: the forward's output as a backward receives it (a backward call
    takes the saved output as an input).  When given, D is rowsum(dO * out)
    over those values -- equal to rowsum(P * dP) for the exact output, since
    dO . O_i = sum_j P_ij (dO_i . V_j) -- so the effect of storing the output
    in a 16-bit type can be modelled exactly.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    _check_shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    T_q, h_q, d = q.shape
    h_kv = k.shape[1]
    group = h_q // h_kv
    scale = _default_scale(d, scale)

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows_q = sequence_rows(cu_q, batch_size, cu_q_padded)
    rows_k = sequence_rows(cu_kv, batch_size, cu_kv_padded)
    for b in range(batch_size):
        oq, lq = rows_q[b]
        ok, lk = rows_k[b]
        if lq <= 0 or lk <= 0:
            continue
        allowed = visible_keys(lq, lk, _mask_type(mask_type, b))
        has_key = allowed.any(axis=1)
        for hq in range(h_q):
            hk = hq // group
            Q = q[oq:oq + lq, hq, :]
            K = k[ok:ok + lk, hk, :]
            V = v[ok:ok + lk, hk, :]
            dO = dout[oq:oq + lq, hq, :]
            S = np.where(allowed, scale * (Q @ K.T), -np.inf)
            m = np.where(has_key, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.where(allowed, np.exp(S - m[:, None]), 0.0)
            denom = E.sum(axis=1)
            P = np.divide(E, denom[:, None], out=np.zeros_like(E),
                          where=has_key[:, None])
            dV = P.T @ dO
            dP = dO @ V.T
            if out is None:
                Drow = (P * dP).sum(axis=1)
            else:
                Drow = (dO * np.asarray(out[oq:oq + lq, hq, :], dtype=np.float64)).sum(axis=1)
            dS = P * (dP - Drow[:, None])
            dq[oq:oq + lq, hq, :] += scale * (dS @ K)
            dk[ok:ok + lk, hk, :] += scale * (dS.T @ Q)
            dv[ok:ok + lk, hk, :] += dV
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Selected rows of one sequence and head (for checks at full size)
# ---------------------------------------------------------------------------

def attn_rows(q, k, v, dout, cu_q, cu_kv, b, hq, rows, mask_type=None,
              cu_q_padded=None, cu_kv_padded=None, scale=None):
    """Output, log-sum-exp and dq of chosen query rows of sequence b, head hq.

    The same definitions as ``attn_fwd`` / ``attn_bwd`` evaluated one query row
    at a time: row i needs only its own scores against the sequence's keys, so
    large sequences can be checked on a sample.  ``rows`` are 0-based indices
    inside the sequence.  Returns (out [n, d], lse [n], dq [n, d]); dq is None
    when ``dout`` is None.
    """
    T_q, h_q, d = q.shape
    h_kv = k.shape[1]
    group = h_q // h_kv
    scale = _default_scale(d, scale)
    (oq, lq), = [sequence_rows(cu_q, b + 1, cu_q_padded)[b]]
    (ok, lk), = [sequence_rows(cu_kv, b + 1, cu_kv_padded)[b]]
    mt = _mask_type(mask_type, b)
    hk = hq // group
    K = np.asarray(k[ok:ok + lk, hk, :], dtype=np.float64)
    V = np.asarray(v[ok:ok + lk, hk, :], dtype=np.float64)
    outs, lses, dqs = [], [], []
    for i in rows:
        if not 0 <= i < lq:
            raise IndexError(i)
        qi = np.asarray(q[oq + i, hq, :], dtype=np.float64)
        # keys 0 .. n_vis-1 are visible to row i (visible_keys, one row)
        if mt == MASK_CAUSAL:
            n_vis = min(i + 1, lk)
        elif mt == MASK_CAUSAL_BOTTOM_RIGHT:
            n_vis = min(max(i + 1 + lk - lq, 0), lk)
        else:
            n_vis = lk
        if n_vis == 0:
            outs.append(np.zeros(d)); lses.append(-np.inf); dqs.append(np.zeros(d))
            continue
        s = scale * (K[:n_vis] @ qi)
        m = s.max()
        e = np.exp(s - m)
        p = e / e.sum()
        o = p @ V[:n_vis]
        outs.append(o)
        lses.append(m + np.log(e.sum()))
        if dout is not None:
            g = np.asarray(dout[oq + i, hq, :], dtype=np.float64)
            dp = V[:n_vis] @ g
            ds = p * (dp - (p * dp).sum())
            dqs.append(scale * (ds @ K[:n_vis]))
    dq = np.array(dqs) if dout is not None else None
    return np.array(outs), np.array(lses), dq


# ---------------------------------------------------------------------------
# Key/value gradients of a key range of one long sequence, by query-row blocks
# ---------------------------------------------------------------------------

def attn_bwd_key_range(q, k, v, dout, cu_q, cu_kv, b, hk, key_ranges, mask_type=None,
                       cu_q_padded=None, cu_kv_padded=None, scale=None, row_block=1024):
    """dK and dV of key ranges [lo, hi) of sequence b, kv head hk, summed over
    the query heads of hk's GQA group (the ``attn_bwd`` definitions).

    Key j's gradients are sums over query rows i: dV_j = sum_i P_ij dO_i and
    dK_j = scale sum_i dS_ij Q_i, with dS_ij = P_ij (dP_ij - D_i).  P_ij and
    D_i need the whole row i (its softmax normaliser and rowsum(P * dP)), so
    the rows are taken in blocks of at most ``row_block``: each block's scores
    against the keys its rows can see give its P and dP, and the block adds
    its terms for the chosen keys.  This bounds memory for sequences of tens of
    thousands of tokens.  Under a causal mask type no row of a block sees a
    key past its last row's diagonal, so those keys (whose P is exactly 0) are
    not formed.  ``key_ranges``: list of (lo, hi); returns a list of
    (dk, dv), each [hi - lo, d].
    """
    T_q, h_q, d = q.shape
    h_kv = k.shape[1]
    group = h_q // h_kv
    scale = _default_scale(d, scale)
    (oq, lq), = [sequence_rows(cu_q, b + 1, cu_q_padded)[b]]
    (ok, lk), = [sequence_rows(cu_kv, b + 1, cu_kv_padded)[b]]
    for lo, hi in key_ranges:
        if not 0 <= lo <= hi <= lk:
            raise IndexError((lo, hi, lk))
    mt = _mask_type(mask_type, b)
    off = lk - lq if mt == MASK_CAUSAL_BOTTOM_RIGHT else 0
    K = np.asarray(k[ok:ok + lk, hk, :], dtype=np.float64)
    V = np.asarray(v[ok:ok + lk, hk, :], dtype=np.float64)
    res = [(np.zeros((hi - lo, d)), np.zeros((hi - lo, d))) for lo, hi in key_ranges]
    for hq in range(hk * group, (hk + 1) * group):
        for r0 in range(0, lq, row_block):
            r1 = min(r0 + row_block, lq)
            # keys [0, n) can be visible to rows r0 .. r1-1
            n = lk if mt not in (MASK_CAUSAL, MASK_CAUSAL_BOTTOM_RIGHT) else \
                min(max(r1 + off, 0), lk)
            Q = np.asarray(q[oq + r0:oq + r1, hq, :], dtype=np.float64)
            dO = np.asarray(dout[oq + r0:oq + r1, hq, :], dtype=np.float64)
            # rows r0 .. r1-1 of visible_keys(lq, lk, mt), keys 0 .. n-1
            i = np.arange(r0, r1)[:, None]
            j = np.arange(n)[None, :]
            allowed = np.ones((r1 - r0, n), dtype=bool)
            if mt == MASK_CAUSAL:
                allowed &= j <= i
            elif mt == MASK_CAUSAL_BOTTOM_RIGHT:
                allowed &= j <= i + (lk - lq)
            has_key = allowed.any(axis=1)
            S = np.where(allowed, scale * (Q @ K[:n].T), -np.inf)
            m = np.where(has_key, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.where(allowed, np.exp(S - m[:, None]), 0.0)
            denom = E.sum(axis=1)
            P = np.divide(E, denom[:, None], out=np.zeros_like(E), where=has_key[:, None])
            dP = dO @ V[:n].T
            Drow = (P * dP).sum(axis=1)
            for (lo, hi), (dk, dv) in zip(key_ranges, res):
                a, z = min(lo, n), min(hi, n)        # keys past n: P = 0, no term
                if a == z:
                    continue
                Pr = P[:, a:z]
                dS = Pr * (dP[:, a:z] - Drow[:, None])
                dv[a - lo:z - lo] += Pr.T @ dO
                dk[a - lo:z - lo] += scale * (dS.T @ Q)
    return res


# ---------------------------------------------------------------------------
# Rounding to the 16-bit storage types
# ---------------------------------------------------------------------------

def round_to_storage(x, dtype):
    """x (any float array) rounded to nearest-even in "fp16" or "bf16" and
    returned as float64: the values a 16-bit tensor of that type holds.

    fp16 is numpy's half.  bf16 keeps the upper 16 bits of the IEEE binary32
    pattern: x is first rounded to binary32, then the lower 16 bits are
    rounded away to nearest, ties to even (add 0x7FFF plus the lowest kept
    bit, then truncate).  NaN is kept as a quiet NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    with np.errstate(over="ignore"):
        f = x.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    return np.where(np.isnan(x), np.nan, out)
