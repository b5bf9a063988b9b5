"""Context parallelism, the share of one rank, on one GPU.

Megatron-LM issue "How to pad sequences that cannot be evenly split in context
parallelism (CP)?" (question and repro): a sequence split over n devices is
padded to a multiple of 2n and the pad is marked with ``cu_seqlens_padded``.
Here sequence b (valid length len_b) owns a global slot of P_b = 2n * C_b rows,
C_b = ceil(len_b / 2n), valid rows first; it is cut into 2n chunks of C_b rows
and rank r holds chunks r and 2n-1-r as one local slot.  Rank r's attention is
the log-sum-exp merge of one forward per rank t (the KV ring), each on the views
that ``thd_cp_layout`` describes; on one GPU every shard is local, so the ring's
send/recv is replaced by reading the peer's shard in place.

The backward of rank r is one attention backward per ring step on the same
views, with the merged output and log-sum-exp of its queries: the dq of the
steps add up to rank r's dq, and each step's dk / dv is rank r's contribution
to the shard of the rank whose keys it read (in a ring they travel back to that
rank, which sums what every rank sends).  Sums are fp32.  Up to 8 steps, the
merge and the sums read every step's result once (thd_attn_lse_merge_n,
thd_sum_n); beyond that they go through an fp32 accumulator step by step.

Everything here is argument marshalling; the layout, the gather, the attention
steps, the merge and the sums run in libthdattn.so.
"""
import ctypes

import torch

from . import _lib
from .attention import _ptr, _require_cuda, _stream, attn_bwd, attn_fwd

SIDE_Q = 0
SIDE_KV = 1

_DECLARED = set()


def _lib_cp():
    lib = _lib.load()
    if id(lib) not in _DECLARED:
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.thd_cp_layout.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        lib.thd_cp_layout.restype = ctypes.c_int
        lib.thd_cp_gather.argtypes = [vp, vp, vp, i32, i32, i32, vp, i64, vp, i64, i32, vp]
        lib.thd_cp_gather.restype = ctypes.c_int
        lib.thd_attn_lse_merge.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp]
        lib.thd_attn_lse_merge.restype = ctypes.c_int
        lib.thd_accumulate.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        lib.thd_accumulate.restype = ctypes.c_int
        lib.thd_attn_lse_merge_n.argtypes = [vp, vp, i32, vp, vp, i64, i32, i32, i32, vp]
        lib.thd_attn_lse_merge_n.restype = ctypes.c_int
        lib.thd_sum_n.argtypes = [vp, i32, vp, i64, i32, vp]
        lib.thd_sum_n.restype = ctypes.c_int
        _DECLARED.add(id(lib))
    return lib


def _opt(t):
    return None if t is None else _ptr(t)


def cp_layout(cu_seqlens, cp_size, rank, peer, side, *, mask_type=None, batch_size=None):
    """Device metadata of one step's view (see thd_cp_layout in thd_attn.h).

    Returns a dict of int32 tensors ``cu_seqlens``, ``cu_seqlens_padded``,
    ``global_cu_seqlens_padded`` ([batch+1] each) and uint8 ``mask_type``
    ([batch]).
    """
    _require_cuda("cu_seqlens", cu_seqlens, torch.int32)
    b = cu_seqlens.numel() - 1 if batch_size is None else int(batch_size)
    if mask_type is not None:
        _require_cuda("mask_type", mask_type, torch.uint8)
    dev = cu_seqlens.device
    out = {k: torch.empty(b + 1, dtype=torch.int32, device=dev)
           for k in ("cu_seqlens", "cu_seqlens_padded", "global_cu_seqlens_padded")}
    out["mask_type"] = torch.empty(max(b, 1), dtype=torch.uint8, device=dev)
    st = _lib_cp().thd_cp_layout(_ptr(cu_seqlens), _opt(mask_type), b, cp_size, rank, peer, side,
                                 _ptr(out["cu_seqlens"]), _ptr(out["cu_seqlens_padded"]),
                                 _ptr(out["global_cu_seqlens_padded"]), _ptr(out["mask_type"]),
                                 _stream(dev))
    _lib.check(st, "thd_cp_layout")
    return out


def cp_shard(x, cu_seqlens, cp_size, rank, total_local, *, batch_size=None, out=None):
    """Rank ``rank``'s shard [total_local, ...] of ``x`` [T_padded, ...] (global
    padded layout); ``total_local`` = T_padded / cp_size."""
    _require_cuda("x", x)
    own = cp_layout(cu_seqlens, cp_size, rank, rank, SIDE_Q, batch_size=batch_size)
    b = cu_seqlens.numel() - 1 if batch_size is None else int(batch_size)
    if out is None:
        out = torch.zeros((total_local,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    row_bytes = x[0].numel() * x.element_size() if x.shape[0] else out[0].numel() * out.element_size()
    st = _lib_cp().thd_cp_gather(_ptr(cu_seqlens), _ptr(own["cu_seqlens_padded"]),
                                 _ptr(own["global_cu_seqlens_padded"]), b, cp_size, rank, _ptr(x),
                                 x.shape[0], _ptr(out), total_local, row_bytes, _stream(x.device))
    _lib.check(st, "thd_cp_gather")
    return out


def lse_merge(o_part, lse_part, o_acc, lse_acc, *, first, o_out=None):
    """Fold (o_part, lse_part) into the fp32 accumulator (o_acc, lse_acc) in place."""
    _require_cuda("o_part", o_part)
    _require_cuda("o_acc", o_acc, torch.float32)
    _require_cuda("lse_part", lse_part, torch.float32)
    _require_cuda("lse_acc", lse_acc, torch.float32)
    total, h, d = o_part.shape
    dt = _lib.THD_BF16 if o_part.dtype == torch.bfloat16 else _lib.THD_FP16
    st = _lib_cp().thd_attn_lse_merge(_ptr(o_part), _ptr(lse_part), _ptr(o_acc), _ptr(lse_acc),
                                      _opt(o_out), total, h, d, dt, int(bool(first)),
                                      _stream(o_part.device))
    _lib.check(st, "thd_attn_lse_merge")


MAX_PARTS = 8  # partials one thd_attn_lse_merge_n / thd_sum_n call takes


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def lse_merge_n(o_parts, lse_parts, *, out=None, lse_out=None):
    """One-pass log-sum-exp merge of up to 8 partial outputs (storage dtype)
    and their lse ([h, total] fp32); returns (out, lse_out)."""
    n = len(o_parts)
    if not 1 <= n <= MAX_PARTS or len(lse_parts) != n:
        raise ValueError("lse_merge_n: 1..8 partials, one lse each")
    for t in o_parts:
        _require_cuda("o_part", t, o_parts[0].dtype)
    for t in lse_parts:
        _require_cuda("lse_part", t, torch.float32)
    total, h, d = o_parts[0].shape
    out = torch.empty_like(o_parts[0]) if out is None else out
    lse_out = (torch.empty((h, total), dtype=torch.float32, device=out.device)
               if lse_out is None else lse_out)
    dt = _lib.THD_BF16 if out.dtype == torch.bfloat16 else _lib.THD_FP16
    st = _lib_cp().thd_attn_lse_merge_n(_ptr_array(o_parts), _ptr_array(lse_parts), n, _ptr(out),
                                        _ptr(lse_out), total, h, d, dt, _stream(out.device))
    _lib.check(st, "thd_attn_lse_merge_n")
    return out, lse_out


def sum_n(parts, *, out=None):
    """One-pass fp32 sum of up to 8 same-shaped tensors, in their dtype."""
    n = len(parts)
    if not 1 <= n <= MAX_PARTS:
        raise ValueError("sum_n: 1..8 partials")
    for t in parts:
        _require_cuda("part", t, parts[0].dtype)
        if t.numel() != parts[0].numel():
            raise ValueError("sum_n: sizes differ")
    out = torch.empty_like(parts[0]) if out is None else out
    dt = _lib.THD_BF16 if out.dtype == torch.bfloat16 else _lib.THD_FP16
    st = _lib_cp().thd_sum_n(_ptr_array(parts), n, _ptr(out), out.numel(), dt, _stream(out.device))
    _lib.check(st, "thd_sum_n")
    return out


def cp_views(cu_seqlens, cp_size, rank, *, mask_type=None, batch_size=None):
    """The (query view, key view) of every ring step of rank ``rank``, in ring
    order (step s reads the keys of rank (rank - s) mod cp_size)."""
    n = int(cp_size)
    out = []
    for s in range(n):
        t = (rank - s) % n
        out.append((t, cp_layout(cu_seqlens, n, rank, t, SIDE_Q, mask_type=mask_type,
                                 batch_size=batch_size),
                    cp_layout(cu_seqlens, n, rank, t, SIDE_KV, mask_type=mask_type,
                              batch_size=batch_size)))
    return out


def cp_attn_fwd(q_local, k_shards, v_shards, cu_seqlens, cp_size, rank, max_seqlen, *,
                mask_type=None, softmax_scale=None, batch_size=None, views=None):
    """Rank ``rank``'s attention output over its local queries.

    ``q_local``: its query shard; ``k_shards`` / ``v_shards``: the key and value
    shards of every rank (index = rank).  ``max_seqlen``: bound on the global
    valid lengths.  Returns (out [T_local, h_q, d], lse [h_q, T_local] fp32).
    """
    n = int(cp_size)
    b = cu_seqlens.numel() - 1 if batch_size is None else int(batch_size)
    max_local = 2 * ((int(max_seqlen) + 2 * n - 1) // (2 * n))
    T, hq, d = q_local.shape
    views = views or cp_views(cu_seqlens, n, rank, mask_type=mask_type, batch_size=b)
    if n <= MAX_PARTS:
        # every step's output kept, then merged in one pass
        outs, lses = [], []
        for t, vq, vk in views:
            o_s, l_s = attn_fwd(q_local, k_shards[t], v_shards[t], vq["cu_seqlens"],
                                vk["cu_seqlens"], max_local, max_local,
                                cu_seqlens_q_padded=vq["cu_seqlens_padded"],
                                cu_seqlens_kv_padded=vk["cu_seqlens_padded"],
                                mask_type=vq["mask_type"][:b], softmax_scale=softmax_scale,
                                batch_size=b)
            outs.append(o_s)
            lses.append(l_s)
        return lse_merge_n(outs, lses)
    o_acc = torch.empty((T, hq, d), dtype=torch.float32, device=q_local.device)
    lse_acc = torch.empty((hq, T), dtype=torch.float32, device=q_local.device)
    out = torch.empty_like(q_local)
    o_step = torch.empty_like(q_local)
    lse_step = torch.empty((hq, T), dtype=torch.float32, device=q_local.device)
    for s, (t, vq, vk) in enumerate(views):
        attn_fwd(q_local, k_shards[t], v_shards[t], vq["cu_seqlens"], vk["cu_seqlens"],
                 max_local, max_local, cu_seqlens_q_padded=vq["cu_seqlens_padded"],
                 cu_seqlens_kv_padded=vk["cu_seqlens_padded"], mask_type=vq["mask_type"][:b],
                 softmax_scale=softmax_scale, batch_size=b, out=o_step, lse=lse_step)
        lse_merge(o_step, lse_step, o_acc, lse_acc, first=(s == 0),
                  o_out=out if s == n - 1 else None)
    return out, lse_acc


def accumulate(src, acc, *, first, out=None):
    """acc (+)= src in fp32 (first: =); out, if given, receives the sum in src's dtype."""
    _require_cuda("src", src)
    _require_cuda("acc", acc, torch.float32)
    if acc.numel() != src.numel() or (out is not None and out.numel() != src.numel()):
        raise ValueError("accumulate: sizes differ")
    dt = _lib.THD_BF16 if src.dtype == torch.bfloat16 else _lib.THD_FP16
    st = _lib_cp().thd_accumulate(_ptr(src), _ptr(acc), _opt(out), src.numel(), dt,
                                  int(bool(first)), _stream(src.device))
    _lib.check(st, "thd_accumulate")


def cp_attn_bwd(q_local, k_shards, v_shards, out_local, dout_local, lse_local, cu_seqlens,
                cp_size, rank, max_seqlen, *, mask_type=None, softmax_scale=None,
                batch_size=None, views=None):
    """Rank ``rank``'s backward.  ``out_local`` / ``lse_local``: its merged
    forward outputs (``cp_attn_fwd``).  Returns (dq [T_local, h_q, d], parts):
    parts[t] = (dk, dv) of rank t's key shard contributed by this rank's
    queries, in the storage dtype (the shard's owner sums them with
    ``cp_reduce``)."""
    n = int(cp_size)
    b = cu_seqlens.numel() - 1 if batch_size is None else int(batch_size)
    max_local = 2 * ((int(max_seqlen) + 2 * n - 1) // (2 * n))
    parts = [None] * n
    dqs = []
    views = views or cp_views(cu_seqlens, n, rank, mask_type=mask_type, batch_size=b)
    for s, (t, vq, vk) in enumerate(views):
        dq_s, dk_s, dv_s = attn_bwd(
            q_local, k_shards[t], v_shards[t], out_local, dout_local, lse_local,
            vq["cu_seqlens"], vk["cu_seqlens"], max_local, max_local,
            cu_seqlens_q_padded=vq["cu_seqlens_padded"], cu_seqlens_kv_padded=vk["cu_seqlens_padded"],
            mask_type=vq["mask_type"][:b], softmax_scale=softmax_scale, batch_size=b)
        dqs.append(dq_s)
        parts[t] = (dk_s, dv_s)
    if n <= MAX_PARTS:
        return sum_n(dqs), parts
    dq_acc = torch.empty(q_local.shape, dtype=torch.float32, device=q_local.device)
    dq = torch.empty_like(q_local)
    for s, dq_s in enumerate(dqs):
        accumulate(dq_s, dq_acc, first=(s == 0), out=dq if s == n - 1 else None)
    return dq, parts


def cp_reduce(parts):
    """Sum of the contributions to one shard (a list of same-shaped tensors) in
    fp32, returned in their dtype."""
    if len(parts) <= MAX_PARTS:
        return sum_n(list(parts))
    acc = torch.empty(parts[0].shape, dtype=torch.float32, device=parts[0].device)
    out = torch.empty_like(parts[0])
    for i, p in enumerate(parts):
        accumulate(p, acc, first=(i == 0), out=out if i == len(parts) - 1 else None)
    return out
