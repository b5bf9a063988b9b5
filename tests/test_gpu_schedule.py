"""GPU: the work schedules the forward and backward pre passes build on the
device, read back from their workspaces and compared with the order they are
defined to have.

Each schedule lists the (sequence, tile) items of its pass: query tiles of
128 rows for the forward and the backward's dq pass, key tiles of 128 or 256
keys for its dk/dv pass.  An item's work W is the number of key tiles (forward and
dq pass, BN keys each: 32 at d > 32, 64 at d <= 32) or 32-row query tiles
(dk/dv pass) it walks: all of them without a causal mask, else those up to
the diagonal (top-left, or shifted by lk - lq for bottom-right).  The order:
sequences by their largest item's work, largest first, ties in sequence
order; within a sequence, its items largest first.  Workspace layouts (sizes
from the library's own size queries): forward = the schedule; backward =
-D and -LSE/scale [2][h_q][T_q], then the dq pass's schedule, then the dk/dv
pass's, each part starting on a 256-byte boundary.  Schedule = int32
[count, 7 unused, then per rank 8 words: b, t, the sequence's query and key
slot starts, its query and key lengths, its mask type, unused].
Bit-exact comparison: the schedule is integer work.
"""
import numpy as np
import pytest
import torch

import variable_length_packed_amd as thd
import workloads
from gpu_helpers import dev_meta, gpu_fwd

pytestmark = pytest.mark.gpu


def ceil_div(a, b):
    return -((-a) // b)


def expected_schedule(lens_items, lens_walk, types, per_item, per_walk, slope):
    """(b, t) in schedule order.  lens_items: lengths cut into items of
    per_item rows; lens_walk: lengths walked in tiles of per_walk; slope: the
    change of W from one item to the next on a causal sequence."""
    seqs = []
    for b, (li, lw, mt) in enumerate(zip(lens_items, lens_walk, types)):
        x = ceil_div(int(li), per_item)
        H = ceil_div(int(lw), per_walk)
        causal = int(mt) in (1, 2)
        if causal:
            lq, lk = (li, lw) if slope > 0 else (lw, li)
            off = int(lk) - int(lq) if int(mt) == 2 else 0
            c = (slope if slope > 0 else H) + ceil_div(off, per_walk)
            work = [min(max(slope * t + c, 0), H) for t in range(x)]
        else:
            work = [H] * x
        top = max(work) if x else -1
        # the documented order within a sequence: descending t for a positive
        # causal slope, ascending otherwise (W is monotone in t)
        if causal and slope > 0:
            order = list(range(x - 1, -1, -1))
        else:
            order = list(range(x))
        assert [work[t] for t in order] == sorted(work, reverse=True)
        seqs.append((-top, b, [(b, t) for t in order]))
    out = []
    for _, _, items in sorted(seqs):
        out.extend(items)
    return out


HEADER, WORDS = 8, 8   # int32 words before the first item, and per item


def read_schedule(ws, offset, w=None, types=None):
    """(b, t) per rank.  With the workload, also checks each item's other
    fields: the sequence's slot starts, lengths and mask type."""
    a = ws[offset:].view(torch.int32).cpu().numpy()
    n = int(a[0])
    items = a[HEADER:HEADER + WORDS * n].reshape(n, WORDS) if n else np.zeros((0, WORDS), int)
    if w is not None:
        sq, sk = w.starts_q(), w.starts_kv()
        for rank, (b, t, s_q, s_k, l_q, l_k, mt, _) in enumerate(items.tolist()):
            assert (s_q, s_k, l_q, l_k, mt) == (int(sq[b]), int(sk[b]), int(w.lens_q[b]),
                                                int(w.lens_kv[b]), int(types[b])), rank
    return [(int(b), int(t)) for b, t in items[:, :2].tolist()]


def align256(x):
    return (x + 255) & ~255


CASES = [
    dict(seed=201, batch=9, max_len=700, h_q=2, d=128, causal="mixed"),
    dict(seed=202, batch=12, max_len=1100, h_q=4, h_kv=1, d=128, causal="all", min_len=0),
    dict(seed=203, batch=7, max_len=900, h_q=2, d=64, causal="types", cross=True,
         slot_multiple=64, gap_before=3, extra_cu=2),
    dict(seed=204, batch=10, max_len=500, h_q=2, d=32, causal="types", cross=True),
    dict(seed=205, batch=6, max_len=400, h_q=2, d=128, causal="none", extra_cu=3),
]


@pytest.mark.parametrize("kw", CASES, ids=[f"s{c['seed']}" for c in CASES])
def test_schedules_match_definition(kw):
    kw = dict(kw)
    seed = kw.pop("seed")
    w = workloads.random_layout(seed, dtype="bf16", **kw)
    print(f"case {w.name}: B={w.batch} Tq={w.T_q} Tkv={w.T_kv} h={w.h_q}/{w.h_kv} d={w.d}",
          flush=True)
    # the tiled forward, not the split-KV one (that needs few query rows)
    assert w.max_seqlen_q * (w.h_q // w.h_kv) > 32
    q, k, v, do = (t.cuda() for t in workloads.make_tensors(w))
    meta = dev_meta(w)
    types = np.asarray(w.causal)[:w.batch]

    need = thd.fwd_workspace_size(q, k, meta["cu_seqlens_q"], meta["cu_seqlens_kv"],
                                  w.max_seqlen_q, w.max_seqlen_kv, batch_size=w.batch)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    o, lse = gpu_fwd(w, q, k, v, meta, workspace=ws)
    torch.cuda.synchronize()
    bn = 32 if w.d > 32 else 64
    exp_f = expected_schedule(w.lens_q, w.lens_kv, types, 128, bn, 128 // bn)
    assert read_schedule(ws, 0, w, types) == exp_f

    need_b = thd.bwd_workspace_size(q, k, meta["cu_seqlens_q"], meta["cu_seqlens_kv"],
                                    batch_size=w.batch)
    ws_b = torch.full((need_b,), 0x7F, dtype=torch.uint8, device="cuda")
    thd.attn_bwd(q, k, v, o, do, lse, meta["cu_seqlens_q"], meta["cu_seqlens_kv"],
                 w.max_seqlen_q, w.max_seqlen_kv,
                 cu_seqlens_q_padded=meta["cu_seqlens_q_padded"],
                 cu_seqlens_kv_padded=meta["cu_seqlens_kv_padded"],
                 is_causal=meta["is_causal"], batch_size=w.batch, workspace=ws_b)
    torch.cuda.synchronize()
    off_q = align256(w.T_q * w.h_q * 2 * 4)
    n_qtiles = ceil_div(w.T_q, 128) + w.batch   # the dq pass's query-tile bound
    off_k = off_q + align256((HEADER + WORDS * n_qtiles) * 4)
    assert read_schedule(ws_b, off_q, w, types) == exp_f
    # key tiles of the dk/dv pass: 128 keys when max_seqlen_q times the GQA
    # group is at most 4096, else 256
    bk = 128 if w.max_seqlen_q * (w.h_q // w.h_kv) <= 4096 else 256
    exp_b = expected_schedule(w.lens_kv, w.lens_q, types, bk, 32, -(bk // 32))
    assert read_schedule(ws_b, off_k, w, types) == exp_b
