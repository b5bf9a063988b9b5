"""The whole path (both padding masks, forward, backward) captured in one HIP
graph and replayed.  No call synchronises or reads device data on the host
(TransformerEngine PR "[PyTorch] Build the attention padding mask without host
syncs", Description), which is what makes capture possible.  Every replay,
with eager work and synchronisations between replays, is checked against the
eager results: bit for bit, except dq, whose fp32 accumulation adds its
atomics in a different order on every run."""
import numpy as np
import pytest
import torch

import variable_length_packed_amd as thd
import workloads
from gpu_helpers import assert_close, dev_meta, f64

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    w = workloads.random_layout(140, batch=7, max_len=300, h_q=4, h_kv=2, d=128, dtype="bf16",
                                causal="mixed", slot_multiple=16)
    print(f"graph capture: T_q={w.T_q} batch={w.batch}", flush=True)
    q, k, v, do = (t.cuda() for t in workloads.make_tensors(w))
    m = dev_meta(w)
    o, lse = torch.empty_like(q), torch.empty((w.h_q, w.T_q), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = dict(cu_seqlens_q_padded=m["cu_seqlens_q_padded"],
              cu_seqlens_kv_padded=m["cu_seqlens_kv_padded"], is_causal=m["is_causal"],
              batch_size=w.batch)
    fws = torch.empty(max(thd.fwd_workspace_size(q, k, m["cu_seqlens_q"], m["cu_seqlens_kv"],
                                                 w.max_seqlen_q, w.max_seqlen_kv,
                                                 batch_size=w.batch), 1),
                      dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(thd.bwd_workspace_size(q, k, m["cu_seqlens_q"], m["cu_seqlens_kv"],
                                                 batch_size=w.batch), 1),
                      dtype=torch.uint8, device="cuda")

    def step():
        mq = thd.padding_mask(m["cu_seqlens_q"], w.batch, w.max_seqlen_q)
        mk = thd.padding_mask(m["cu_seqlens_kv"], w.batch, w.max_seqlen_kv)
        thd.attn_fwd(q, k, v, m["cu_seqlens_q"], m["cu_seqlens_kv"], w.max_seqlen_q,
                     w.max_seqlen_kv, out=o, lse=lse, workspace=fws, **kw)
        thd.attn_bwd(q, k, v, o, do, lse, m["cu_seqlens_q"], m["cu_seqlens_kv"], w.max_seqlen_q,
                     w.max_seqlen_kv, dq=dq, dk=dk, dv=dv, workspace=bws, **kw)
        return mq, mk

    ref_masks = [x.clone() for x in step()]
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        masks = step()
    torch.cuda.synchronize()

    for rep in range(3):
        for x in (o, dq, dk, dv):           # eager work between replays
            x.fill_(float("nan"))
        lse.fill_(123.0)
        for x in masks:
            x.fill_(rep % 2 == 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = lambda t: t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)
        for name, got, want in zip(("o", "lse", "dk", "dv"), (o, lse, dk, dv),
                                   (ref[0], ref[1], ref[3], ref[4])):
            assert torch.equal(bits(got), bits(want)), f"replay {rep}: {name} differs from eager"
        vq = np.asarray(w.row_is_valid_q(), bool)
        assert_close(f"replay {rep} dq", f64(dq)[vq], f64(ref[2])[vq], w.dtype)
        assert np.all(dq.view(torch.int16).cpu().numpy()[~vq] == 0)
        for got, want in zip(masks, ref_masks):
            assert torch.equal(got, want), f"replay {rep}: padding mask differs from eager"
