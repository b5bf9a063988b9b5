"""GPU: thd_attn_fwd_noalloc (the forward for callers that cannot allocate)
against thd_attn_fwd through the C ABI.  Both launch the same kernels, so the
outputs must agree bit for bit; the no-alloc calls run back to back on the
device's one scratch array, the later ones with smaller inputs than the
first (stale contents must not matter), and the split-KV path (few query rows
per sequence) keeps its partials there too."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import assert_close, assert_pad_rows_zero, f64
from oracle import attn_fwd
from variable_length_packed_amd import _lib
from variable_length_packed_amd.attention import _make_args, _ptr, _stream

pytestmark = pytest.mark.gpu


def _layouts():
    big = workloads.random_layout(301, batch=6, max_len=700, h_q=4, h_kv=2, d=128, dtype="bf16",
                                  causal="types", cross=True, slot_multiple=64, gap_before=2)
    small = workloads.random_layout(302, batch=3, max_len=150, h_q=4, h_kv=2, d=128,
                                    dtype="bf16", causal="mixed")
    rng = np.random.default_rng(303)   # few query rows per sequence: the split-KV path
    decode = workloads.packed(rng.integers(1, 3, size=5, endpoint=True),
                              rng.integers(0, 900, size=5, endpoint=True),
                              causal=np.array([2, 0, 1, 2, 2], np.uint8), h_q=8, h_kv=2, d=64,
                              dtype="fp16", seed=303, slot_multiple=16, name="dec303")
    assert decode.max_seqlen_q * 4 <= 32
    return [big, small, decode]


def _call(lib, w, q, k, v, no_alloc):
    dev = q.device
    t32 = lambda x: None if x is None else torch.from_numpy(np.asarray(x, np.int32)).to(dev)
    cu_q, cu_kv = t32(w.cu_q), t32(w.cu_kv)
    pad_q, pad_kv = t32(w.cu_q_padded), t32(w.cu_kv_padded)
    mt = torch.from_numpy(np.asarray(w.causal, np.uint8)).to(dev)
    a = _make_args(q, k, cu_q, cu_kv, w.max_seqlen_q, w.max_seqlen_kv, pad_q, pad_kv, mt,
                   None, w.batch)
    o = torch.full_like(q, 7.0)
    lse = torch.full((w.h_q, w.T_q), 7.0, dtype=torch.float32, device=dev)
    need = int(lib.thd_attn_fwd_workspace_size(a))
    assert 0 < need <= _lib.FWD_NOALLOC_MAX_WORKSPACE
    if no_alloc:
        st = lib.thd_attn_fwd_noalloc(a, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _stream(dev))
    else:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        st = lib.thd_attn_fwd(a, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), need,
                              _stream(dev))
    _lib.check(st, "noalloc" if no_alloc else "fwd")
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_forward_matches_forward_on_successive_calls():
    lib = _lib.load()
    for w in _layouts():
        print(f"case {w.name}: B={w.batch} Tq={w.T_q} Tkv={w.T_kv} max_q={w.max_seqlen_q}",
              flush=True)
        q, k, v, _ = (t.cuda() for t in workloads.make_tensors(w))
        o_ref, lse_ref = _call(lib, w, q, k, v, no_alloc=False)
        o, lse = _call(lib, w, q, k, v, no_alloc=True)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse, lse_ref)
        vq = w.row_is_valid_q()
        assert_pad_rows_zero("out", o, vq)
        args = (w.cu_q, w.cu_kv, w.batch, w.causal, w.cu_q_padded, w.cu_kv_padded)
        ro, _ = attn_fwd(f64(q), f64(k), f64(v), *args)
        assert_close("out", f64(o)[vq], ro[vq], w.dtype)
