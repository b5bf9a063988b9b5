"""Pins for the oracle's attention forward and backward (CPU only).

Each test ties the oracle to something outside itself: numbers printed on the
pages, the maintainer's two-call decomposition with the page's own arrays,
closed forms, an independent library routine (torch's scaled_dot_product_attention
and autograd on CPU in float64), central finite differences, and invariants
that any correct softmax attention satisfies.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import attn_bwd, attn_fwd, valid_pairs, sequence_rows

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f64(t):
    return t.to(torch.float64).numpy()


def fwd_w(w, q, k, v, **kw):
    return attn_fwd(f64(q), f64(k), f64(v), w.cu_q, w.cu_kv, w.batch, w.causal,
                    w.cu_q_padded, w.cu_kv_padded, **kw)


def bwd_w(w, q, k, v, do, **kw):
    return attn_bwd(f64(q), f64(k), f64(v), f64(do), w.cu_q, w.cu_kv, w.batch,
                    w.causal, w.cu_q_padded, w.cu_kv_padded, **kw)


# ---------------------------------------------------------------------------
# The issue's printed reference output
# ---------------------------------------------------------------------------

def test_seven_token_example_matches_printed_output():
    g = json.load(open(os.path.join(GOLD, "seven_token_example.json")))
    w = workloads.config("1b")
    q, k, v, _ = workloads.make_tensors(w)
    out, lse = fwd_w(w, q, k, v)
    o16 = out.astype(np.float16)
    fmt = "%.{}f".format(g["printed_decimals"])
    for r in range(4):
        assert {fmt % x for x in o16[r, 0]} == {g["rows_0_3"]}
    for r in range(4, 7):
        assert {fmt % x for x in o16[r, 0]} == {g["rows_4_6"]}
    # pad row: output exactly +0
    assert np.all(out[7] == 0) and not np.any(np.signbit(out[7]))
    assert lse[0, 7] == -np.inf
    # pad value and an explicit cu_seqlens_padded change nothing
    q2, k2, v2 = (t.clone() for t in (q, k, v))
    for t in (q2, k2, v2):
        t[7] = 0.0
    out2, _ = fwd_w(w, q2, k2, v2)
    np.testing.assert_array_equal(out, out2)
    out3, _ = attn_fwd(f64(q), f64(k), f64(v), w.cu_q, w.cu_kv, 1, [0],
                       np.array([0, 8], np.int32), np.array([0, 8], np.int32))
    np.testing.assert_array_equal(out, out3)


def test_seven_token_example_pins_default_scale():
    # Only 1/sqrt(d) reproduces the printed values; 1 and 1/d do not.
    w = workloads.config("1b")
    q, k, v, _ = workloads.make_tensors(w)
    out_default, _ = fwd_w(w, q, k, v)
    out_explicit, _ = fwd_w(w, q, k, v, scale=1.0 / math.sqrt(8))
    np.testing.assert_array_equal(out_default, out_explicit)
    for wrong in (1.0, 1.0 / 8):
        o, _ = fwd_w(w, q, k, v, scale=wrong)
        assert "%.4f" % np.float16(o[0, 0, 0]) != "1.9268"
    # closed form of the example: row of value a attends 4 ones and 3 twos
    d, s = 8, 1 / math.sqrt(8)
    for a, row in ((1.0, 0), (2.0, 5)):
        e1, e2 = math.exp(s * a * 1 * d), math.exp(s * a * 2 * d)
        ref = (4 * e1 * 1 + 3 * e2 * 2) / (4 * e1 + 3 * e2)
        assert abs(out_default[row, 0, 0] - ref) < 1e-12


def test_pad_tokens_leak_would_be_visible():
    # If the pad token (100) were attended, outputs would be ~100.
    w = workloads.config("1b")
    q, k, v, _ = workloads.make_tensors(w)
    leak, _ = attn_fwd(f64(q), f64(k), f64(v), np.array([0, 8], np.int32),
                       np.array([0, 8], np.int32), 1, [0])
    assert leak[0, 0, 0] > 50
    out, _ = fwd_w(w, q, k, v)
    assert out[0, 0, 0] < 2.5


# ---------------------------------------------------------------------------
# The maintainer's two-call example with the page's arrays
# ---------------------------------------------------------------------------

def _two_call():
    g = json.load(open(os.path.join(GOLD, "two_call_example.json")))
    w = workloads.config("1a")
    assert list(w.lens_q) == g["lengths"] and list(w.causal) == g["is_causal"]
    assert w.T_q == g["total_tokens"]
    return g, w


def test_mixed_call_equals_two_call_sum_forward():
    g, w = _two_call()
    q, k, v, _ = workloads.make_tensors(w)
    mixed, _ = fwd_w(w, q, k, v)
    parts = []
    for key, causal in (("causal_call", 1), ("full_call", 0)):
        c = g[key]
        cu = np.array(c["cu_seqlens"], np.int32)
        pad = np.array(c["cu_seqlens_padded"], np.int32)
        n = len(cu) - 1
        o, _ = attn_fwd(f64(q), f64(k), f64(v), cu, cu, n, [causal] * n, pad, pad)
        parts.append(o)
    summed = parts[0] + parts[1]
    np.testing.assert_allclose(mixed, summed, rtol=0, atol=1e-15)
    # each call's output is zero outside its own sequences
    assert np.all(parts[0][3:6] == 0) and np.all(parts[1][0:3] == 0)


def test_mixed_call_equals_two_call_sum_backward():
    g, w = _two_call()
    q, k, v, do = workloads.make_tensors(w)
    mixed = bwd_w(w, q, k, v, do)
    acc = [np.zeros_like(x) for x in mixed]
    for key, causal in (("causal_call", 1), ("full_call", 0)):
        c = g[key]
        cu = np.array(c["cu_seqlens"], np.int32)
        pad = np.array(c["cu_seqlens_padded"], np.int32)
        n = len(cu) - 1
        grads = attn_bwd(f64(q), f64(k), f64(v), f64(do), cu, cu, n,
                         [causal] * n, pad, pad)
        for a, gr in zip(acc, grads):
            a += gr
    for m, a in zip(mixed, acc):
        np.testing.assert_allclose(m, a, rtol=0, atol=1e-14)


def test_mixed_call_equals_each_sequence_alone():
    g, w = _two_call()
    q, k, v, do = workloads.make_tensors(w)
    mixed, _ = fwd_w(w, q, k, v)
    dmixed = bwd_w(w, q, k, v, do)
    for b, (s, n) in enumerate(sequence_rows(w.cu_q, w.batch)):
        cu = np.array([0, n], np.int32)
        sl = slice(s, s + n)
        o, _ = attn_fwd(f64(q[sl]), f64(k[sl]), f64(v[sl]), cu, cu, 1, [w.causal[b]])
        np.testing.assert_allclose(mixed[sl], o, rtol=0, atol=1e-15)
        grads = attn_bwd(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), cu, cu,
                         1, [w.causal[b]])
        for full, alone in zip(dmixed, grads):
            np.testing.assert_allclose(full[sl], alone, rtol=0, atol=1e-14)


def test_valid_pair_count_of_two_call_layout():
    _, w = _two_call()
    assert valid_pairs(w.cu_q, w.cu_kv, w.batch, w.causal) == 18 + 29


# ---------------------------------------------------------------------------
# Independent library routine: torch SDPA / autograd on CPU in float64
# ---------------------------------------------------------------------------

def _torch_reference(w, q, k, v, do):
    """Per-sequence torch SDPA (float64, CPU) with autograd."""
    q = q.to(torch.float64).clone().requires_grad_(True)
    k = k.to(torch.float64).clone().requires_grad_(True)
    v = v.to(torch.float64).clone().requires_grad_(True)
    out = torch.zeros_like(q)
    group = w.h_q // w.h_kv
    rq = sequence_rows(w.cu_q, w.batch, w.cu_q_padded)
    rk = sequence_rows(w.cu_kv, w.batch, w.cu_kv_padded)
    pieces = []
    for b in range(w.batch):
        (oq, lq), (ok, lk) = rq[b], rk[b]
        if lq == 0 or lk == 0:
            continue
        Q = q[oq:oq + lq].transpose(0, 1)
        K = k[ok:ok + lk].repeat_interleave(group, dim=1).transpose(0, 1)
        V = v[ok:ok + lk].repeat_interleave(group, dim=1).transpose(0, 1)
        if w.causal[b]:
            mask = torch.ones(lq, lk, dtype=torch.bool).tril()
            o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        else:
            o = torch.nn.functional.scaled_dot_product_attention(Q, K, V)
        pieces.append((oq, lq, o.transpose(0, 1)))
    for oq, lq, o in pieces:
        out = out.index_put((torch.arange(oq, oq + lq),), o)
    (out * do.to(torch.float64)).sum().backward()
    return out.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("seed,kw", [
    (11, dict(batch=5, max_len=9, h_q=2, d=16, causal="mixed")),
    (12, dict(batch=4, max_len=12, h_q=4, h_kv=2, d=8, causal="all")),
    (13, dict(batch=3, max_len=7, h_q=3, h_kv=1, d=8, causal="none", cross=True)),
    (14, dict(batch=6, max_len=10, h_q=2, d=8, causal="mixed", slot_multiple=4,
              gap_before=3, min_len=1)),
    (15, dict(batch=4, max_len=11, h_q=2, d=8, causal="all", cross=True, min_len=1)),
])
def test_against_torch_sdpa_and_autograd(seed, kw):
    w = workloads.random_layout(seed, dtype="fp16", **kw)
    q, k, v, do = workloads.make_tensors(w)
    out, _ = fwd_w(w, q, k, v)
    dq, dk, dv = bwd_w(w, q, k, v, do)
    r_out, r_dq, r_dk, r_dv = _torch_reference(w, q, k, v, do)
    for a, b in ((out, r_out), (dq, r_dq), (dk, r_dk), (dv, r_dv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_equal_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(0)
    L, d = 6, 4
    q = rng.standard_normal((L, 1, d))
    k = np.tile(rng.standard_normal((1, 1, d)), (L, 1, 1))
    v = rng.standard_normal((L, 1, d))
    cu = np.array([0, L], np.int32)
    full, _ = attn_fwd(q, k, v, cu, cu, 1, [0])
    causal, _ = attn_fwd(q, k, v, cu, cu, 1, [1])
    for i in range(L):
        np.testing.assert_allclose(full[i, 0], v[:, 0].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(causal[i, 0], v[:i + 1, 0].mean(axis=0), atol=1e-14)


def test_length_one_and_causal_first_row():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 2, 8))
    k = rng.standard_normal((5, 2, 8))
    v = rng.standard_normal((5, 2, 8))
    cu = np.array([0, 1, 5], np.int32)
    out, lse = attn_fwd(q, k, v, cu, cu, 2, [0, 1])
    np.testing.assert_allclose(out[0], v[0], atol=1e-15)      # length 1
    np.testing.assert_allclose(out[1], v[1], atol=1e-15)      # causal row 0
    # lse of a single visible key is its scaled score
    s = 1 / math.sqrt(8)
    assert abs(lse[0, 0] - s * q[0, 0] @ k[0, 0]) < 1e-13


def test_empty_kv_and_empty_batch():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 1, 8))
    k = rng.standard_normal((2, 1, 8))
    out, lse = attn_fwd(q, k, k, np.array([0, 3], np.int32), np.array([0, 0], np.int32), 1)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    dq, dk, dv = attn_bwd(q, k, k, q, np.array([0, 3], np.int32),
                          np.array([0, 0], np.int32), 1)
    assert not dq.any() and not dk.any() and not dv.any()
    out, lse = attn_fwd(q, k, k, np.array([0], np.int32), np.array([0], np.int32), 0)
    assert not out.any()


# ---------------------------------------------------------------------------
# Backward: finite differences and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed,cross", [(21, False), (22, True)])
def test_backward_central_differences(seed, cross):
    w = workloads.random_layout(seed, batch=3, max_len=5, h_q=2, h_kv=1, d=4,
                                dtype="fp16", causal="mixed", cross=cross,
                                min_len=1, slot_multiple=2 if not cross else None)
    q, k, v, do = (f64(t) for t in workloads.make_tensors(w))
    args = (w.cu_q, w.cu_kv, w.batch, w.causal, w.cu_q_padded, w.cu_kv_padded)

    def loss(qq, kk, vv):
        o, _ = attn_fwd(qq, kk, vv, *args)
        return float((o * do).sum())

    grads = attn_bwd(q, k, v, do, *args)
    eps = 1e-6
    for idx, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp = x.copy(); xp[pos] += eps
            xm = x.copy(); xm[pos] -= eps
            ins_p = [q, k, v]; ins_p[idx] = xp
            ins_m = [q, k, v]; ins_m[idx] = xm
            num[pos] = (loss(*ins_p) - loss(*ins_m)) / (2 * eps)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(g), 1e-30)
        assert err < 1e-7, (idx, err)


def test_backward_invariants():
    w = workloads.random_layout(31, batch=4, max_len=16, h_q=4, h_kv=2, d=8,
                                dtype="bf16", causal="mixed", min_len=1)
    q, k, v, do = workloads.make_tensors(w)
    dq, dk, dv = bwd_w(w, q, k, v, do)
    do64 = f64(do)
    for (s, n) in sequence_rows(w.cu_q, w.batch):
        for hk in range(w.h_kv):
            heads = range(hk * 2, hk * 2 + 2)
            # P rows sum to one: sum_j dV_j = sum_i dO_i over the group
            np.testing.assert_allclose(dv[s:s + n, hk].sum(axis=0),
                                       do64[s:s + n, list(heads)].sum(axis=(0, 1)),
                                       atol=1e-12)
            # rows of dS sum to zero: sum_j dK_j = 0
            np.testing.assert_allclose(dk[s:s + n, hk].sum(axis=0), 0, atol=1e-12)


def test_gqa_equals_repeated_kv_heads():
    w = workloads.random_layout(41, batch=3, max_len=9, h_q=6, h_kv=2, d=8,
                                dtype="bf16", causal="mixed", min_len=1)
    q, k, v, do = workloads.make_tensors(w)
    out, lse = fwd_w(w, q, k, v)
    grads = bwd_w(w, q, k, v, do)
    kr, vr = (t.repeat_interleave(3, dim=1) for t in (k, v))
    w_mha = workloads.packed(w.lens_q, None, w.causal, h_q=6, d=8)
    out2, lse2 = fwd_w(w_mha, q, kr, vr)
    np.testing.assert_array_equal(out, out2)
    g2 = bwd_w(w_mha, q, kr, vr, do)
    np.testing.assert_allclose(grads[0], g2[0], atol=1e-15)
    np.testing.assert_allclose(grads[1], g2[1].reshape(w.T_kv, 2, 3, 8).sum(2), atol=1e-13)
    np.testing.assert_allclose(grads[2], g2[2].reshape(w.T_kv, 2, 3, 8).sum(2), atol=1e-13)


def test_pad_garbage_does_not_change_valid_outputs():
    w = workloads.random_layout(51, batch=5, max_len=8, h_q=2, d=8, dtype="bf16",
                                causal="mixed", slot_multiple=4, gap_before=2)
    q, k, v, do = workloads.make_tensors(w)
    base = fwd_w(w, q, k, v)[0], bwd_w(w, q, k, v, do)
    vq = torch.from_numpy(w.row_is_valid_q())
    for garbage in (0.0, -3e4):
        q2, k2, v2, do2 = (t.clone() for t in (q, k, v, do))
        for t in (q2, k2, v2, do2):
            t[~vq] = garbage
        o = fwd_w(w, q2, k2, v2)[0]
        np.testing.assert_array_equal(o, base[0])
        for a, b in zip(bwd_w(w, q2, k2, v2, do2), base[1]):
            np.testing.assert_array_equal(a, b)
    # pad rows of every output are exactly +0
    inv = ~w.row_is_valid_q()
    assert np.all(base[0][inv] == 0) and not np.signbit(base[0][inv]).any()
    for g in base[1]:
        assert np.all(g[inv] == 0) and not np.signbit(g[inv]).any()


def test_valid_pairs_closed_form():
    w = workloads.config("2")
    L = w.lens_q.astype(np.int64)
    assert valid_pairs(w.cu_q, w.cu_kv, w.batch, w.causal) == int((L * (L + 1) // 2).sum())
    w5 = workloads.config("5")
    assert valid_pairs(w5.cu_q, w5.cu_kv, w5.batch, w5.causal) == \
        int((w5.lens_q * w5.lens_kv).sum())


def test_row_sampled_oracle_matches_whole_sequence_oracle():
    from oracle import attn_rows
    w = workloads.random_layout(61, batch=4, max_len=20, h_q=4, h_kv=2, d=8,
                                dtype="bf16", causal="mixed", cross=True, min_len=0,
                                extra_cu=2)
    q, k, v, do = (f64(t) for t in workloads.make_tensors(w))
    out, lse = attn_fwd(q, k, v, w.cu_q, w.cu_kv, w.batch, w.causal)
    dq, _, _ = attn_bwd(q, k, v, do, w.cu_q, w.cu_kv, w.batch, w.causal)
    for b, (s, n) in enumerate(sequence_rows(w.cu_q, w.batch)):
        for hq in range(w.h_q):
            rows = list(range(n))
            o_r, l_r, dq_r = attn_rows(q, k, v, do, w.cu_q, w.cu_kv, b, hq, rows, w.causal)
            if n == 0:
                continue
            np.testing.assert_allclose(o_r, out[s:s + n, hq], atol=1e-13)
            np.testing.assert_allclose(l_r, lse[hq, s:s + n], atol=1e-13)
            np.testing.assert_allclose(dq_r, dq[s:s + n, hq], atol=1e-13)


# ---------------------------------------------------------------------------
# Bottom-right causal alignment (the third per-sequence mask type of the
# maintainer's proposal in "Add per-sequence causal policy to packed THD
# attention"): each case reduces to the top-left or full attention above.
# ---------------------------------------------------------------------------

def _one_seq(q, k, v, do, mt):
    cq = np.array([0, q.shape[0]], np.int32)
    ck = np.array([0, k.shape[0]], np.int32)
    out, lse = attn_fwd(q, k, v, cq, ck, 1, [mt])
    grads = attn_bwd(q, k, v, do, cq, ck, 1, [mt])
    return out, lse, grads


@pytest.mark.parametrize("lq,lk", [(5, 9), (1, 7), (3, 3)])
def test_bottom_right_is_top_left_with_queries_prepended(lq, lk):
    # lk >= lq: query i sees keys 0 .. i + lk - lq, which is what query
    # i + lk - lq sees under top-left alignment when lk - lq extra queries
    # come first.  Extra queries get dO = 0, so dK and dV agree as well.
    rng = np.random.default_rng(lq * 31 + lk)
    q = rng.standard_normal((lq, 2, 8))
    extra = rng.standard_normal((lk - lq, 2, 8))
    k = rng.standard_normal((lk, 1, 8))
    v = rng.standard_normal((lk, 1, 8))
    do = rng.standard_normal((lq, 2, 8))
    out, lse, (dq, dk, dv) = _one_seq(q, k, v, do, 2)
    qx = np.concatenate([extra, q])
    dox = np.concatenate([np.zeros_like(extra), do])
    out_t, lse_t, (dq_t, dk_t, dv_t) = _one_seq(qx, k, v, dox, 1)
    np.testing.assert_allclose(out, out_t[lk - lq:], atol=1e-13)
    np.testing.assert_allclose(lse, lse_t[:, lk - lq:], atol=1e-13)
    np.testing.assert_allclose(dq, dq_t[lk - lq:], atol=1e-13)
    np.testing.assert_allclose(dk, dk_t, atol=1e-13)
    np.testing.assert_allclose(dv, dv_t, atol=1e-13)


@pytest.mark.parametrize("lq,lk", [(9, 5), (4, 1)])
def test_bottom_right_with_more_queries_than_keys(lq, lk):
    # lq > lk: the first lq - lk queries see no key (output 0, log-sum-exp
    # -inf, no gradient); the rest are the top-left causal attention of the
    # last lk queries.
    rng = np.random.default_rng(lq * 7 + lk)
    q = rng.standard_normal((lq, 2, 8))
    k = rng.standard_normal((lk, 2, 8))
    v = rng.standard_normal((lk, 2, 8))
    do = rng.standard_normal((lq, 2, 8))
    out, lse, (dq, dk, dv) = _one_seq(q, k, v, do, 2)
    n0 = lq - lk
    assert not out[:n0].any() and not dq[:n0].any()
    assert np.all(np.isneginf(lse[:, :n0]))
    out_t, lse_t, (dq_t, dk_t, dv_t) = _one_seq(q[n0:], k, v, do[n0:], 1)
    np.testing.assert_allclose(out[n0:], out_t, atol=1e-13)
    np.testing.assert_allclose(lse[:, n0:], lse_t, atol=1e-13)
    np.testing.assert_allclose(dq[n0:], dq_t, atol=1e-13)
    np.testing.assert_allclose(dk, dk_t, atol=1e-13)
    np.testing.assert_allclose(dv, dv_t, atol=1e-13)


def test_bottom_right_single_query_sees_every_key():
    # one query against a long kv sequence (the decode shape): bottom-right
    # causal leaves every key visible, so it equals `padding`, while top-left
    # causal would show it only key 0.
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((6, 1, 8))
    v = rng.standard_normal((6, 1, 8))
    do = rng.standard_normal((1, 1, 8))
    br = _one_seq(q, k, v, do, 2)
    full = _one_seq(q, k, v, do, 0)
    tl = _one_seq(q, k, v, do, 1)
    np.testing.assert_allclose(br[0], full[0], atol=1e-14)
    for a, b in zip(br[2], full[2]):
        np.testing.assert_allclose(a, b, atol=1e-14)
    np.testing.assert_allclose(tl[0][0, 0], v[0, 0], atol=1e-14)


def test_bottom_right_visible_counts_and_rows():
    from oracle import attn_rows, visible_keys
    # counts: row i sees min(max(i + 1 + lk - lq, 0), lk) keys
    for lq, lk in [(3, 8), (8, 3), (5, 5), (0, 4), (4, 0)]:
        vk = visible_keys(lq, lk, 2)
        for i in range(lq):
            assert vk[i].sum() == min(max(i + 1 + lk - lq, 0), lk)
            assert not vk[i, vk[i].sum():].any()
    # the row sampler agrees with the whole-sequence oracle on mixed types
    w = workloads.random_layout(77, batch=5, max_len=12, h_q=2, h_kv=1, d=8,
                                dtype="bf16", causal="types", cross=True, min_len=0)
    assert 2 in w.causal
    q, k, v, do = (f64(t) for t in workloads.make_tensors(w))
    out, lse = attn_fwd(q, k, v, w.cu_q, w.cu_kv, w.batch, w.causal)
    dq, _, _ = attn_bwd(q, k, v, do, w.cu_q, w.cu_kv, w.batch, w.causal)
    for b, (s, n) in enumerate(sequence_rows(w.cu_q, w.batch)):
        if n == 0:
            continue
        for hq in range(w.h_q):
            o_r, l_r, dq_r = attn_rows(q, k, v, do, w.cu_q, w.cu_kv, b, hq, list(range(n)),
                                       w.causal)
            np.testing.assert_allclose(o_r, out[s:s + n, hq], atol=1e-13)
            np.testing.assert_allclose(l_r, lse[hq, s:s + n], atol=1e-13)
            np.testing.assert_allclose(dq_r, dq[s:s + n, hq], atol=1e-13)


@pytest.mark.parametrize("seed", [23, 24])
def test_bottom_right_backward_central_differences(seed):
    w = workloads.random_layout(seed, batch=3, max_len=5, h_q=2, h_kv=1, d=4,
                                dtype="fp16", causal="types", cross=True, min_len=1)
    q, k, v, do = (f64(t) for t in workloads.make_tensors(w))
    args = (w.cu_q, w.cu_kv, w.batch, np.full(w.batch, 2, np.uint8))

    def loss(qq, kk, vv):
        o, _ = attn_fwd(qq, kk, vv, *args)
        return float((o * do).sum())

    grads = attn_bwd(q, k, v, do, *args)
    eps = 1e-6
    for idx, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp = x.copy(); xp[pos] += eps
            xm = x.copy(); xm[pos] -= eps
            ins_p = [q, k, v]; ins_p[idx] = xp
            ins_m = [q, k, v]; ins_m[idx] = xm
            num[pos] = (loss(*ins_p) - loss(*ins_m)) / (2 * eps)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(g), 1e-30)
        assert err < 1e-7, (idx, err)
