"""Pins of the oracle functions used by the full-length and page-example GPU
checks: the key-range backward (by query-row blocks), the backward that takes
the stored forward output, and rounding to the 16-bit storage types.  Each is
checked against something other than itself: torch's fp64 autograd, the
whole-sequence oracle, closed forms, and torch's own dtype conversions."""
import numpy as np
import pytest
import torch

from oracle import attn_bwd, attn_bwd_key_range, attn_fwd, round_to_storage


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _single_seq(lq, lk, h_q, h_kv, d, seed):
    rng = np.random.default_rng(seed)
    q = _rand((lq + 3, h_q, d), rng)           # three trailing pad rows
    k = _rand((lk + 2, h_kv, d), rng)
    v = _rand((lk + 2, h_kv, d), rng)
    do = _rand((lq + 3, h_q, d), rng)
    return q, k, v, do


CASES = [
    # lq, lk, mask type, h_q, h_kv, d
    (23, 23, 1, 4, 1, 8),
    (17, 29, 0, 2, 2, 16),
    (19, 31, 2, 4, 2, 8),       # bottom-right, more keys than queries
    (31, 12, 2, 2, 1, 8),       # bottom-right, first 19 rows see no key
    (40, 40, 1, 8, 2, 24),
]


@pytest.mark.parametrize("lq,lk,mt,h_q,h_kv,d", CASES)
@pytest.mark.parametrize("row_block", [1, 5, 64])
def test_key_range_equals_whole_sequence_backward(lq, lk, mt, h_q, h_kv, d, row_block):
    q, k, v, do = _single_seq(lq, lk, h_q, h_kv, d, seed=lq * 100 + lk + mt)
    cu_q = np.array([0, lq], np.int32)
    cu_k = np.array([0, lk], np.int32)
    _, dk, dv = attn_bwd(q, k, v, do, cu_q, cu_k, 1, [mt])
    ranges = [(0, min(8, lk)), (lk // 3, min(lk // 3 + 7, lk)), (max(lk - 5, 0), lk), (4, 4),
              (0, lk)]
    for hk in range(h_kv):
        got = attn_bwd_key_range(q, k, v, do, cu_q, cu_k, 0, hk, ranges, [mt],
                                 row_block=row_block)
        for (lo, hi), (rk, rv) in zip(ranges, got):
            np.testing.assert_allclose(rk, dk[lo:hi, hk], rtol=0, atol=1e-12)
            np.testing.assert_allclose(rv, dv[lo:hi, hk], rtol=0, atol=1e-12)


def test_key_range_against_torch_autograd_with_offsets():
    """A sequence placed behind another one (row offsets from the cumulative
    buffers and padded starts), checked against torch's fp64 autograd of the
    masked softmax attention of that sequence alone."""
    rng = np.random.default_rng(7)
    h_q, h_kv, d = 6, 2, 16
    lens = [9, 37]
    starts = [0, 12]
    T = 52
    q, do = _rand((T, h_q, d), rng), _rand((T, h_q, d), rng)
    k, v = _rand((T, h_kv, d), rng), _rand((T, h_kv, d), rng)
    cu = np.array([0, 9, 46], np.int32)
    pad = np.array(starts + [T], np.int32)
    scale = 0.3
    for hk in range(h_kv):
        (rk, rv), = attn_bwd_key_range(q, k, v, do, cu, cu, 1, hk, [(10, 30)], [0, 1],
                                       cu_q_padded=pad, cu_kv_padded=pad, scale=scale,
                                       row_block=8)
        K = torch.tensor(k[12:49, hk], requires_grad=True)
        V = torch.tensor(v[12:49, hk], requires_grad=True)
        loss = 0
        for hq in range(hk * 3, hk * 3 + 3):
            Q = torch.tensor(q[12:49, hq])
            S = scale * Q @ K.T
            S = S.masked_fill(torch.triu(torch.ones(37, 37, dtype=torch.bool), 1), -torch.inf)
            loss = loss + (torch.softmax(S, -1) @ V * torch.tensor(do[12:49, hq])).sum()
        loss.backward()
        np.testing.assert_allclose(rk, K.grad.numpy()[10:30], rtol=0, atol=1e-11)
        np.testing.assert_allclose(rv, V.grad.numpy()[10:30], rtol=0, atol=1e-11)


def test_backward_from_exact_output_is_unchanged():
    q, k, v, do = _single_seq(21, 26, 4, 2, 16, seed=3)
    cu_q, cu_k = np.array([0, 21], np.int32), np.array([0, 26], np.int32)
    o, _ = attn_fwd(q, k, v, cu_q, cu_k, 1, [2])
    ref = attn_bwd(q, k, v, do, cu_q, cu_k, 1, [2])
    got = attn_bwd(q, k, v, do, cu_q, cu_k, 1, [2], out=o)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("storage", ["fp16", "bf16"])
def test_backward_from_stored_output_closed_form(storage):
    """With the stored output O' = O + E, D_i moves by dD_i = dO_i . E_i and
    the gradients by dQ_i -= scale dD_i sum_j P_ij K_j,
    dK_j -= scale sum_i P_ij dD_i Q_i, dV unchanged."""
    lq = lk = 30
    q, k, v, do = _single_seq(lq, lk, 2, 1, 8, seed=11)
    cu = np.array([0, lq], np.int32)
    scale = 1 / np.sqrt(8)
    o, _ = attn_fwd(q, k, v, cu, cu, 1, [1])
    o_st = round_to_storage(o, storage)
    dq0, dk0, dv0 = attn_bwd(q, k, v, do, cu, cu, 1, [1])
    dq1, dk1, dv1 = attn_bwd(q, k, v, do, cu, cu, 1, [1], out=o_st)
    np.testing.assert_allclose(dv1, dv0, rtol=0, atol=1e-12)
    K = k[:lk, 0]
    want_dk = np.zeros_like(K)
    for hq in range(2):
        Q = q[:lq, hq]
        S = scale * Q @ K.T
        S[np.triu_indices(lq, 1)] = -np.inf
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        dD = (do[:lq, hq] * (o_st[:lq, hq] - o[:lq, hq])).sum(1)
        np.testing.assert_allclose(dq1[:lq, hq] - dq0[:lq, hq],
                                   -scale * dD[:, None] * (P @ K), rtol=0, atol=1e-12)
        want_dk += -scale * (P * dD[:, None]).T @ Q
    np.testing.assert_allclose(dk1[:lk, 0] - dk0[:lk, 0], want_dk, rtol=0, atol=1e-12)
    assert np.abs(dq1 - dq0).max() > 0     # the rounding does move the gradients


@pytest.mark.parametrize("storage,tdtype", [("fp16", torch.float16), ("bf16", torch.bfloat16)])
def test_round_to_storage_matches_torch(storage, tdtype):
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, size=20000),
        # exact ties between neighbours of both types, and their neighbours
        1.0 + np.arange(-40, 40) * 2.0 ** -12, 1.0 + np.arange(-40, 40) * 2.0 ** -9,
        [0.0, -0.0, 65504.0, 65520.0, 1e30, -1e30, np.inf, -np.inf, 1e-8, 5.9604644775390625e-08],
    ])
    # binary32 inputs: torch converts from binary32 with one rounding, as the
    # device does when it stores an fp32 result
    x = x.astype(np.float32).astype(np.float64)
    got = round_to_storage(x, storage)
    want = torch.tensor(x, dtype=torch.float32).to(tdtype).double().numpy()
    np.testing.assert_array_equal(got, want)
    assert np.isnan(round_to_storage([np.nan], storage)).all()
