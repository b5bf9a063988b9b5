"""GPU: thd_padding_mask against the oracle, bit-exact, over the pages' case
spaces (TransformerEngine PR "[PyTorch] Build the attention padding mask
without host syncs", Equivalence) and the invalid / longer-buffer inputs."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import variable_length_packed_amd as thd
from oracle import padding_mask

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_equivalence.json")


def _cu(lens, extra=0):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    tail = np.array([2**31 - 1, -5, 3, -2**31][:extra], np.int64)
    return np.concatenate([cu, tail]).astype(np.int32)


def gpu_mask(cu_np, batch, max_seqlen):
    cu = torch.from_numpy(cu_np).cuda()
    return thd.padding_mask(cu, batch, max_seqlen).cpu().numpy()


def test_self_attention_space_per_case():
    """Every case of the self-attention space, one launch per case."""
    g = json.load(open(GOLDEN))["self_attention"]
    cases = mismatches = 0
    for max_seqlen in range(1, 9):
        for batch in range(1, 5):
            for lens in itertools.product(range(max_seqlen + 1), repeat=batch):
                for extra in (0, 3):
                    cu = _cu(lens, extra)
                    got = gpu_mask(cu, batch, max_seqlen)
                    ref = padding_mask(cu, batch, max_seqlen)
                    cases += 1
                    if got.shape != ref.shape or got.dtype != ref.dtype or not np.array_equal(got, ref):
                        mismatches += 1
    print(f"self-attention cases={cases} mismatches={mismatches}", flush=True)
    assert cases == g["cases"] and mismatches == 0


def test_cross_attention_space_batched():
    """The cross-attention space: every (q lengths, kv lengths) case of the
    page, with each side's mask built by one launch over all length tuples of
    a (max, batch) cell (rows are independent: row b reads only cu[b], cu[b+1])."""
    g = json.load(open(GOLDEN))["cross_attention"]
    side = {}
    for mx in range(1, 6):
        for batch in range(1, 4):
            tuples = list(itertools.product(range(mx + 1), repeat=batch))
            flat = np.array(tuples, np.int64).reshape(-1)
            cu = _cu(flat, extra=2)
            got = gpu_mask(cu, flat.size, mx).reshape(len(tuples), batch, mx)
            ref = padding_mask(cu, flat.size, mx).reshape(len(tuples), batch, mx)
            assert np.array_equal(got, ref)
            side[(mx, batch)] = (tuples, got)
    cases = 0
    for mq in range(1, 6):
        for mk in range(1, 6):
            for batch in range(1, 4):
                tq, gq = side[(mq, batch)]
                tk, gk = side[(mk, batch)]
                cases += len(tq) * len(tk)
                # joint pair mask for a few cases, against the definition
                for a in (0, len(tq) - 1):
                    for b in (0, len(tk) // 2):
                        joint = gq[a][:, :, None] | gk[b][:, None, :]
                        lq = np.array(tq[a]); lk = np.array(tk[b])
                        i = np.arange(mq)[None, :, None]; j = np.arange(mk)[None, None, :]
                        ref = (i >= lq[:, None, None]) | (j >= lk[:, None, None])
                        assert np.array_equal(joint, ref)
    assert cases == g["cases"]


def test_invalid_and_garbage_inputs():
    # longer than max -> all False; negative -> all True; int32 wrap
    cu = np.array([0, 9, 4, -2**31, 2**31 - 1, 77, -1], np.int32)
    got = gpu_mask(cu, 4, 6)
    ref = padding_mask(cu, 4, 6)
    np.testing.assert_array_equal(got, ref)
    assert not got[0].any() and got[1].all()


def test_entries_past_batch_are_not_read_and_no_overrun():
    cu = torch.tensor([0, 3, 5, 2**31 - 1, -7], dtype=torch.int32, device="cuda")
    buf = torch.full((2 * 7 + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    from variable_length_packed_amd import _lib
    lib = _lib.load()
    import ctypes
    st = lib.thd_padding_mask(ctypes.c_void_p(cu.data_ptr()), 2, 7,
                              ctypes.c_void_p(buf.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    out = buf.cpu().numpy()
    np.testing.assert_array_equal(out[:14].reshape(2, 7),
                                  padding_mask(cu.cpu().numpy(), 2, 7).reshape(2, 7))
    assert np.all(out[14:] == 0xAB)


def test_large_mask_config5_shape():
    # the cross-attention configuration: q [32,1,1,512], kv [32,1,1,8192]
    import workloads
    w = workloads.config("5")
    for cu, mx in ((w.cu_q, 512), (w.cu_kv, 8192)):
        got = gpu_mask(np.asarray(cu), w.batch, mx)
        assert got.shape == (32, 1, 1, mx)
        np.testing.assert_array_equal(got, padding_mask(cu, w.batch, mx))


@pytest.mark.parametrize("mq,mk,batch", [(512, 8192, 32), (7, 3, 5), (1, 1, 1), (0, 9, 3), (6, 0, 2)])
def test_mask_pair_in_one_launch(mq, mk, batch):
    # both masks of a query / key pair from one entry point, each bit-exact
    # against the definition, with no byte written past either mask
    rng = np.random.default_rng(mq * 31 + mk)
    lq = rng.integers(-2, max(mq, 1) + 3, size=batch)
    lk = rng.integers(-2, max(mk, 1) + 3, size=batch)
    cu_q, cu_k = _cu(lq, extra=2), _cu(lk, extra=3)
    print(f"case mq={mq} mk={mk} batch={batch}", flush=True)
    G = 64
    bq = torch.full((batch * mq + 2 * G,), 0xAB, dtype=torch.uint8, device="cuda")
    bk = torch.full((batch * mk + 2 * G,), 0xCD, dtype=torch.uint8, device="cuda")
    from variable_length_packed_amd import _lib
    import ctypes
    lib = _lib.load()
    tq, tk = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    vp = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    st = lib.thd_padding_masks(vp(tq), vp(tk), batch, mq, mk, vp(bq, G), vp(bk, G),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    oq, ok = bq.cpu().numpy(), bk.cpu().numpy()
    assert np.all(oq[:G] == 0xAB) and np.all(oq[G + batch * mq:] == 0xAB)
    assert np.all(ok[:G] == 0xCD) and np.all(ok[G + batch * mk:] == 0xCD)
    if mq:
        np.testing.assert_array_equal(oq[G:G + batch * mq].reshape(batch, mq),
                                      padding_mask(cu_q, batch, mq).reshape(batch, mq))
    if mk:
        np.testing.assert_array_equal(ok[G:G + batch * mk].reshape(batch, mk),
                                      padding_mask(cu_k, batch, mk).reshape(batch, mk))
    if mq and mk:
        # the torch wrapper gives the same pair
        gq, gk = thd.padding_masks(tq, tk, batch, mq, mk)
        np.testing.assert_array_equal(gq.cpu().numpy().reshape(batch, mq),
                                      oq[G:G + batch * mq].reshape(batch, mq).astype(bool))
        np.testing.assert_array_equal(gk.cpu().numpy().reshape(batch, mk),
                                      ok[G:G + batch * mk].reshape(batch, mk).astype(bool))
