"""Pins for the oracle's padding mask (CPU only).

The two oracle forms -- the definitional ``positions >= seqlens`` and the
older per-sequence list loop -- are independent implementations.  The pages
state that they agree on every case of two exhaustively enumerated spaces and
give the case counts; those counts and the zero-mismatch result are the pins
(tests/golden/mask_equivalence.json).
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import padding_mask, padding_mask_loop

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mask_equivalence.json")


def _cu(lens, extra=0):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    # a buffer sized for a larger batch: the extra entries must be ignored
    cu += [2**31 - 1, -5, 3][:extra] + [7] * max(0, extra - 3)
    return np.array(cu, dtype=np.int32)


def test_mask_rows_match_list_definition():
    # row b is [False]*len_b + [True]*(max - len_b), shape [B,1,1,max]
    m = padding_mask(np.array([0, 3, 5, 9], np.int32), 3, 5)
    assert m.shape == (3, 1, 1, 5) and m.dtype == bool
    expect = np.array([[0, 0, 0, 1, 1], [0, 0, 1, 1, 1], [0, 0, 0, 0, 1]], bool)
    np.testing.assert_array_equal(m.reshape(3, 5), expect)


def test_self_attention_space_exhaustive():
    g = json.load(open(GOLDEN))["self_attention"]
    cases = mismatches = 0
    for max_seqlen in range(1, 9):
        for batch in range(1, 5):
            for lens in itertools.product(range(max_seqlen + 1), repeat=batch):
                for longer in (False, True):
                    cu = _cu(lens, extra=3 if longer else 0)
                    a = padding_mask(cu, batch, max_seqlen)
                    b = padding_mask_loop(cu, batch, max_seqlen)
                    cases += 1
                    if a.shape != b.shape or a.dtype != b.dtype or not np.array_equal(a, b):
                        mismatches += 1
    assert cases == g["cases"]
    assert mismatches == g["mismatches"]


def test_cross_attention_space_exhaustive():
    g = json.load(open(GOLDEN))["cross_attention"]
    cache = {}

    def both(lens, mx):
        key = (lens, mx)
        if key not in cache:
            cu = _cu(lens)
            cache[key] = (padding_mask(cu, len(lens), mx).reshape(len(lens), mx),
                          padding_mask_loop(cu, len(lens), mx).reshape(len(lens), mx))
        return cache[key]

    cases = mismatches = 0
    for mq in range(1, 6):
        for mk in range(1, 6):
            for batch in range(1, 4):
                for lq in itertools.product(range(mq + 1), repeat=batch):
                    aq, bq = both(lq, mq)
                    for lk in itertools.product(range(mk + 1), repeat=batch):
                        ak, bk = both(lk, mk)
                        # joint mask of a (query, key) pair: either side is pad
                        ja = aq[:, :, None] | ak[:, None, :]
                        jb = bq[:, :, None] | bk[:, None, :]
                        cases += 1
                        if not np.array_equal(ja, jb):
                            mismatches += 1
    assert cases == g["cases"]
    assert mismatches == g["mismatches"]


def test_invalid_length_longer_than_max():
    # Equivalence: the only divergence is a length above max_seqlen; the loop
    # raises, the vectorised form gives an all-False row.
    cu = np.array([0, 2, 9], np.int32)      # second sequence has 7 > max 4
    with pytest.raises(ValueError):
        padding_mask_loop(cu, 2, 4)
    m = padding_mask(cu, 2, 4).reshape(2, 4)
    np.testing.assert_array_equal(m[1], np.zeros(4, bool))
    np.testing.assert_array_equal(m[0], np.array([0, 0, 1, 1], bool))


def test_negative_length_and_extra_entries():
    # Formula only: a negative length pads the whole row; entries after
    # batch+1 are never read, whatever they hold.
    cu = np.array([5, 3, 2**31 - 1, -2**31], np.int32)
    m = padding_mask(cu, 1, 6).reshape(1, 6)
    np.testing.assert_array_equal(m[0], np.ones(6, bool))
    cu2 = np.array([0, 3, 2**31 - 1, -2**31], np.int32)
    np.testing.assert_array_equal(padding_mask(cu2, 1, 4).reshape(4),
                                  np.array([0, 0, 0, 1], bool))


def test_int32_wraparound_is_formula():
    # cu entries are int32: a difference that overflows wraps, as on the
    # int32 tensor of the page.
    cu = np.array([-2**31, 2**31 - 1], np.int32)   # diff = 2^32-1 -> -1
    m = padding_mask(cu, 1, 3).reshape(3)
    np.testing.assert_array_equal(m, np.ones(3, bool))


def test_empty_batch_and_zero_width():
    assert padding_mask(np.array([0], np.int32), 0, 5).shape == (0, 1, 1, 5)
    assert padding_mask(np.array([0, 3], np.int32), 1, 0).shape == (1, 1, 1, 0)
