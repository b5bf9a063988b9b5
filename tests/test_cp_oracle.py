"""Pins of the oracle's context-parallel split (Megatron-LM issue "How to pad
sequences that cannot be evenly split in context parallelism (CP)?").

The page fixes the padding (a length-7 sequence over 2 devices is padded to
8, the pad masked out) and prints the full attention the split must
reproduce; the load-balanced chunk assignment is our reading and is pinned by
the properties any split must have plus the balance it is chosen for."""
import json
import os

import numpy as np
import pytest

from oracle import thd_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
def test_split_covers_every_padded_position_once(n):
    rng = np.random.default_rng(n)
    for length in list(range(0, 40)) + list(rng.integers(1, 5000, 20)):
        padded = orc.cp_padded_length(length, n)
        # least multiple of 2n that holds the sequence
        assert padded % (2 * n) == 0 and padded >= length and padded - length < 2 * n
        seen = []
        for r in range(n):
            pos = orc.cp_local_positions(length, n, r)
            assert len(pos) == padded // n            # equal shares
            valid = [p < length for p in pos]
            # valid rows form a prefix of the rank's local order
            assert valid == sorted(valid, reverse=True)
            seen += pos
        assert sorted(seen) == list(range(padded))


def test_page_padding_of_seven_tokens_over_two_devices():
    # the question: length 7 with CP over 2 devices is padded to 8
    assert orc.cp_padded_length(7, 2) == 8
    held = [orc.cp_local_positions(7, 2, r) for r in range(2)]
    assert sum(len(h) for h in held) == 8
    assert sum(p < 7 for h in held for p in h) == 7


@pytest.mark.parametrize("n", [2, 4])
def test_causal_work_is_balanced(n):
    # a query at position p sees p + 1 keys under the causal mask; the split
    # gives every rank the same total when the length is a multiple of 2n
    length = 16 * n
    work = [sum(p + 1 for p in orc.cp_local_positions(length, n, r)) for r in range(n)]
    assert len(set(work)) == 1


def test_rank_outputs_reproduce_page_reference():
    """Each rank's valid rows carry the page's printed full-attention values
    (the seven-token example: 1.9268 for tokens 0-3, 1.9951 for 4-6)."""
    g = json.load(open(os.path.join(GOLD, "seven_token_example.json")))
    x = np.concatenate([np.full((4, 1, 8), 1.0), np.full((3, 1, 8), 2.0)])
    for r in range(2):
        o, lse = orc.cp_attn_rank(x, x, x, [7], 2, r)
        for j, pos in enumerate(orc.cp_local_positions(7, 2, r)):
            if pos >= 7:
                assert np.all(o[j] == 0) and np.all(lse[:, j] == -np.inf)
                continue
            got = {"%.4f" % float(np.float16(t)) for t in o[j, 0]}
            assert got == {g["rows_0_3"] if pos < 4 else g["rows_4_6"]}
