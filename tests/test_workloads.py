"""The synthetic workload recipes reproduce the stated sizes."""
import numpy as np

import workloads


def test_config_sizes():
    w2 = workloads.config("2")
    assert (w2.batch, w2.T_q, w2.h_q, w2.d) == (16, 16640, 16, 128)
    assert w2.causal.all() and w2.cu_q_padded is None
    w3 = workloads.config("3")
    assert int(w3.lens_q.sum()) == 30261 and w3.T_q == 34432
    assert np.all(np.diff(w3.cu_q_padded[:65].astype(np.int64)) % 128 == 0)
    w4 = workloads.config("4")
    assert (w4.batch, w4.T_q, int(w4.lens_q.max()), w4.h_q, w4.h_kv) == (42, 131072, 19484, 32, 8)
    w5 = workloads.config("5")
    assert (w5.T_q, w5.T_kv, len(w5.cu_q), len(w5.cu_kv)) == (7572, 133300, 65, 65)
    assert np.all(w5.cu_q[33:] == 2**31 - 1)


def test_pad_rows_and_layout():
    w = workloads.random_layout(3, batch=4, max_len=6, h_q=2, d=8, slot_multiple=4,
                                gap_before=2, min_len=1)
    q, k, v, do = workloads.make_tensors(w)
    valid = w.row_is_valid_q()
    assert not valid[:2].any()
    assert (q[~valid].float() == 100).all() and (do[~valid].float() == 100).all()
    assert valid.sum() == w.lens_q.sum()


def test_valid_pair_accounting_matches_oracle_masks():
    # the benchmark's pair count (host arithmetic) against the oracle's masks,
    # for every mask type and both lq <= lk and lq > lk
    from oracle import visible_keys
    from variable_length_packed_amd.metrics import valid_pairs as host_pairs
    rng = np.random.default_rng(9)
    lq = rng.integers(0, 40, size=60)
    lk = rng.integers(0, 40, size=60)
    mt = rng.integers(0, 4, size=60).astype(np.uint8)
    expect = sum(int(visible_keys(a, b, t).sum()) for a, b, t in zip(lq, lk, mt))
    assert host_pairs(lq, lk, mt, h_q=3) == 3 * expect
