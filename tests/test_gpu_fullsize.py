"""GPU: the synthetic configurations at full size, in the benchmark's launch
configuration, checked against the oracle on samples it can compute quickly:
output, LSE and dq of selected query rows (the oracle evaluates those rows
alone), dk/dv of whole selected sequences, and every pad row bit-exact +0."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn_bwd, attn_rows
from gpu_helpers import assert_close, assert_pad_rows_zero, dev_meta, gpu_bwd, gpu_fwd

pytestmark = pytest.mark.gpu


def seq_slice(t, start, n, head):
    return t[start:start + n, head:head + 1].to("cpu", torch.float64).numpy()


def check_config(name, n_row_seqs=3, n_full_seqs=2, max_full_len=1200):
    w = workloads.config(name)
    print(f"config {name}: B={w.batch} Tq={w.T_q} Tkv={w.T_kv} h={w.h_q}/{w.h_kv}", flush=True)
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    meta = dev_meta(w)
    o, lse = gpu_fwd(w, q, k, v, meta)
    dq, dk, dv = gpu_bwd(w, q, k, v, o, do, lse, meta)
    torch.cuda.synchronize()
    vq, vk = w.row_is_valid_q(), w.row_is_valid_kv()
    for nm, t, valid in (("out", o, vq), ("dq", dq, vq), ("dk", dk, vk), ("dv", dv, vk)):
        assert_pad_rows_zero(nm, t, valid)
        assert torch.isfinite(t.float()).all(), nm
    sq, sk = w.starts_q(), w.starts_kv()
    group = w.h_q // w.h_kv
    rng = np.random.default_rng(1000 + int(name))
    order = np.argsort(w.lens_q)
    row_seqs = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2])})[:n_row_seqs]
    # --- sampled query rows: out, lse, dq --------------------------------
    got_o, ref_o, got_dq, ref_dq = [], [], [], []
    for b in row_seqs:
        lq, lk = int(w.lens_q[b]), int(w.lens_kv[b])
        if lq == 0:
            continue
        rows = sorted({0, lq - 1, lq // 2, *rng.integers(0, lq, size=5).tolist()})
        for hq in sorted({0, w.h_q - 1, int(rng.integers(0, w.h_q))}):
            hk = hq // group
            Q = seq_slice(q, sq[b], lq, hq)
            K = seq_slice(k, sk[b], lk, hk)
            V = seq_slice(v, sk[b], lk, hk)
            G = seq_slice(do, sq[b], lq, hq)
            cu_q = np.array([0, lq], np.int32)
            cu_k = np.array([0, lk], np.int32)
            ro, rl, rdq = attn_rows(Q, K, V, G, cu_q, cu_k, 0, 0, rows, [w.causal[b]])
            idx = torch.tensor([sq[b] + r for r in rows], device="cuda")
            got_o.append(o[idx, hq].cpu().double().numpy())
            got_dq.append(dq[idx, hq].cpu().double().numpy())
            ref_o.append(ro)
            ref_dq.append(rdq)
            gl = lse[hq, idx].cpu().double().numpy()
            assert np.abs(gl - rl).max() < 1e-3
    assert_close(f"cfg{name} out rows", np.concatenate(got_o), np.concatenate(ref_o), w.dtype)
    assert_close(f"cfg{name} dq rows", np.concatenate(got_dq), np.concatenate(ref_dq), w.dtype)
    # --- whole sequences: dk, dv (all query heads of one kv head) ----------
    cand = [int(b) for b in order if 0 < w.lens_q[b] <= max_full_len and w.lens_kv[b] > 0]
    full_seqs = cand[:1] + cand[-1:] if len(cand) > 1 else cand
    for b in full_seqs[:n_full_seqs]:
        lq, lk = int(w.lens_q[b]), int(w.lens_kv[b])
        hk = int(rng.integers(0, w.h_kv))
        heads = list(range(hk * group, (hk + 1) * group))
        Q = q[sq[b]:sq[b] + lq, heads].to("cpu", torch.float64).numpy()
        G = do[sq[b]:sq[b] + lq, heads].to("cpu", torch.float64).numpy()
        K = seq_slice(k, sk[b], lk, hk)
        V = seq_slice(v, sk[b], lk, hk)
        cu_q = np.array([0, lq], np.int32)
        cu_k = np.array([0, lk], np.int32)
        _, rdk, rdv = attn_bwd(Q, K, V, G, cu_q, cu_k, 1, [w.causal[b]])
        assert_close(f"cfg{name} dk seq{b}", dk[sk[b]:sk[b] + lk, hk].cpu().double().numpy(),
                     rdk[:, 0], w.dtype)
        assert_close(f"cfg{name} dv seq{b}", dv[sk[b]:sk[b] + lk, hk].cpu().double().numpy(),
                     rdv[:, 0], w.dtype)
    print(f"config {name}: ok", flush=True)


@pytest.mark.parametrize("name", ["2", "3", "5", "4", "6", "7"])
def test_full_size_config(name):
    check_config(name)
