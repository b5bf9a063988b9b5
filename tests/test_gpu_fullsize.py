"""GPU: the synthetic configurations at full size, in the benchmark's launch
configuration, checked against the oracle on samples it can compute quickly:
output, LSE and dq of selected query rows (the oracle evaluates those rows
alone); dk/dv of the shortest sequence, the one with the most query rows and
the one with the most keys -- whole when the oracle is cheap, else the first,
a middle and the last 256-key tile over every query head of one kv head (the
oracle takes such a key range by query-row blocks); and every pad row
bit-exact +0.  The same checks run on config 2's lengths at head dims 32, 64,
96, 192 and 256 (fewer heads), so that every tile shape walks full-length
sequences.  On the workloads whose per-head oracle takes about a second
(configs 2, 3, 5, 6 and 7), every valid row of one kv head and its query
heads is compared too: output, LSE, dq, dk and dv over every sequence."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn_bwd, attn_bwd_key_range, attn_fwd, attn_rows
from gpu_helpers import assert_close, assert_pad_rows_zero, dev_meta, gpu_bwd, gpu_fwd

pytestmark = pytest.mark.gpu


def seq_slice(t, start, n, head):
    return t[start:start + n, head:head + 1].to("cpu", torch.float64).numpy()


# Sequences with at most this many (query, key) pairs get whole dk/dv from the
# whole-sequence oracle; longer ones three 256-key tiles from the key-range one.
WHOLE_PAIRS = 1 << 23
TILE = 256


def check_config(name, n_row_seqs=3, w=None):
    w = workloads.config(name) if w is None else w
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
    rng = np.random.default_rng(1000 + int(str(name).split("-")[0]))
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
    # --- dk, dv of chosen sequences (all query heads of one kv head) ----------
    have = [int(b) for b in range(w.batch) if w.lens_q[b] > 0 and w.lens_kv[b] > 0]
    chosen = sorted({min(have, key=lambda b: (w.lens_q[b], b)),
                     max(have, key=lambda b: (w.lens_q[b], -b)),
                     max(have, key=lambda b: (w.lens_kv[b], -b))})
    for b in chosen:
        lq, lk = int(w.lens_q[b]), int(w.lens_kv[b])
        hk = int(rng.integers(0, w.h_kv))
        heads = list(range(hk * group, (hk + 1) * group))
        got_k = dk[sk[b]:sk[b] + lk, hk].cpu().double().numpy()
        got_v = dv[sk[b]:sk[b] + lk, hk].cpu().double().numpy()
        if lq * lk <= WHOLE_PAIRS:
            Q = q[sq[b]:sq[b] + lq, heads].to("cpu", torch.float64).numpy()
            G = do[sq[b]:sq[b] + lq, heads].to("cpu", torch.float64).numpy()
            K = seq_slice(k, sk[b], lk, hk)
            V = seq_slice(v, sk[b], lk, hk)
            cu_q = np.array([0, lq], np.int32)
            cu_k = np.array([0, lk], np.int32)
            _, rdk, rdv = attn_bwd(Q, K, V, G, cu_q, cu_k, 1, [w.causal[b]])
            ranges, refs = [(0, lk)], [(rdk[:, 0], rdv[:, 0])]
        else:
            n_t = (lk + TILE - 1) // TILE
            ranges = [(t * TILE, min((t + 1) * TILE, lk)) for t in sorted({0, n_t // 2, n_t - 1})]
            # one kv head and its query heads, as a sequence of their own
            Q = q[sq[b]:sq[b] + lq, heads].to("cpu", torch.float64).numpy()
            G = do[sq[b]:sq[b] + lq, heads].to("cpu", torch.float64).numpy()
            K = seq_slice(k, sk[b], lk, hk)
            V = seq_slice(v, sk[b], lk, hk)
            cu_q = np.array([0, lq], np.int32)
            cu_k = np.array([0, lk], np.int32)
            refs = attn_bwd_key_range(Q, K, V, G, cu_q, cu_k, 0, 0, ranges, [w.causal[b]])
        for (lo, hi), (rk, rv) in zip(ranges, refs):
            print(f"config {name}: dk/dv seq {b} (lq={lq}, lk={lk}) keys [{lo},{hi}) "
                  f"kv head {hk}", flush=True)
            assert_close(f"cfg{name} dk seq{b} [{lo},{hi})", got_k[lo:hi], rk, w.dtype)
            assert_close(f"cfg{name} dv seq{b} [{lo},{hi})", got_v[lo:hi], rv, w.dtype)
    print(f"config {name}: ok", flush=True)


@pytest.mark.timeout(400)   # the long-sequence oracle tiles take tens of seconds on the host
@pytest.mark.parametrize("name", ["2", "3", "5", "4", "6", "7"])
def test_full_size_config(name):
    check_config(name)


def wide_head_config(d, dtype):
    """Config 2's lengths (16 causal sequences of 64 to 2,048 tokens) at
    another head dim, 4 query heads over 2 kv heads."""
    rng = np.random.default_rng(2)
    lens = rng.integers(64, 2048, size=16, endpoint=True)
    return workloads.packed(lens, causal=np.ones(16, np.uint8), h_q=4, h_kv=2, d=d,
                            dtype=dtype, seed=2, name=f"2-d{d}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("d,dtype", [(192, "bf16"), (256, "fp16"), (256, "bf16"),
                                     (32, "bf16"), (64, "fp16"), (96, "bf16"),
                                     (128, "fp16")])
def test_full_length_other_head_dims(d, dtype):
    # every tile shape walks full-length sequences (up to 2,034 rows per key
    # tile): 64-key tiles at d = 32, the three-wave dq pass at d = 64, d = 96
    # padded to 128, and the 256-wide passes
    check_config(f"2-d{d}", w=wide_head_config(d, dtype))


@pytest.mark.parametrize("name", ["2", "3", "5", "6", "7"])
def test_full_size_whole_head(name):
    """Every valid row of one kv head and its query heads, at full size and in
    the benchmark's launch configuration, against the oracle run on that head
    slice of the whole packed layout (the slice is a layout of its own: the
    same cu_seqlens, padded offsets and mask types, h_kv = 1)."""
    w = workloads.config(name)
    print(f"config {name} whole head: B={w.batch} Tq={w.T_q} Tkv={w.T_kv} h={w.h_q}/{w.h_kv}",
          flush=True)
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    meta = dev_meta(w)
    o, lse = gpu_fwd(w, q, k, v, meta)
    dq, dk, dv = gpu_bwd(w, q, k, v, o, do, lse, meta)
    torch.cuda.synchronize()
    group = w.h_q // w.h_kv
    hk = w.h_kv - 1
    heads = list(range(hk * group, (hk + 1) * group))
    f64 = lambda t: t.to("cpu", torch.float64).numpy()
    Q, G = f64(q[:, heads]), f64(do[:, heads])
    K, V = f64(k[:, hk:hk + 1]), f64(v[:, hk:hk + 1])
    args = (w.cu_q, w.cu_kv, w.batch, np.asarray(w.causal)[:w.batch])
    pads = dict(cu_q_padded=w.cu_q_padded, cu_kv_padded=w.cu_kv_padded)
    ro, rl = attn_fwd(Q, K, V, *args, **pads)
    rdq, rdk, rdv = attn_bwd(Q, K, V, G, *args, **pads)
    vq, vk = w.row_is_valid_q(), w.row_is_valid_kv()
    got_lse = f64(lse[heads])[:, vq]
    ref_lse = rl[:, vq]
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin), "rows without a visible key differ"
    assert np.abs(got_lse[fin] - ref_lse[fin]).max() < 1e-3
    for nm, got, ref, valid in (("out", o[:, heads], ro, vq), ("dq", dq[:, heads], rdq, vq),
                                ("dk", dk[:, hk:hk + 1], rdk, vk),
                                ("dv", dv[:, hk:hk + 1], rdv, vk)):
        ex, rr = assert_close(f"cfg{name} {nm} kv head {hk}", f64(got)[valid], ref[valid],
                              w.dtype)
        print(f"config {name} whole head {nm}: abs error beyond rounding {ex:.2e}, "
              f"relative rms {rr:.2e}", flush=True)
    print(f"config {name} whole head: ok", flush=True)


def test_full_size_gqa_whole_sequences():
    """Config 4 (GQA 32/8, 131,072 tokens): every sequence of at most 2,048
    tokens (22 of its 42), whole, for one kv head and its four query heads --
    output, LSE, dq, dk and dv against the oracle run on each sequence alone.
    The longer sequences are checked by key ranges in test_full_size_config."""
    w = workloads.config("4")
    print(f"config 4 GQA sequences: B={w.batch} Tq={w.T_q} h={w.h_q}/{w.h_kv}", flush=True)
    q, k, v, do = workloads.make_tensors(w, device="cuda")
    meta = dev_meta(w)
    o, lse = gpu_fwd(w, q, k, v, meta)
    dq, dk, dv = gpu_bwd(w, q, k, v, o, do, lse, meta)
    torch.cuda.synchronize()
    group = w.h_q // w.h_kv
    hk = 2
    heads = list(range(hk * group, (hk + 1) * group))
    sq, sk = w.starts_q(), w.starts_kv()
    f64 = lambda t: t.to("cpu", torch.float64).numpy()
    chosen = [b for b in range(w.batch) if 0 < w.lens_q[b] <= 2048]
    assert len(chosen) >= 16
    got = {n: [] for n in ("out", "dq", "dk", "dv")}
    ref = {n: [] for n in got}
    for b in chosen:
        lq, lk = int(w.lens_q[b]), int(w.lens_kv[b])
        qs, ks = slice(sq[b], sq[b] + lq), slice(sk[b], sk[b] + lk)
        Q, G = f64(q[qs, heads]), f64(do[qs, heads])
        K, V = f64(k[ks, hk:hk + 1]), f64(v[ks, hk:hk + 1])
        cu_q, cu_k = np.array([0, lq], np.int32), np.array([0, lk], np.int32)
        ro, rl = attn_fwd(Q, K, V, cu_q, cu_k, 1, [w.causal[b]])
        rdq, rdk, rdv = attn_bwd(Q, K, V, G, cu_q, cu_k, 1, [w.causal[b]])
        assert np.abs(f64(lse[heads][:, qs]) - rl).max() < 1e-3, b
        for n, g, r in (("out", o[qs, heads], ro), ("dq", dq[qs, heads], rdq),
                        ("dk", dk[ks, hk:hk + 1], rdk), ("dv", dv[ks, hk:hk + 1], rdv)):
            got[n].append(f64(g).reshape(-1))
            ref[n].append(r.reshape(-1))
    for n in got:
        ex, rr = assert_close(f"cfg4 {n} of {len(chosen)} sequences, kv head {hk}",
                              np.concatenate(got[n]), np.concatenate(ref[n]), w.dtype)
        print(f"config 4 GQA sequences {n}: abs error beyond rounding {ex:.2e}, "
              f"relative rms {rr:.2e}", flush=True)
