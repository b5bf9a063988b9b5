"""Context parallelism on one GPU (Megatron-LM issue "How to pad sequences that
cannot be evenly split in context parallelism (CP)?"): the device layout of
each ring step, the shard gather and each rank's merged attention, against
the oracle's split and full attention."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import thd_oracle as orc
from variable_length_packed_amd import cp
from gpu_helpers import assert_close, f64

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")
DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _i32(a):
    return torch.from_numpy(np.asarray(a, np.int32)).cuda()


def _global_layout(lengths, n):
    padded = [orc.cp_padded_length(L, n) for L in lengths]
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)


def _expected_view(lengths, causal, n, r, p, side):
    """(cu_seqlens, view starts, global starts, mask) of one step's view, from
    the oracle's chunk positions."""
    owner = r if side == cp.SIDE_Q else p
    cu, starts, g = [0], [], _global_layout(lengths, n)
    slot = 0
    for b, L in enumerate(lengths):
        pos = orc.cp_local_positions(L, n, owner)
        c = len(pos) // 2
        v1 = sum(q < L for q in pos[:c])
        v2 = sum(q < L for q in pos[c:])
        valid, start = v1 + v2, slot
        if causal[b] and side == cp.SIDE_Q and p > r:
            valid, start = v2, slot + c
        elif causal[b] and side == cp.SIDE_KV and p < r:
            valid = v1
        cu.append(cu[-1] + valid)
        starts.append(start)
        slot += len(pos)
    starts.append(slot)
    mask = [1 if (causal[b] and p == r) else 0 for b in range(len(lengths))]
    return np.array(cu), np.array(starts), g, np.array(mask)


def _lengths(seed, batch, max_len, n):
    rng = np.random.default_rng(seed)
    lens = list(rng.integers(1, max_len, size=batch))
    return lens + [0, 1, 2 * n - 1, 2 * n, 2 * n + 1]  # the small and ragged cases


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_layout_matches_oracle_split(n):
    lengths = _lengths(200 + n, 9, 300, n)
    causal = (np.arange(len(lengths)) % 3 != 1).astype(np.uint8)
    cu_g = _i32(np.concatenate([[0], np.cumsum(lengths)]))
    mt = torch.from_numpy(causal).cuda()
    for r in range(n):
        for p in range(n):
            for side in (cp.SIDE_Q, cp.SIDE_KV):
                got = cp.cp_layout(cu_g, n, r, p, side, mask_type=mt)
                ecu, est, eg, em = _expected_view(lengths, causal, n, r, p, side)
                assert got["cu_seqlens"].cpu().numpy().tolist() == ecu.tolist()
                assert got["cu_seqlens_padded"].cpu().numpy().tolist() == est.tolist()
                assert got["global_cu_seqlens_padded"].cpu().numpy().tolist() == eg.tolist()
                assert got["mask_type"][:len(lengths)].cpu().numpy().tolist() == em.tolist()


@pytest.mark.parametrize("n", [1, 2, 4])
def test_shard_gather_is_the_oracle_split(n):
    lengths = _lengths(300 + n, 7, 200, n)
    g = _global_layout(lengths, n)
    T = int(g[-1])
    rows = torch.arange(T, dtype=torch.int32).view(T, 1, 1).repeat(1, 2, 8).cuda()  # [T, 2, 8] ids
    cu_g = _i32(np.concatenate([[0], np.cumsum(lengths)]))
    for r in range(n):
        sh = cp.cp_shard(rows, cu_g, n, r, T // n).cpu().numpy()
        want = [g[b] + p for b, L in enumerate(lengths) for p in orc.cp_local_positions(L, n, r)]
        assert sh[:, 0, 0].tolist() == want
        assert np.all(sh == sh[:, :1, :1])


def _run_cp(lengths, n, h_q, h_kv, d, dtype, causal, seed, pad_value=100.0):
    """Global padded q, k, v (valid rows from one packed draw, pads =
    pad_value), every rank's merged output, and the oracle's per rank."""
    rng = torch.Generator().manual_seed(seed)
    tot = int(np.sum(lengths))
    qp = torch.randn((tot, h_q, d), generator=rng).to(DT[dtype])
    kp = torch.randn((tot, h_kv, d), generator=rng).to(DT[dtype])
    vp = torch.randn((tot, h_kv, d), generator=rng).to(DT[dtype])
    g = _global_layout(lengths, n)
    T = int(g[-1])
    cu_p = np.concatenate([[0], np.cumsum(lengths)])
    glob = []
    for x in (qp, kp, vp):
        y = torch.full((T,) + tuple(x.shape[1:]), pad_value, dtype=x.dtype)
        for b, L in enumerate(lengths):
            y[g[b]:g[b] + L] = x[cu_p[b]:cu_p[b] + L]
        glob.append(y.cuda())
    cu_g = _i32(cu_p)
    mt = torch.from_numpy(np.asarray(causal, np.uint8)).cuda()
    shards = [[cp.cp_shard(t, cu_g, n, r, T // n) for r in range(n)] for t in glob]
    outs = []
    for r in range(n):
        o, lse = cp.cp_attn_fwd(shards[0][r], shards[1], shards[2], cu_g, n, r, max(lengths),
                                mask_type=mt)
        ro, rl = orc.cp_attn_rank(f64(qp), f64(kp), f64(vp), lengths, n, r,
                                  mask_type=np.asarray(causal, np.uint8))
        valid = np.array([p < L for L in lengths for p in orc.cp_local_positions(L, n, r)])
        outs.append((o, lse, ro, rl, valid))
    return outs


CASES = [
    dict(seed=401, n=2, batch=6, max_len=400, h_q=2, h_kv=2, d=128, dtype="bf16", causal="mixed"),
    dict(seed=402, n=4, batch=5, max_len=700, h_q=4, h_kv=2, d=128, dtype="bf16", causal="all"),
    dict(seed=403, n=3, batch=7, max_len=300, h_q=2, h_kv=1, d=64, dtype="fp16", causal="none"),
    dict(seed=404, n=2, batch=4, max_len=900, h_q=2, h_kv=2, d=32, dtype="fp16", causal="all"),
]


@pytest.mark.parametrize("c", CASES, ids=[f"cp{c['n']}_{c['seed']}" for c in CASES])
def test_cp_forward_matches_full_attention(c):
    lengths = _lengths(c["seed"], c["batch"], c["max_len"], c["n"])
    k = len(lengths)
    causal = {"none": np.zeros(k), "all": np.ones(k),
              "mixed": (np.arange(k) % 2 == 0)}[c["causal"]].astype(np.uint8)
    print(f"case {c}", flush=True)
    for r, (o, lse, ro, rl, valid) in enumerate(_run_cp(lengths, c["n"], c["h_q"], c["h_kv"],
                                                        c["d"], c["dtype"], causal, c["seed"])):
        assert_close(f"rank {r} out", f64(o)[valid], ro[valid], c["dtype"])
        bits = o.detach().view(torch.int16).cpu().numpy()[~valid]
        assert np.all(bits == 0), f"rank {r}: nonzero pad rows"
        gl = lse.cpu().numpy()
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin)
        assert np.max(np.abs(gl[fin] - rl[fin]), initial=0.0) <= 1e-3 * max(1.0, np.abs(rl[fin]).max(initial=1.0))


def test_cp_page_example_two_devices():
    """The page's length-7 sequence over 2 devices (padded to 8, the pad token
    100): every rank's valid rows print as the page's full-attention values."""
    gold = json.load(open(os.path.join(GOLD, "seven_token_example.json")))
    lengths = [7]
    g = _global_layout(lengths, 2)
    x = torch.full((int(g[-1]), 1, 8), 100.0)
    x[0:4] = 1.0
    x[4:7] = 2.0
    x = x.to(torch.float16).cuda()
    cu_g = _i32([0, 7])
    shards = [cp.cp_shard(x, cu_g, 2, r, 4) for r in range(2)]
    for r in range(2):
        o, _ = cp.cp_attn_fwd(shards[r], shards, shards, cu_g, 2, r, 7)
        oc = o.cpu().float().numpy()
        for j, pos in enumerate(orc.cp_local_positions(7, 2, r)):
            if pos >= 7:
                assert np.all(oc[j] == 0)
                continue
            assert {"%.4f" % t for t in oc[j, 0]} == {gold["rows_0_3"] if pos < 4 else gold["rows_4_6"]}


BWD_CASES = [
    dict(seed=411, n=2, batch=5, max_len=300, h_q=2, h_kv=2, d=128, dtype="bf16", causal="mixed"),
    dict(seed=412, n=4, batch=4, max_len=500, h_q=4, h_kv=2, d=64, dtype="bf16", causal="all"),
    dict(seed=413, n=3, batch=5, max_len=200, h_q=2, h_kv=1, d=128, dtype="fp16", causal="none"),
]


@pytest.mark.parametrize("c", BWD_CASES, ids=[f"cp{c['n']}_{c['seed']}" for c in BWD_CASES])
def test_cp_backward_matches_full_attention(c):
    """Each rank's dq, and every shard's dk / dv summed over the ranks'
    contributions, equal the full backward at the shard's rows."""
    n = c["n"]
    lengths = _lengths(c["seed"], c["batch"], c["max_len"], n)
    k = len(lengths)
    causal = {"none": np.zeros(k), "all": np.ones(k),
              "mixed": (np.arange(k) % 2 == 0)}[c["causal"]].astype(np.uint8)
    print(f"case {c}", flush=True)
    rng = torch.Generator().manual_seed(c["seed"])
    tot = int(np.sum(lengths))
    dt = DT[c["dtype"]]
    qp = torch.randn((tot, c["h_q"], c["d"]), generator=rng).to(dt)
    kp = torch.randn((tot, c["h_kv"], c["d"]), generator=rng).to(dt)
    vp = torch.randn((tot, c["h_kv"], c["d"]), generator=rng).to(dt)
    dop = torch.randn((tot, c["h_q"], c["d"]), generator=rng).to(dt)
    g = _global_layout(lengths, n)
    T = int(g[-1])
    cu_p = np.concatenate([[0], np.cumsum(lengths)])
    glob = []
    for x in (qp, kp, vp, dop):
        y = torch.full((T,) + tuple(x.shape[1:]), 100.0, dtype=x.dtype)
        for b, L in enumerate(lengths):
            y[g[b]:g[b] + L] = x[cu_p[b]:cu_p[b] + L]
        glob.append(y.cuda())
    cu_g = _i32(cu_p)
    mt = torch.from_numpy(causal).cuda()
    q_s, k_s, v_s, do_s = ([cp.cp_shard(t, cu_g, n, r, T // n) for r in range(n)] for t in glob)
    parts, dqs = [], []
    for r in range(n):
        o, lse = cp.cp_attn_fwd(q_s[r], k_s, v_s, cu_g, n, r, max(lengths), mask_type=mt)
        dq, pr = cp.cp_attn_bwd(q_s[r], k_s, v_s, o, do_s[r], lse, cu_g, n, r, max(lengths),
                                mask_type=mt)
        dqs.append(dq)
        parts.append(pr)
    rdq, rdk, rdv = orc.attn_bwd(f64(qp), f64(kp), f64(vp), f64(dop), cu_p, cu_p, k,
                                 mask_type=causal)

    def at_rank(full, r):
        rows = []
        for b, L in enumerate(lengths):
            for pos in orc.cp_local_positions(L, n, r):
                rows.append(full[cu_p[b] + pos] if pos < L else np.zeros_like(full[0]))
        return np.stack(rows)

    for r in range(n):
        valid = np.array([p < L for L in lengths for p in orc.cp_local_positions(L, n, r)])
        assert_close(f"rank {r} dq", f64(dqs[r])[valid], at_rank(rdq, r)[valid], c["dtype"])
        dk = cp.cp_reduce([parts[s][r][0] for s in range(n)])
        dv = cp.cp_reduce([parts[s][r][1] for s in range(n)])
        assert_close(f"shard {r} dk", f64(dk)[valid], at_rank(rdk, r)[valid], c["dtype"])
        assert_close(f"shard {r} dv", f64(dv)[valid], at_rank(rdv, r)[valid], c["dtype"])
        for name, t in (("dq", dqs[r]), ("dk", dk), ("dv", dv)):
            bits = t.detach().view(torch.int16).cpu().numpy()[~valid]
            assert np.all(bits == 0), f"rank {r} {name}: nonzero pad rows"


def _merge_reference(os_, ls_):
    """The log-sum-exp merge written out in fp64: lse = log sum_k e^(l_k),
    o = sum_k e^(l_k - lse) o_k; rows whose l_k are all -inf give -inf and 0."""
    L = np.stack([l.astype(np.float64) for l in ls_])          # [n, h, T]
    m = L.max(axis=0)
    fin = np.isfinite(m)
    w = np.where(np.isfinite(L), np.exp(L - np.where(fin, m, 0.0)), 0.0)
    s = w.sum(axis=0)
    lse = np.where(fin, np.where(fin, m, 0.0) + np.log(np.where(fin, s, 1.0)), -np.inf)
    wn = np.where(fin, w / np.where(fin, s, 1.0), 0.0)          # [n, h, T]
    o = sum(wn[k].T[:, :, None] * os_[k].astype(np.float64) for k in range(len(os_)))
    return o, lse


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_lse_merge_n_matches_definition(n):
    print(f"lse_merge_n: {n} partials", flush=True)
    g = torch.Generator().manual_seed(300 + n)
    T, h, d = 97, 3, 128
    os_ = [torch.randn((T, h, d), generator=g).to(torch.bfloat16) for _ in range(n)]
    ls_ = [4 * torch.randn((h, T), generator=g) for _ in range(n)]
    for k in range(n):              # some partials see no key: -inf
        ls_[k][:, (torch.arange(T) + k) % 5 == 0] = -float("inf")
    ls_[0][:, 3] = -float("inf")    # row 3: -inf in every partial when n == 1
    if n > 1:
        for l in ls_:
            l[:, 7] = -float("inf")  # row 7: -inf in every partial
    for k in range(n):              # a partial that saw no key has o = 0
        os_[k] = torch.where(torch.isinf(ls_[k]).T[:, :, None], torch.zeros_like(os_[k]),
                             os_[k]).contiguous()
    ro, rl = _merge_reference([o.float().numpy() for o in os_], [l.numpy() for l in ls_])
    out, lse = cp.lse_merge_n([o.cuda() for o in os_], [l.cuda() for l in ls_])
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse.cpu().numpy()), fin)
    assert np.abs(lse.cpu().numpy()[fin] - rl[fin]).max() < 1e-5
    got = out.float().cpu().numpy()
    # one rounding to bf16 of an fp32 sum of at most 8 weighted terms
    assert np.all(np.abs(got - ro) <= 2 ** -8 * np.abs(ro) + 1e-6)
    assert np.all(got.transpose(1, 0, 2)[~fin] == 0)
    # the step-by-step fp32 accumulator merge agrees with the same definition
    o_acc = torch.empty((T, h, d), dtype=torch.float32, device="cuda")
    l_acc = torch.empty((h, T), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out)
    for k in range(n):
        cp.lse_merge(os_[k].cuda(), ls_[k].cuda(), o_acc, l_acc, first=(k == 0),
                     o_out=out2 if k == n - 1 else None)
    got2 = out2.float().cpu().numpy()
    assert np.all(np.abs(got2 - ro) <= 2 ** -7 * np.abs(ro) + 1e-6)
    assert np.abs(l_acc.cpu().numpy()[fin] - rl[fin]).max() < 1e-5


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_sum_n_is_the_fp32_sum(n):
    print(f"sum_n: {n} partials", flush=True)
    g = torch.Generator().manual_seed(400 + n)
    parts = [torch.randn((61, 4, 64), generator=g).to(torch.bfloat16) for _ in range(n)]
    acc = torch.zeros(parts[0].shape, dtype=torch.float32)
    for p in parts:                 # fp32, in the order given, one rounding
        acc = acc + p.float()
    want = acc.to(torch.bfloat16)
    got = cp.sum_n([p.cuda() for p in parts]).cpu()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    # the fp32 accumulator form gives the same bits
    a = torch.empty(parts[0].shape, dtype=torch.float32, device="cuda")
    out = torch.empty_like(parts[0], device="cuda")
    for k, p in enumerate(parts):
        cp.accumulate(p.cuda(), a, first=(k == 0), out=out if k == n - 1 else None)
    assert torch.equal(out.cpu().view(torch.int16), want.view(torch.int16))
