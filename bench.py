"""Benchmark: packed-thd attention forward + backward on one MI355X.

One step = the whole hot path over one synthetic packed batch: the two
padding masks (query and key side, one thd_padding_masks launch), thd_attn_fwd
and thd_attn_bwd, all on the current stream with inputs already resident in
HBM.  Workload: 16 causal
sequences with lengths uniform in [64, 2048] (seed 2, 16,640 tokens), 16
heads, head_dim 128, bf16, dO ~ N(0,1).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--spinup-seconds 1.5]
                    [--no-cpu-baseline]

Before the W warm-up steps the same step runs untimed for --spinup-seconds:
the first few hundred milliseconds under load run at lower clocks, which
would otherwise make the timed steps depend on what ran before them.  The K
timed steps are plain steps; a second pass of the same steps records HIP
events between the kernels for the per-kernel times, and a third replays the
step from one HIP graph (spun up the same way).

Prints one JSON line.  `value` is valid-pair TFLOP/s of fwd+bwd (14*d FLOPs
per valid (query, key) pair and head); `roofline` describes the dominant
kernel, timed with HIP events on the stream it runs on (its `traffic`, and
the `counters` object -- MFMA busy, LDS active and HBM bytes of the attention
kernels -- come from the committed rocprofv3 records of this workload, and
are null once a kernel's sources differ from those the records were taken
on); `cpu_baseline` is the fp64 oracle timed on the host on a bounded sample
of the same workload.  Other workloads: --config 3..7, --fwd-only.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--spinup-seconds", type=float, default=1.5)
    ap.add_argument("--config", default="2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time the padding masks and the forward only, against the HBM "
                         "roofline (for the split-KV decode workload)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (read + write) a few "
                         "times, to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# Sources each timed kernel is built from: a counter record of a kernel stays
# valid while these files are unchanged.
KERNEL_SOURCES = {
    "thd_bwd_dkdv_kernel": ("thd_bwd_dkdv.hip", "thd_bwd_split.hpp", "thd_common.hpp"),
    "thd_bwd_dq_kernel": ("thd_bwd_split.hip", "thd_bwd_split.hpp", "thd_common.hpp"),
    "thd_fwd_kernel": ("thd_fwd.hip", "thd_common.hpp", "thd_launch.hpp"),
}


def source_digest(kernel):
    """Digest of the HIP sources of one kernel and of the compiler flags they
    are built with; its counter-based traffic is valid only for them."""
    import hashlib
    from variable_length_packed_amd.build import compile_flags
    h = hashlib.sha256()
    flags = compile_flags(KERNEL_SOURCES[kernel][0])
    h.update(" ".join(f for f in flags if not f.startswith("-I")).encode())
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode())
        with open(os.path.join(ROOT, "variable_length_packed_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_record(kernel, workload_tag):
    """The committed rocprofv3 counter record of this kernel and workload, or
    None when the kernel has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_tag}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if kernel not in KERNEL_SOURCES or rec.get("source_digest") != source_digest(kernel):
        return None
    return rec


def measured_traffic(kernel, workload_tag):
    """HBM bytes per launch (FETCH_SIZE / WRITE_SIZE, copy-calibrated)."""
    rec = counter_record(kernel, workload_tag)
    return None if rec is None else int(rec["bytes_per_launch"])


def measured_busy(workload_tag):
    """MFMA-busy and LDS-active percentages of the attention kernels, from the
    committed counter records (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs, and
    SQ_LDS_IDX_ACTIVE / CUs, over GRBM_GUI_ACTIVE), and the HBM rate those
    records' traffic gives at this run's kernel times."""
    out = {}
    for kernel in KERNEL_SOURCES:
        rec = counter_record(kernel, workload_tag)
        if rec is not None and "mfma_busy_pct" in rec:
            out[kernel] = {"mfma_busy_pct": rec["mfma_busy_pct"],
                           "lds_active_pct": rec["lds_active_pct"],
                           "hbm_bytes_per_launch": rec["bytes_per_launch"]}
    return out or None


def copy_calibration(mib):
    """A plain copy kernel of known size: reads and writes exactly mib MiB."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f'{{"copy_calibration_bytes": {n * 4}}}', flush=True)


def cpu_baseline(w, q, k, v, do, budget_s):
    """Time the fp64 oracle (fwd + bwd) on whole heads of the workload until
    about `budget_s` seconds of work are done; scale to valid-pair TFLOP/s."""
    import numpy as np
    import torch
    from oracle import attn_bwd, attn_fwd
    from variable_length_packed_amd.metrics import valid_pairs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    args = (w.cu_q, w.cu_kv, w.batch, w.causal, w.cu_q_padded, w.cu_kv_padded)
    group = w.h_q // w.h_kv
    # head by head, starting over after the last head, until the budget is spent
    elapsed, heads = 0.0, 0
    while elapsed < budget_s:
        hq = heads % w.h_q
        hk = hq // group
        Q = q[:, hq:hq + 1].to("cpu", torch.float64).numpy()
        K = k[:, hk:hk + 1].to("cpu", torch.float64).numpy()
        V = v[:, hk:hk + 1].to("cpu", torch.float64).numpy()
        G = do[:, hq:hq + 1].to("cpu", torch.float64).numpy()
        t0 = time.perf_counter()
        attn_fwd(Q, K, V, *args)
        attn_bwd(Q, K, V, G, *args)
        elapsed += time.perf_counter() - t0
        heads += 1
    pairs = valid_pairs(w.lens_q, w.lens_kv, w.causal, heads)
    flops = 14 * w.d * pairs
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "affinity_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"fp64 numpy oracle, fwd+bwd of {heads} head passes ({heads / w.h_q:.2f} "
                      f"times the {w.h_q} heads) over all {w.batch} sequences of the same "
                      f"workload ({flops / 1e9:.1f} GFLOP in {elapsed:.1f} s)"}


def main():
    a = parse()
    if a.copy_calibration_mib:
        copy_calibration(a.copy_calibration_mib)
        return
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {a.gpus} is not supported "
              "(the path shards by head or by whole sequence with no exchange, see the design "
              "notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import variable_length_packed_amd as thd
    import workloads
    from variable_length_packed_amd import _lib
    from variable_length_packed_amd.attention import _make_args, _ptr, _stream
    from variable_length_packed_amd.metrics import attention_flops, valid_pairs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.config(a.config)
    q, k, v, do = workloads.make_tensors(w, device=dev)
    t32 = lambda x: None if x is None else torch.from_numpy(np.asarray(x, np.int32)).to(dev)
    cu_q, cu_kv = t32(w.cu_q), t32(w.cu_kv)
    pad_q, pad_kv = t32(w.cu_q_padded), t32(w.cu_kv_padded)
    causal = torch.from_numpy(np.asarray(w.causal, np.uint8)).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.h_q, w.T_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    mask_q = torch.empty((w.batch, 1, 1, w.max_seqlen_q), dtype=torch.bool, device=dev)
    mask_kv = torch.empty((w.batch, 1, 1, w.max_seqlen_kv), dtype=torch.bool, device=dev)

    lib = _lib.load()
    args = _make_args(q, k, cu_q, cu_kv, w.max_seqlen_q, w.max_seqlen_kv, pad_q, pad_kv,
                      causal, None, w.batch)
    ws_bytes = int(lib.thd_attn_bwd_workspace_size(args))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fws_bytes = int(lib.thd_attn_fwd_workspace_size(args))
    fws = torch.empty(max(fws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = _stream(dev)
    P = {n: _ptr(t) for n, t in dict(q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv,
                                     ws=ws, fws=fws, cu_q=cu_q, cu_kv=cu_kv, mq=mask_q,
                                     mkv=mask_kv).items()}
    import ctypes
    n_ev = 7   # 0/1 around the forward, 2..5 the backward passes, 6 the step start
    total = a.warmup + a.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(total)]
    cur = torch.cuda.current_stream(dev)
    for evs in events:             # materialise the underlying HIP events
        for e in evs:
            e.record(cur)
    torch.cuda.synchronize()
    ev_arrays = [(ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in evs[2:6]])
                 for evs in events]

    def step(i):
        evs = events[i]
        evs[6].record(cur)
        _lib.check(lib.thd_padding_masks(P["cu_q"], P["cu_kv"], w.batch, w.max_seqlen_q,
                                         w.max_seqlen_kv, P["mq"], P["mkv"], stream), "masks")
        evs[0].record(cur)
        _lib.check(lib.thd_attn_fwd(args, P["q"], P["k"], P["v"], P["o"], P["lse"], P["fws"],
                                    fws_bytes, stream), "fwd")
        evs[1].record(cur)
        if a.fwd_only:
            return
        _lib.check(lib.thd_attn_bwd_timed(args, P["q"], P["k"], P["v"], P["o"], P["do"],
                                          P["lse"], P["dq"], P["dk"], P["dv"], P["ws"],
                                          ws_bytes, stream, ev_arrays[i]), "bwd")

    def untimed_step(st=None):
        st = stream if st is None else st
        _lib.check(lib.thd_padding_masks(P["cu_q"], P["cu_kv"], w.batch, w.max_seqlen_q,
                                         w.max_seqlen_kv, P["mq"], P["mkv"], st), "masks")
        _lib.check(lib.thd_attn_fwd(args, P["q"], P["k"], P["v"], P["o"], P["lse"], P["fws"],
                                    fws_bytes, st), "fwd")
        if a.fwd_only:
            return
        _lib.check(lib.thd_attn_bwd(args, P["q"], P["k"], P["v"], P["o"], P["do"], P["lse"],
                                    P["dq"], P["dk"], P["dv"], P["ws"], ws_bytes, st), "bwd")

    def spin_up(run):
        # the first few hundred milliseconds under load run at lower clocks
        t_spin = time.perf_counter()
        while time.perf_counter() - t_spin < a.spinup_seconds:
            for _ in range(10):
                run()
            torch.cuda.synchronize()

    # Timed region: K plain steps (nothing but the step's own launches).
    spin_up(untimed_step)
    for _ in range(a.warmup):
        untimed_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        untimed_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # The same steps again with HIP events recorded between the kernels, on
    # the stream they run on, for the per-kernel times (the event records
    # themselves leave gaps between kernels, so this pass is not the one the
    # throughput is taken from).
    for i in range(total):
        step(i)
    torch.cuda.synchronize()

    # The same step captured once in a HIP graph and replayed: the launches of
    # the eager step above cost host time between kernels, a replay does not.
    # The replays are spun up like the eager steps: after the idle time of the
    # capture, the first replays run at lower clocks.  (Reported beside the
    # eager figures; a capture failure only drops it.)
    def graph_time():
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)  # default priority
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            untimed_step(_stream(dev))
        cur.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            untimed_step(_stream(dev))   # the capture stream
        torch.cuda.synchronize()
        spin_up(g.replay)
        for _ in range(a.warmup):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(cur)
        for _ in range(a.steps):
            g.replay()
        g1.record(cur)
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) / a.steps

    try:
        graph_ms = graph_time()
    except Exception as e:  # pragma: no cover - reported, not fatal
        print(f"bench.py: graph replay not measured: {e}", file=sys.stderr)
        graph_ms = None

    timed = events[a.warmup:]
    if a.fwd_only:
        res = fwd_only_result(a, w, timed, elapsed)
        res["graph_replay_ms_per_step"] = None if graph_ms is None else round(graph_ms, 4)
        print(json.dumps(res), flush=True)
        return
    fwd_ms = [e[0].elapsed_time(e[1]) for e in timed]
    # the backward's launches (head dims up to 128): pre pass, dq pass, dk/dv pass
    pre_ms = [e[2].elapsed_time(e[3]) for e in timed]
    dq_ms = [e[3].elapsed_time(e[4]) for e in timed]
    dkdv_ms = [e[4].elapsed_time(e[5]) for e in timed]
    mask_ms = [e[6].elapsed_time(e[0]) for e in timed]
    step_ms = sorted(e[6].elapsed_time(e[5]) for e in timed)
    mean = lambda xs: sum(xs) / len(xs)

    pairs = valid_pairs(w.lens_q, w.lens_kv, w.causal, w.h_q)
    flops = attention_flops(pairs, w.d, "fwd+bwd")
    ms_per_step = elapsed * 1e3 / a.steps
    value = flops / (elapsed / a.steps) / 1e12

    kern = {"thd_fwd_kernel": (mean(fwd_ms), attention_flops(pairs, w.d, "fwd")),
            "thd_bwd_dq_kernel": (mean(dq_ms), attention_flops(pairs, w.d, "bwd_dq_pass")),
            "thd_bwd_dkdv_kernel": (mean(dkdv_ms), attention_flops(pairs, w.d, "bwd_dkdv_pass"))}
    dom = max(kern, key=lambda n: kern[n][0])
    dom_ms, dom_flops = kern[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": (measured_traffic(dom, "16seq_causal_h16_d128") if w.name == "2" else None),
                "avg_launch_ms": round(dom_ms, 4),
                "flops_per_launch": int(dom_flops)}
    busy = measured_busy("16seq_causal_h16_d128") if w.name == "2" else None
    if busy is not None:
        for kernel, rec in busy.items():
            rec["hbm_gbs"] = round(rec["hbm_bytes_per_launch"] / (kern[kernel][0] * 1e-3) / 1e9, 1)

    out = {
        "metric": "packed-THD attention valid-pair TFLOP/s fwd+bwd; % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp16",
        "data": "synthetic",
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        # the same time credited with 12*d FLOPs per valid pair (no S recompute)
        "value_no_recompute_credit": round(value * 12 / 14, 2),
        "step_ms_events": {"median": round(step_ms[len(step_ms) // 2], 4),
                           "min": round(step_ms[0], 4)},
        # rocprofv3 counters of the attention kernels on this workload and build
        "counters": busy,
        # the same step replayed from one HIP graph (no launch gaps)
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 4),
            "value": round(flops / (graph_ms * 1e-3) / 1e12, 2)},
        "config": {
            "workload": (f"packed thd {'self-' if w.self_attention else 'cross-'}attention, "
                         f"config {w.name}: {w.batch} sequences, {w.T_q} query tokens"
                         f"{'' if w.self_attention else f' / {w.T_kv} kv tokens'}, "
                         f"h_q={w.h_q} h_kv={w.h_kv} d={w.d} {w.dtype}, "
                         f"{int((w.causal == 1).sum())} top-left causal, "
                         f"{int((w.causal == 2).sum())} bottom-right causal, "
                         f"fwd+bwd incl. both padding masks"),
            "tokens": int(w.T_q), "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv,
            "head_dim": w.d, "valid_pairs": int(pairs), "flops_per_step": int(flops),
            "seed": w.seed,
        },
        "kernel_ms": {"masks": round(mean(mask_ms), 4),
                      "fwd": round(mean(fwd_ms), 4), "bwd_pre": round(mean(pre_ms), 4),
                      "bwd_dq": round(mean(dq_ms), 4), "bwd_dkdv": round(mean(dkdv_ms), 4)},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, do, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def fwd_only_result(a, w, timed, elapsed):
    """The forward alone (with both padding masks), against the HBM roofline:
    algorithmic bytes = valid q, k, v read once (k, v at h_kv) + o written over
    all query rows + the log-sum-exp."""
    from variable_length_packed_amd.metrics import attention_flops, valid_pairs
    import numpy as np
    mean = lambda xs: sum(xs) / len(xs)
    fwd_ms = [e[0].elapsed_time(e[1]) for e in timed]
    mask_ms = [e[6].elapsed_time(e[0]) for e in timed]
    step_ms = sorted(e[6].elapsed_time(e[1]) for e in timed)
    pairs = valid_pairs(w.lens_q, w.lens_kv, w.causal, w.h_q)
    flops = attention_flops(pairs, w.d, "fwd")
    elem = 2
    nbytes = (int(np.sum(w.lens_q)) * w.h_q * w.d * elem
              + 2 * int(np.sum(w.lens_kv)) * w.h_kv * w.d * elem
              + int(w.T_q) * w.h_q * w.d * elem + int(w.T_q) * w.h_q * 4)
    f_ms = mean(fwd_ms)
    gbs = nbytes / (f_ms * 1e-3) / 1e9
    value = flops / (elapsed / a.steps) / 1e12
    return {
        "metric": "packed-THD attention valid-pair TFLOP/s fwd only",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(elapsed * 1e3 / a.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp16", "data": "synthetic",
        "step_ms_events": {"median": round(step_ms[len(step_ms) // 2], 4),
                           "min": round(step_ms[0], 4)},
        "config": {
            "workload": (f"packed thd attention, config {w.name}: {w.batch} sequences, "
                         f"{w.T_q} query tokens / {w.T_kv} kv tokens, h_q={w.h_q} "
                         f"h_kv={w.h_kv} d={w.d} {w.dtype}, {int((w.causal == 2).sum())} "
                         f"bottom-right causal, forward incl. both padding masks"),
            "tokens": int(w.T_q), "batch": w.batch, "valid_pairs": int(pairs),
            "flops_per_step": int(flops), "algorithmic_bytes": int(nbytes), "seed": w.seed,
        },
        "kernel_ms": {"masks": round(mean(mask_ms), 4), "fwd": round(f_ms, 4)},
        "roofline": {"bound": "hbm", "kernel": "thd_attn_fwd (all its launches)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_launch_ms": round(f_ms, 4)},
        "cpu_baseline": None,
    }


if __name__ == "__main__":
    main()

