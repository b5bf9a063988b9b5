"""Glue shared by the GPU parity tests: move a workload to the device, call the
HIP library through its binding, and compare with the oracle to the stated bar
on valid rows -- relative RMS error <= 5e-3 and absolute error <= 2e-2 beyond
the rounding of each value to its storage type (|got - ref| <= 2e-2 + u |ref|,
u = 2^-8 for bf16, 2^-11 for fp16: an exact result stored in bf16 already
misses a flat 2e-2 bound for |ref| > 5.12) -- and pad rows exactly +0."""
import numpy as np
import torch

import variable_length_packed_amd as thd

MAX_ABS = 2e-2
REL_RMS = 5e-3
UNIT_ROUNDOFF = {"bf16": 2.0**-8, "fp16": 2.0**-11, torch.bfloat16: 2.0**-8,
                 torch.float16: 2.0**-11}


def dev_meta(w, device="cuda"):
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.int32)).to(device)
    return dict(
        cu_seqlens_q=t(w.cu_q),
        cu_seqlens_kv=t(w.cu_kv),
        cu_seqlens_q_padded=t(w.cu_q_padded),
        cu_seqlens_kv_padded=t(w.cu_kv_padded),
        is_causal=torch.from_numpy(np.asarray(w.causal, np.uint8)).to(device),
        batch_size=w.batch,
    )


def gpu_fwd(w, q, k, v, meta=None, **kw):
    m = meta or dev_meta(w, q.device)
    return thd.attn_fwd(q, k, v, m["cu_seqlens_q"], m["cu_seqlens_kv"], w.max_seqlen_q,
                        w.max_seqlen_kv, cu_seqlens_q_padded=m["cu_seqlens_q_padded"],
                        cu_seqlens_kv_padded=m["cu_seqlens_kv_padded"],
                        is_causal=m["is_causal"], batch_size=m["batch_size"], **kw)


def gpu_bwd(w, q, k, v, o, do, lse, meta=None, **kw):
    m = meta or dev_meta(w, q.device)
    return thd.attn_bwd(q, k, v, o, do, lse, m["cu_seqlens_q"], m["cu_seqlens_kv"],
                        w.max_seqlen_q, w.max_seqlen_kv,
                        cu_seqlens_q_padded=m["cu_seqlens_q_padded"],
                        cu_seqlens_kv_padded=m["cu_seqlens_kv_padded"],
                        is_causal=m["is_causal"], batch_size=m["batch_size"], **kw)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def errors(got, ref, u=0.0):
    """(max abs error beyond storage rounding, plain max abs error, rel RMS error)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0, 0.0, 0.0
    diff = np.abs(got - ref)
    excess = float((diff - u * np.abs(ref)).max())
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return excess, float(diff.max()), rel


def assert_close(name, got, ref, dtype="bf16", max_abs=MAX_ABS, rel_rms=REL_RMS):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    ex, ma, rr = errors(got, ref, UNIT_ROUNDOFF[dtype])
    assert ex <= max_abs and rr <= rel_rms, \
        f"{name}: abs_err_beyond_rounding={ex:.3e} max_abs={ma:.3e} rel_rms={rr:.3e}"
    return ex, rr


def assert_pad_rows_zero(name, t, valid_rows):
    """Rows outside every sequence must be +0.0 bit for bit."""
    inv = ~np.asarray(valid_rows, bool)
    if not inv.any():
        return
    bits = t.detach().view(torch.int16).cpu().numpy()[inv]
    assert np.all(bits == 0), f"{name}: {int((bits != 0).sum())} nonzero pad elements"
