"""Seeded synthetic workloads for packed-thd attention.

This module only draws inputs: sequence lengths, causal flags, slot layouts
and N(0,1) tensors.  It holds none of the attention arithmetic, so the HIP
library's tests, the oracle's tests and the benchmark can all share it.

Recipes (lengths from ``numpy.random.default_rng(seed)``, integer ranges
inclusive; tensors from a seeded ``torch.Generator`` in the order q, k, v, dO,
drawn in float32 and rounded to the storage dtype):

* ``1a`` -- the 19-token layout ``[111aaa222bb3344cccc]`` of the maintainer's
  example in "Add per-sequence causal policy to packed THD attention":
  lengths 3,3,3,2,2,2,4, numbered sequences causal, lettered ones full;
  fp16, h=1, d=8, seed 1.
* ``1b`` -- the issue's 7-token constant example: four tokens of 1.0 then
  three of 2.0 in q, k and v, one pad token of 100 (padded to 8), fp16,
  h=1, d=8, cu_seqlens [0, 7], max_seqlen 8.
* ``2``  -- 16 causal sequences, lengths uniform in [64, 2048], bf16,
  h=16, d=128, contiguous, seed 2 (16,640 tokens).
* ``3``  -- 64 sequences, lengths uniform in [1, 1024], causal flag
  Bernoulli(0.5), each slot rounded up to a multiple of 128 through
  cu_seqlens_padded, pads = 100, bf16, h=32, d=128, seed 3.
* ``4``  -- GQA 32 query / 8 kv heads, all causal, bf16, d=128, lengths
  lognormal(ln 2048, sigma 1.0) rounded, clamped to [1, 32768], drawn until
  the total reaches 131,072 and the last trimmed to hit it exactly, seed 4.
* ``5``  -- cross attention, 32 pairs, q lengths uniform in [1, 512], kv
  lengths uniform in [1, 8192], full (no causal), bf16, h=16, d=128; the
  cu_seqlens buffers hold 2B+1 entries, the extra ones INT32_MAX; seed 5.
* ``6``  -- bottom-right causal (the third mask type of the per-sequence
  causal PR's maintainer review) on the chunked-prefill shape it serves:
  32 sequences, a query chunk of U[64, 512] rows against a key/value history
  of the chunk plus U[0, 4096] earlier rows, bf16, h=16, d=128, seed 6.
  (The pages give no such workload; this one exercises the mask type.)
* ``7``  -- the KV-cache / decode shape: 64 sequences of U[1, 4] new query
  tokens against U[256, 16384] keys (history included), bottom-right causal,
  GQA 32 query / 8 kv heads, bf16, d=128, seed 7.  Also not on the pages;
  it exercises the split-KV forward.
"""

from dataclasses import dataclass, field
import math
from typing import Optional

import numpy as np

INT32_MAX = 2**31 - 1


@dataclass
class Workload:
    name: str
    dtype: str                       # "bf16" | "fp16"
    h_q: int
    h_kv: int
    d: int
    lens_q: np.ndarray               # int64 [B]
    lens_kv: np.ndarray              # int64 [B]
    causal: np.ndarray               # uint8 [B] mask type: 0 padding, 1 top-left
                                     # causal, 2 bottom-right causal
    cu_q: np.ndarray                 # int32, >= B+1 entries
    cu_kv: np.ndarray                # int32, >= B+1 entries
    cu_q_padded: Optional[np.ndarray] = None
    cu_kv_padded: Optional[np.ndarray] = None
    T_q: int = 0
    T_kv: int = 0
    pad_value: float = 100.0
    seed: int = 0
    self_attention: bool = True
    notes: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.lens_q.shape[0])

    @property
    def max_seqlen_q(self):
        return int(self.lens_q.max()) if self.batch else 0

    @property
    def max_seqlen_kv(self):
        return int(self.lens_kv.max()) if self.batch else 0

    def starts_q(self):
        src = self.cu_q if self.cu_q_padded is None else self.cu_q_padded
        return np.asarray(src[:self.batch], dtype=np.int64)

    def starts_kv(self):
        src = self.cu_kv if self.cu_kv_padded is None else self.cu_kv_padded
        return np.asarray(src[:self.batch], dtype=np.int64)

    def row_is_valid_q(self):
        m = np.zeros(self.T_q, dtype=bool)
        for s, n in zip(self.starts_q(), self.lens_q):
            m[s:s + n] = True
        return m

    def row_is_valid_kv(self):
        m = np.zeros(self.T_kv, dtype=bool)
        for s, n in zip(self.starts_kv(), self.lens_kv):
            m[s:s + n] = True
        return m


def _cumsum32(lens, extra=0, fill=INT32_MAX):
    cu = np.zeros(len(lens) + 1 + extra, dtype=np.int64)
    cu[1:len(lens) + 1] = np.cumsum(lens)
    if extra:
        cu[len(lens) + 1:] = fill
    return cu.astype(np.int32)


def packed(lens_q, lens_kv=None, causal=None, *, h_q=1, h_kv=None, d=8,
           dtype="bf16", slot_multiple=None, gap_before=0, extra_cu=0,
           pad_value=100.0, seed=0, name="custom"):
    """Build a Workload from explicit lengths.

    ``slot_multiple`` rounds each sequence slot up to that multiple and passes
    the slot starts as cu_seqlens_padded (shared by q and kv when self
    attention); ``gap_before`` adds that many pad rows before the first slot;
    ``extra_cu`` appends INT32_MAX entries to the cumulative buffers.
    """
    lens_q = np.asarray(lens_q, dtype=np.int64)
    self_attn = lens_kv is None
    lens_kv = lens_q.copy() if self_attn else np.asarray(lens_kv, dtype=np.int64)
    B = len(lens_q)
    causal = np.zeros(B, np.uint8) if causal is None else np.asarray(causal, np.uint8)
    h_kv = h_q if h_kv is None else h_kv
    cu_q = _cumsum32(lens_q, extra_cu)
    cu_kv = cu_q if self_attn else _cumsum32(lens_kv, extra_cu)
    cu_q_pad = cu_kv_pad = None
    if slot_multiple is not None or gap_before:
        def slots(lens):
            sm = slot_multiple or 1
            sl = [((int(n) + sm - 1) // sm) * sm for n in lens]
            st = np.zeros(B + 1 + extra_cu, dtype=np.int64)
            st[0] = gap_before
            st[1:B + 1] = gap_before + np.cumsum(sl)
            if extra_cu:
                st[B + 1:] = INT32_MAX
            return st.astype(np.int32), gap_before + int(np.sum(sl))
        cu_q_pad, T_q = slots(lens_q)
        if self_attn:
            cu_kv_pad, T_kv = cu_q_pad, T_q
        else:
            cu_kv_pad, T_kv = slots(lens_kv)
    else:
        T_q, T_kv = int(lens_q.sum()), int(lens_kv.sum())
    return Workload(name=name, dtype=dtype, h_q=h_q, h_kv=h_kv, d=d,
                    lens_q=lens_q, lens_kv=lens_kv, causal=causal,
                    cu_q=cu_q, cu_kv=cu_kv, cu_q_padded=cu_q_pad,
                    cu_kv_padded=cu_kv_pad, T_q=T_q, T_kv=T_kv,
                    pad_value=pad_value, seed=seed, self_attention=self_attn)


def config(name):
    """The named synthetic configurations (see the module docstring)."""
    name = str(name)
    if name == "1a":
        w = packed([3, 3, 3, 2, 2, 2, 4], causal=[1, 0, 1, 0, 1, 1, 0],
                   h_q=1, d=8, dtype="fp16", seed=1, name="1a")
        return w
    if name == "1b":
        w = packed([7], causal=[0], h_q=1, d=8, dtype="fp16", seed=0, name="1b")
        w.T_q = w.T_kv = 8          # one pad row after the sequence
        w.notes["constant_example"] = True
        return w
    if name == "2":
        rng = np.random.default_rng(2)
        lens = rng.integers(64, 2048, size=16, endpoint=True)
        return packed(lens, causal=np.ones(16, np.uint8), h_q=16, d=128,
                      dtype="bf16", seed=2, name="2")
    if name == "3":
        rng = np.random.default_rng(3)
        lens = rng.integers(1, 1024, size=64, endpoint=True)
        causal = (rng.random(64) < 0.5).astype(np.uint8)
        return packed(lens, causal=causal, h_q=32, d=128, dtype="bf16",
                      slot_multiple=128, seed=3, name="3")
    if name == "4":
        rng = np.random.default_rng(4)
        lens = []
        while sum(lens) < 131072:
            x = int(round(rng.lognormal(math.log(2048), 1.0)))
            lens.append(min(max(x, 1), 32768))
        lens[-1] -= sum(lens) - 131072
        return packed(lens, causal=np.ones(len(lens), np.uint8), h_q=32, h_kv=8,
                      d=128, dtype="bf16", seed=4, name="4")
    if name == "5":
        rng = np.random.default_rng(5)
        lq = rng.integers(1, 512, size=32, endpoint=True)
        lk = rng.integers(1, 8192, size=32, endpoint=True)
        return packed(lq, lk, causal=np.zeros(32, np.uint8), h_q=16, d=128,
                      dtype="bf16", extra_cu=32, seed=5, name="5")
    if name == "6":
        rng = np.random.default_rng(6)
        lq = rng.integers(64, 512, size=32, endpoint=True)
        lk = lq + rng.integers(0, 4096, size=32, endpoint=True)
        return packed(lq, lk, causal=np.full(32, 2, np.uint8), h_q=16, d=128,
                      dtype="bf16", seed=6, name="6")
    if name == "7":
        rng = np.random.default_rng(7)
        lq = rng.integers(1, 4, size=64, endpoint=True)
        lk = rng.integers(256, 16384, size=64, endpoint=True)
        return packed(lq, lk, causal=np.full(64, 2, np.uint8), h_q=32, h_kv=8, d=128,
                      dtype="bf16", seed=7, name="7")
    raise KeyError(name)


def random_layout(seed, batch, max_len, *, h_q=2, h_kv=None, d=64,
                  dtype="bf16", causal="mixed", cross=False, slot_multiple=None,
                  gap_before=0, extra_cu=0, min_len=0, name=None):
    """A small random layout for parity tests (ragged lengths, zeros allowed)."""
    rng = np.random.default_rng(seed)
    lq = rng.integers(min_len, max_len, size=batch, endpoint=True)
    lk = rng.integers(min_len, max_len, size=batch, endpoint=True) if cross else None
    if causal == "mixed":
        flags = (rng.random(batch) < 0.5).astype(np.uint8)
    elif causal == "types":  # all three mask types
        flags = rng.integers(0, 2, size=batch, endpoint=True).astype(np.uint8)
    elif causal in ("all", True):
        flags = np.ones(batch, np.uint8)
    else:
        flags = np.zeros(batch, np.uint8)
    return packed(lq, lk, flags, h_q=h_q, h_kv=h_kv, d=d, dtype=dtype,
                  slot_multiple=slot_multiple, gap_before=gap_before,
                  extra_cu=extra_cu, seed=seed, name=name or f"rand{seed}")


def torch_dtype(w):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]


def make_tensors(w, device="cpu", with_dout=True):
    """Seeded q, k, v (and dO) for a workload, pads set to ``pad_value``.

    Returns torch tensors of the workload's dtype on ``device``.
    """
    import torch
    dt = torch_dtype(w)
    if w.notes.get("constant_example"):
        q = torch.full((w.T_q, w.h_q, w.d), w.pad_value, dtype=torch.float32)
        q[0:4] = 1.0
        q[4:7] = 2.0
        k = q.clone()
        v = q.clone()
        g = torch.Generator("cpu").manual_seed(w.seed)
        dout = torch.randn((w.T_q, w.h_q, w.d), generator=g, dtype=torch.float32)
        out = [t.to(dt).to(device) for t in (q, k, v, dout)]
        return tuple(out) if with_dout else tuple(out[:3])
    gen_dev = torch.device(device)
    g = torch.Generator(gen_dev.type if gen_dev.type != "cuda" else gen_dev)
    g.manual_seed(int(w.seed))
    shape_q = (w.T_q, w.h_q, w.d)
    shape_k = (w.T_kv, w.h_kv, w.d)
    ts = []
    for shape in (shape_q, shape_k, shape_k, shape_q):
        ts.append(torch.randn(shape, generator=g, dtype=torch.float32,
                              device=gen_dev).to(dt))
    q, k, v, dout = ts
    vq = torch.from_numpy(w.row_is_valid_q()).to(gen_dev)
    vk = torch.from_numpy(w.row_is_valid_kv()).to(gen_dev)
    q[~vq] = w.pad_value
    dout[~vq] = w.pad_value
    k[~vk] = w.pad_value
    v[~vk] = w.pad_value
    return (q, k, v, dout) if with_dout else (q, k, v)
