"""torch-facing wrappers of the C ABI: packed-thd attention and its padding mask.

Tensor layout follows the Megatron-LM issue "How to pad sequences that cannot
be evenly split in context parallelism (CP)?" (packed ``thd`` q/k/v of shape
[T, h, d] with int32 ``cu_seqlens``); the per-sequence causal flag and
``cu_seqlens_padded`` follow TransformerEngine PR "Add per-sequence causal
policy to packed THD attention".  These functions only check host-visible
properties (device, dtype, shape, contiguity), allocate outputs with torch and
pass raw pointers plus the current HIP stream to libthdattn.so; they never read
device data, so no call synchronises with the host.
"""
import torch

from . import _lib

__all__ = ["padding_mask", "padding_masks", "attn_fwd", "attn_bwd", "bwd_workspace_size", "thd_attention"]

_DTYPES = {torch.float16: _lib.THD_FP16, torch.bfloat16: _lib.THD_BF16}


def _stream(device):
    return ctypes_void(torch.cuda.current_stream(device).cuda_stream)


def ctypes_void(x):
    import ctypes
    return ctypes.c_void_p(int(x)) if x else None


def _ptr(t):
    return ctypes_void(t.data_ptr()) if t is not None and t.numel() > 0 else None


# Device type every tensor argument must live on (the library's kernels run
# on the GPU; the host-side checks below are exercised on the CPU by
# replacing this with "cpu").
_DEVICE_TYPE = "cuda"


def _require_cuda(name, t, dtype=None, shape=None, device=None):
    """Host-visible checks of one tensor argument: type, device, dtype, shape,
    contiguity.  Raises before anything is launched."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_workspace(workspace, need, device):
    _require_cuda("workspace", workspace, torch.uint8, device=device)
    if workspace.numel() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")


def padding_mask(cu_seqlens, batch_size, max_seqlen):
    """Bool mask [batch_size, 1, 1, max_seqlen], True at pad positions.

    Built by one device kernel from ``cu_seqlens`` (entries past
    batch_size + 1 are ignored), with no host synchronisation -- TransformerEngine
    PR "[PyTorch] Build the attention padding mask without host syncs".
    """
    _require_cuda("cu_seqlens", cu_seqlens, torch.int32)
    batch_size, max_seqlen = int(batch_size), int(max_seqlen)
    if batch_size < 0 or max_seqlen < 0:
        raise ValueError("batch_size and max_seqlen must be >= 0")
    if batch_size > 0 and cu_seqlens.numel() < batch_size + 1:
        raise ValueError("cu_seqlens needs at least batch_size + 1 entries")
    mask = torch.empty((batch_size, 1, 1, max_seqlen), dtype=torch.bool,
                       device=cu_seqlens.device)
    lib = _lib.load()
    st = lib.thd_padding_mask(_ptr(cu_seqlens), batch_size, max_seqlen, _ptr(mask),
                              _stream(cu_seqlens.device))
    _lib.check(st, "thd_padding_mask")
    return mask


def padding_masks(cu_seqlens_q, cu_seqlens_kv, batch_size, max_seqlen_q, max_seqlen_kv):
    """The query and key/value masks of ``padding_mask`` ([batch_size, 1, 1,
    max_seqlen_q] and [batch_size, 1, 1, max_seqlen_kv]) built by one kernel
    launch -- the attention_mask_q / attention_mask_kv pair of
    TransformerEngine PR "[PyTorch] Build the attention padding mask without
    host syncs"."""
    _require_cuda("cu_seqlens_q", cu_seqlens_q, torch.int32)
    _require_cuda("cu_seqlens_kv", cu_seqlens_kv, torch.int32, device=cu_seqlens_q.device)
    batch_size = int(batch_size)
    max_seqlen_q, max_seqlen_kv = int(max_seqlen_q), int(max_seqlen_kv)
    if batch_size < 0 or max_seqlen_q < 0 or max_seqlen_kv < 0:
        raise ValueError("batch_size and the max_seqlens must be >= 0")
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if batch_size > 0 and cu.numel() < batch_size + 1:
            raise ValueError(f"{name} needs at least batch_size + 1 entries")
    dev = cu_seqlens_q.device
    mq = torch.empty((batch_size, 1, 1, max_seqlen_q), dtype=torch.bool, device=dev)
    mkv = torch.empty((batch_size, 1, 1, max_seqlen_kv), dtype=torch.bool, device=dev)
    lib = _lib.load()
    st = lib.thd_padding_masks(_ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), batch_size, max_seqlen_q,
                               max_seqlen_kv, _ptr(mq), _ptr(mkv), _stream(dev))
    _lib.check(st, "thd_padding_masks")
    return mq, mkv


def _make_args(q, k, cu_q, cu_kv, max_q, max_kv, cu_q_pad, cu_kv_pad, is_causal,
               softmax_scale, batch_size):
    _require_cuda("q", q, tuple(_DTYPES))
    _require_cuda("k", k, q.dtype, device=q.device)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [T, h, d]")
    if q.shape[2] != k.shape[2]:
        raise ValueError("q and k must share head_dim")
    for name, t in (("cu_seqlens_q", cu_q), ("cu_seqlens_kv", cu_kv),
                    ("cu_seqlens_q_padded", cu_q_pad), ("cu_seqlens_kv_padded", cu_kv_pad)):
        if t is not None:
            _require_cuda(name, t, torch.int32, device=q.device)
    if batch_size is None:
        batch_size = cu_q.numel() - 1
    batch_size = int(batch_size)
    if batch_size < 0:
        raise ValueError("batch_size must be >= 0")
    for name, t in (("cu_seqlens_q", cu_q), ("cu_seqlens_kv", cu_kv),
                    ("cu_seqlens_q_padded", cu_q_pad), ("cu_seqlens_kv_padded", cu_kv_pad)):
        if t is not None and t.numel() < batch_size + (0 if "padded" in name else 1):
            raise ValueError(f"{name} is shorter than the batch")
    if is_causal is not None:
        _require_cuda("mask_type", is_causal, (torch.bool, torch.uint8), device=q.device)
        if is_causal.numel() < batch_size:
            raise ValueError("mask_type / is_causal needs one entry per sequence")
    a = _lib.ThdVarlenArgs()
    a.cu_seqlens_q = _ptr(cu_q)
    a.cu_seqlens_kv = _ptr(cu_kv)
    a.cu_seqlens_q_padded = _ptr(cu_q_pad)
    a.cu_seqlens_kv_padded = _ptr(cu_kv_pad)
    a.mask_type = _ptr(is_causal)
    a.batch = batch_size
    a.max_seqlen_q = int(max_q)
    a.max_seqlen_kv = int(max_kv)
    a.total_q = q.shape[0]
    a.total_kv = k.shape[0]
    a.h_q = q.shape[1]
    a.h_kv = k.shape[1]
    a.head_dim = q.shape[2]
    a.softmax_scale = float(softmax_scale) if softmax_scale is not None else 0.0
    a.dtype = _DTYPES[q.dtype]
    return a


def _mask_arg(is_causal, mask_type):
    if mask_type is not None:
        if is_causal is not None:
            raise ValueError("give mask_type or is_causal, not both")
        return mask_type
    return is_causal


def attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, *,
             cu_seqlens_q_padded=None, cu_seqlens_kv_padded=None, is_causal=None,
             softmax_scale=None, batch_size=None, out=None, lse=None, workspace=None,
             mask_type=None):
    """Forward attention; returns (out [T_q,h_q,d], lse [h_q,T_q] fp32).

    ``mask_type``: one uint8 per sequence, MASK_PADDING / MASK_CAUSAL (top-left) /
    MASK_CAUSAL_BOTTOM_RIGHT (None = all ``padding``); ``is_causal`` (one
    bool/uint8 per sequence) is the same argument under its older name.
    ``softmax_scale``: None = 1/sqrt(head_dim).  ``batch_size``: number of
    sequences when the cu_seqlens buffers are longer than batch + 1.
    ``workspace``: uint8 device buffer of at least ``fwd_workspace_size``
    bytes (allocated here when None).
    """
    is_causal = _mask_arg(is_causal, mask_type)
    a = _make_args(q, k, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                   cu_seqlens_q_padded, cu_seqlens_kv_padded, is_causal, softmax_scale,
                   batch_size)
    _require_cuda("v", v, q.dtype, shape=k.shape, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    _require_cuda("out", out, q.dtype, shape=q.shape, device=q.device)
    _require_cuda("lse", lse, torch.float32, shape=(q.shape[1], q.shape[0]), device=q.device)
    lib = _lib.load()
    need = int(lib.thd_attn_fwd_workspace_size(a))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _require_workspace(workspace, need, q.device)
    st = lib.thd_attn_fwd(a, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace),
                          workspace.numel(), _stream(q.device))
    _lib.check(st, "thd_attn_fwd")
    return out, lse


def fwd_workspace_size(q, k, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                       batch_size=None):
    """Bytes of workspace ``attn_fwd`` needs (the split-KV path for few query
    rows per sequence sizes it from the max_seqlen bounds)."""
    a = _make_args(q, k, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, None, None,
                   None, None, batch_size)
    return int(_lib.load().thd_attn_fwd_workspace_size(a))


def bwd_workspace_size(q, k, cu_seqlens_q, cu_seqlens_kv, batch_size=None):
    a = _make_args(q, k, cu_seqlens_q, cu_seqlens_kv, 0, 0, None, None, None, None, batch_size)
    return int(_lib.load().thd_attn_bwd_workspace_size(a))


def attn_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
             max_seqlen_kv, *, cu_seqlens_q_padded=None, cu_seqlens_kv_padded=None,
             is_causal=None, softmax_scale=None, batch_size=None, workspace=None,
             dq=None, dk=None, dv=None, mask_type=None):
    """Backward attention; returns (dq, dk, dv).  Arguments as ``attn_fwd``;
    ``dq``, ``dk``, ``dv`` (optional outputs) must have the dtype, shape and
    device of q, k, v.  Every tensor is checked before anything is launched."""
    is_causal = _mask_arg(is_causal, mask_type)
    a = _make_args(q, k, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv,
                   cu_seqlens_q_padded, cu_seqlens_kv_padded, is_causal, softmax_scale,
                   batch_size)
    dev = q.device
    for name, t, like in (("v", v, k), ("out", out, q), ("dout", dout, q)):
        _require_cuda(name, t, q.dtype, shape=like.shape, device=dev)
    _require_cuda("lse", lse, torch.float32, shape=(q.shape[1], q.shape[0]), device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _require_cuda(name, t, q.dtype, shape=like.shape, device=dev)
    lib = _lib.load()
    need = int(lib.thd_attn_bwd_workspace_size(a))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _require_workspace(workspace, need, dev)
    st = lib.thd_attn_bwd(a, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                          _stream(dev))
    _lib.check(st, "thd_attn_bwd")
    return dq, dk, dv


class _ThdAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_q, cu_kv, max_q, max_kv, cu_q_pad, cu_kv_pad, is_causal,
                scale, batch_size):
        out, lse = attn_fwd(q, k, v, cu_q, cu_kv, max_q, max_kv, cu_seqlens_q_padded=cu_q_pad,
                            cu_seqlens_kv_padded=cu_kv_pad, is_causal=is_causal,
                            softmax_scale=scale, batch_size=batch_size)
        ctx.save_for_backward(q, k, v, out, lse, cu_q, cu_kv, cu_q_pad, cu_kv_pad, is_causal)
        ctx.meta = (max_q, max_kv, scale, batch_size)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, cu_q, cu_kv, cu_q_pad, cu_kv_pad, is_causal = ctx.saved_tensors
        max_q, max_kv, scale, batch_size = ctx.meta
        dq, dk, dv = attn_bwd(q, k, v, out, dout.contiguous(), lse, cu_q, cu_kv, max_q, max_kv,
                              cu_seqlens_q_padded=cu_q_pad, cu_seqlens_kv_padded=cu_kv_pad,
                              is_causal=is_causal, softmax_scale=scale, batch_size=batch_size)
        return dq, dk, dv, None, None, None, None, None, None, None, None, None


def thd_attention(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q, max_seqlen_kv, *,
                  cu_seqlens_q_padded=None, cu_seqlens_kv_padded=None, is_causal=None,
                  softmax_scale=None, batch_size=None, mask_type=None):
    """Autograd-enabled packed-thd attention (forward and backward in HIP)."""
    return _ThdAttention.apply(q, k, v, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q,
                               max_seqlen_kv, cu_seqlens_q_padded, cu_seqlens_kv_padded,
                               _mask_arg(is_causal, mask_type), softmax_scale, batch_size)


MASK_PADDING = 0
MASK_CAUSAL = 1
MASK_CAUSAL_BOTTOM_RIGHT = 2
