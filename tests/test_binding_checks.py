"""The torch binding checks every tensor argument (device, dtype, shape,
contiguity, workspace size) on the host and raises before anything is
launched: the C ABI sees only raw pointers, so a wrong-shaped buffer would
otherwise become an out-of-bounds access on the device.  Runs on the CPU: the
binding's device requirement is pointed at "cpu" and the library is replaced
by a stub whose launch entry points fail the test if they are reached."""
import pytest
import torch

from variable_length_packed_amd import _lib, attention


class _Launched(Exception):
    pass


class _StubLib:
    def thd_attn_fwd_workspace_size(self, a):
        return 64

    def thd_attn_bwd_workspace_size(self, a):
        return 4096

    def thd_attn_fwd(self, *args):
        raise _Launched("thd_attn_fwd")

    def thd_attn_bwd(self, *args):
        raise _Launched("thd_attn_bwd")

    def thd_padding_mask(self, *args):
        raise _Launched("thd_padding_mask")

    def thd_padding_masks(self, *args):
        raise _Launched("thd_padding_masks")


@pytest.fixture
def host(monkeypatch):
    monkeypatch.setattr(attention, "_DEVICE_TYPE", "cpu")
    monkeypatch.setattr(_lib, "load", lambda path=None: _StubLib())
    monkeypatch.setattr(attention, "_stream", lambda device: None)


T_Q, T_KV, H_Q, H_KV, D = 12, 10, 4, 2, 16


def _inputs(dtype=torch.bfloat16):
    q = torch.zeros(T_Q, H_Q, D, dtype=dtype)
    k = torch.zeros(T_KV, H_KV, D, dtype=dtype)
    v = torch.zeros(T_KV, H_KV, D, dtype=dtype)
    cu_q = torch.tensor([0, 5, 12], dtype=torch.int32)
    cu_kv = torch.tensor([0, 4, 10], dtype=torch.int32)
    return q, k, v, cu_q, cu_kv


def _bwd(**over):
    q, k, v, cu_q, cu_kv = _inputs()
    args = dict(q=q, k=k, v=v, out=torch.zeros_like(q), dout=torch.zeros_like(q),
                lse=torch.zeros(H_Q, T_Q, dtype=torch.float32))
    kw = {}
    for name, val in over.items():
        (args if name in args else kw)[name] = val
    return attention.attn_bwd(args["q"], args["k"], args["v"], args["out"], args["dout"],
                              args["lse"], cu_q, cu_kv, 7, 6, **kw)


def test_valid_backward_arguments_reach_the_launch(host):
    with pytest.raises(_Launched):
        _bwd()


def test_valid_forward_arguments_reach_the_launch(host):
    q, k, v, cu_q, cu_kv = _inputs()
    with pytest.raises(_Launched):
        attention.attn_fwd(q, k, v, cu_q, cu_kv, 7, 6)


@pytest.mark.parametrize("over,exc", [
    (dict(lse=torch.zeros(T_Q, H_Q)), ValueError),                       # transposed lse
    (dict(lse=torch.zeros(H_Q, T_Q, dtype=torch.float64)), TypeError),
    (dict(out=torch.zeros(T_Q, H_Q, 8, dtype=torch.bfloat16)), ValueError),
    (dict(dout=torch.zeros(T_Q, H_Q, D, dtype=torch.float16)), TypeError),
    (dict(v=torch.zeros(T_KV + 1, H_KV, D, dtype=torch.bfloat16)), ValueError),
    (dict(dq=torch.zeros(T_Q, H_Q, D, dtype=torch.float16)), TypeError),
    (dict(dq=torch.zeros(T_Q - 1, H_Q, D, dtype=torch.bfloat16)), ValueError),
    (dict(dk=torch.zeros(T_KV, H_KV, D + 8, dtype=torch.bfloat16)), ValueError),
    (dict(dv=torch.zeros(D, H_KV, T_KV, dtype=torch.bfloat16).transpose(0, 2)), ValueError),
    (dict(dv=torch.zeros(T_KV, H_KV, D, dtype=torch.bfloat16, device="meta")), ValueError),
    (dict(dq=[0.0]), TypeError),
    (dict(workspace=torch.zeros(100, dtype=torch.uint8)), ValueError),    # too small
    (dict(workspace=torch.zeros(4096, dtype=torch.int32)), TypeError),
])
def test_backward_rejects_bad_tensors_before_launch(host, over, exc):
    with pytest.raises(exc):
        _bwd(**over)


@pytest.mark.parametrize("over,exc", [
    (dict(out=torch.zeros(T_Q, H_Q, D, dtype=torch.float16)), TypeError),
    (dict(out=torch.zeros(T_Q, H_Q + 1, D, dtype=torch.bfloat16)), ValueError),
    (dict(lse=torch.zeros(T_Q, H_Q)), ValueError),
    (dict(workspace=torch.zeros(8, dtype=torch.uint8)), ValueError),
])
def test_forward_rejects_bad_tensors_before_launch(host, over, exc):
    q, k, v, cu_q, cu_kv = _inputs()
    with pytest.raises(exc):
        attention.attn_fwd(q, k, v, cu_q, cu_kv, 7, 6, **over)


def test_metadata_must_be_int32_on_the_same_device(host):
    q, k, v, cu_q, cu_kv = _inputs()
    with pytest.raises(TypeError):
        attention.attn_fwd(q, k, v, cu_q.long(), cu_kv, 7, 6)
    with pytest.raises(ValueError):
        attention.attn_fwd(q, k, v, cu_q, cu_kv.to("meta"), 7, 6)


@pytest.mark.parametrize("kw,exc", [
    (dict(batch_size=-1), ValueError),
    (dict(max_seqlen_q=-2), ValueError),
    (dict(max_seqlen_kv=-1), ValueError),
    (dict(cu_seqlens_q=torch.tensor([0, 5], dtype=torch.int32)), ValueError),   # too short
    (dict(cu_seqlens_kv=torch.tensor([0, 4, 10], dtype=torch.int64)), TypeError),
])
def test_mask_pair_rejects_bad_arguments_before_launch(host, kw, exc):
    args = dict(cu_seqlens_q=torch.tensor([0, 5, 12], dtype=torch.int32),
                cu_seqlens_kv=torch.tensor([0, 4, 10], dtype=torch.int32),
                batch_size=2, max_seqlen_q=7, max_seqlen_kv=6)
    args.update(kw)
    with pytest.raises(exc):
        attention.padding_masks(**args)


def test_mask_pair_valid_arguments_reach_the_launch(host):
    with pytest.raises(_Launched, match="thd_padding_masks"):
        attention.padding_masks(torch.tensor([0, 5, 12], dtype=torch.int32),
                                torch.tensor([0, 4, 10], dtype=torch.int32), 2, 7, 6)

