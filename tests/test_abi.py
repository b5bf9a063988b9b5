"""C ABI: the library loads, exports every declared entry point, and rejects
invalid host arguments before launching anything (CPU only, no GPU calls)."""
import ctypes
import os
import re

import pytest

from variable_length_packed_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "thd_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(thd_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("thd_attn_fwd", "thd_attn_bwd", "thd_padding_mask", "thd_attn_fwd_workspace_size",
              "thd_attn_bwd_workspace_size", "thd_status_string", "thd_version"):
        assert n in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert lib.thd_version() >= 100
    assert lib.thd_status_string(0) == b"THD_OK"
    assert lib.thd_status_string(-4).startswith(b"THD_ERR_WORKSPACE")


def _args(**kw):
    a = _lib.ThdVarlenArgs()
    dummy = ctypes.c_void_p(0x1000)
    a.cu_seqlens_q = dummy
    a.cu_seqlens_kv = dummy
    a.batch = 2
    a.max_seqlen_q = a.max_seqlen_kv = 8
    a.total_q = a.total_kv = 16
    a.h_q, a.h_kv, a.head_dim = 4, 2, 64
    a.softmax_scale = 0.0
    a.dtype = _lib.THD_BF16
    for k, v in kw.items():
        setattr(a, k, v)
    return a


P = ctypes.c_void_p(0x2000)   # never dereferenced: every call below fails validation


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), -2),
    (dict(h_q=3, h_kv=2), -2),
    (dict(h_kv=0), -2),
    (dict(total_q=-5), -2),
    (dict(max_seqlen_kv=-1), -2),
    (dict(head_dim=12), -3),
    (dict(head_dim=264), -3),
    (dict(head_dim=252), -3),
    (dict(head_dim=0), -3),
    (dict(dtype=7), -3),
    (dict(cu_seqlens_q=None), -1),
])
def test_fwd_rejects_invalid_arguments(kw, status):
    lib = _lib.load()
    a = _args(**kw)
    assert lib.thd_attn_fwd(ctypes.byref(a), P, P, P, P, P, P, 1 << 30, None) == status
    assert lib.thd_attn_bwd(ctypes.byref(a), P, P, P, P, P, P, P, P, P, P, 1 << 30, None) == status


def test_sequence_size_limits():
    # 32-bit byte offsets per sequence: q / k / v rows of max_seqlen rows must
    # stay below 2^31 bytes, in the forward and the backward alike.
    lib = _lib.load()
    fwd = lambda a: lib.thd_attn_fwd(ctypes.byref(a), P, P, P, P, P, P, 1 << 30, None)
    bwd = lambda a: lib.thd_attn_bwd(ctypes.byref(a), P, P, P, P, P, P, P, P, P, P, 1 << 30, None)
    big_q = dict(max_seqlen_q=(1 << 31) // (4 * 64 * 2), total_q=1 << 20)   # q rows hit 2^31
    assert fwd(_args(**big_q)) == -2 and bwd(_args(**big_q)) == -2
    big_kv = dict(max_seqlen_kv=(1 << 31) // (2 * 64 * 2), total_kv=1 << 21)
    assert fwd(_args(**big_kv)) == -2 and bwd(_args(**big_kv)) == -2
    wide_q = dict(max_seqlen_q=(1 << 31) // (4 * 256 * 2), total_q=1 << 20, head_dim=256)
    assert fwd(_args(**wide_q)) == -2 and bwd(_args(**wide_q)) == -2
    assert lib.thd_attn_bwd_workspace_size(ctypes.byref(_args(**wide_q))) == 0
    # one row fewer passes the size checks in both directions and stops at
    # the (empty) workspace, before anything could be launched with the
    # placeholder pointers
    fits = dict(wide_q, max_seqlen_q=wide_q["max_seqlen_q"] - 1)
    assert lib.thd_attn_fwd_workspace_size(ctypes.byref(_args(**fits))) > 0
    assert lib.thd_attn_bwd_workspace_size(ctypes.byref(_args(**fits))) > 0
    assert lib.thd_attn_fwd(ctypes.byref(_args(**fits)), P, P, P, P, P, P, 0, None) == -4
    assert lib.thd_attn_bwd(ctypes.byref(_args(**fits)), P, P, P, P, P, P, P, P, P, P, 0,
                            None) == -4


def test_null_and_misaligned_tensors():
    lib = _lib.load()
    a = _args()
    big = 1 << 30
    assert lib.thd_attn_fwd(ctypes.byref(a), None, P, P, P, P, P, big, None) == -1
    assert lib.thd_attn_fwd(ctypes.byref(a), P, P, P, P, None, P, big, None) == -1
    odd = ctypes.c_void_p(0x2002)
    assert lib.thd_attn_fwd(ctypes.byref(a), odd, P, P, P, P, P, big, None) == -3
    assert lib.thd_attn_fwd(None, P, P, P, P, P, P, big, None) == -1


def test_fwd_workspace_size_and_check():
    lib = _lib.load()
    a = _args()
    need = lib.thd_attn_fwd_workspace_size(ctypes.byref(a))
    # item count and (sequence, tile) pairs for up to T_q/128 + batch query tiles
    assert need >= (2 + 2 * (1 + 2)) * 4
    assert lib.thd_attn_fwd_workspace_size(ctypes.byref(_args(batch=-1))) == 0
    assert lib.thd_attn_fwd_workspace_size(ctypes.byref(_args(batch=0))) == 0
    assert lib.thd_attn_fwd(ctypes.byref(a), P, P, P, P, P, P, need - 1, None) == -4
    assert lib.thd_attn_fwd(ctypes.byref(a), P, P, P, P, P, None, need, None) == -4
    mis = ctypes.c_void_p(0x2010)
    assert lib.thd_attn_fwd(ctypes.byref(a), P, P, P, P, P, mis, need, None) == -4


def test_noalloc_forward_host_checks():
    # the forward that allocates nothing rejects, before any launch, a problem
    # whose workspace exceeds its fixed device array, and validates like the
    # forward
    lib = _lib.load()
    big = _args(batch=1, max_seqlen_q=64, max_seqlen_kv=64, total_q=300_000_000,
                total_kv=16, h_q=1, h_kv=1, head_dim=8)
    assert lib.thd_attn_fwd_workspace_size(ctypes.byref(big)) > _lib.FWD_NOALLOC_MAX_WORKSPACE
    assert lib.thd_attn_fwd_noalloc(ctypes.byref(big), P, P, P, P, P, None) == -4
    assert lib.thd_attn_fwd_noalloc(ctypes.byref(_args(batch=-1)), P, P, P, P, P, None) == -2
    assert lib.thd_attn_fwd_noalloc(ctypes.byref(_args(head_dim=12)), P, P, P, P, P, None) == -3
    assert lib.thd_attn_fwd_noalloc(ctypes.byref(_args()), None, P, P, P, P, None) == -1
    assert lib.thd_attn_fwd_noalloc(None, P, P, P, P, P, None) == -1


def test_workspace_size_and_check():
    lib = _lib.load()
    a = _args()
    need = lib.thd_attn_bwd_workspace_size(ctypes.byref(a))
    # two fp32 row statistics [h_q, T_q], the dq pass's schedule of query
    # tiles and the dk/dv pass's of key tiles; nothing that grows with the
    # head dim
    assert need >= 2 * 16 * 4 * 4 + 2 * (8 + 8 * (1 + 2)) * 4
    for d in (8, 128, 192, 256):
        assert lib.thd_attn_bwd_workspace_size(ctypes.byref(_args(head_dim=d))) == need
    assert lib.thd_attn_bwd_workspace_size(ctypes.byref(_args(batch=-1))) == 0
    assert lib.thd_attn_bwd(ctypes.byref(a), P, P, P, P, P, P, P, P, P, P, need - 1, None) == -4
    assert lib.thd_attn_bwd(ctypes.byref(a), P, P, P, P, P, P, P, P, P, None, need, None) == -4
    mis = ctypes.c_void_p(0x2010)
    assert lib.thd_attn_bwd(ctypes.byref(a), P, P, P, P, P, P, P, P, P, mis, need, None) == -4


def test_padding_mask_host_checks():
    lib = _lib.load()
    assert lib.thd_padding_mask(P, -1, 4, P, None) == -2
    assert lib.thd_padding_mask(P, 2, -1, P, None) == -2
    assert lib.thd_padding_mask(None, 2, 4, P, None) == -1
    assert lib.thd_padding_mask(P, 2, 4, None, None) == -1
    # nothing to do: returns before any launch
    assert lib.thd_padding_mask(None, 0, 4, None, None) == 0
    assert lib.thd_padding_mask(None, 3, 0, None, None) == 0


def test_padding_mask_pair_host_checks():
    lib = _lib.load()
    m = lib.thd_padding_masks
    assert m(P, P, -1, 4, 4, P, P, None) == -2
    assert m(P, P, 2, -1, 4, P, P, None) == -2
    assert m(P, P, 2, 4, -1, P, P, None) == -2
    assert m(None, P, 2, 4, 4, P, P, None) == -1
    assert m(P, None, 2, 4, 4, P, P, None) == -1
    assert m(P, P, 2, 4, 4, None, P, None) == -1
    assert m(P, P, 2, 4, 4, P, None, None) == -1
    # a mask with no bytes needs no pointers; with none at all nothing launches
    assert m(None, None, 0, 4, 4, None, None, None) == 0
    assert m(None, None, 3, 0, 0, None, None, None) == 0


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "libthdattn.so"))
