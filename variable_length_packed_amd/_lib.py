"""ctypes binding of libthdattn.so (C ABI in include/thd_attn.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  The library
must have been built (``variable_length_packed_amd.build``); loading fails
loudly otherwise -- there is no fallback path.
"""
import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libthdattn.so")

THD_FP16 = 0
THD_BF16 = 1

# THD_FWD_NOALLOC_MAX_WORKSPACE of include/thd_attn.h
FWD_NOALLOC_MAX_WORKSPACE = 16 << 20

STATUS = {
    0: "THD_OK",
    -1: "THD_ERR_NULL",
    -2: "THD_ERR_SHAPE",
    -3: "THD_ERR_UNSUPPORTED",
    -4: "THD_ERR_WORKSPACE",
    -5: "THD_ERR_HIP",
}

# Every entry point declared in include/thd_attn.h.
EXPORTED = (
    "thd_padding_mask",
    "thd_padding_masks",
    "thd_attn_fwd_workspace_size",
    "thd_attn_fwd",
    "thd_attn_fwd_noalloc",
    "thd_attn_bwd_workspace_size",
    "thd_attn_bwd",
    "thd_attn_bwd_timed",
    "thd_status_string",
    "thd_version",
)


class ThdVarlenArgs(ctypes.Structure):
    """Mirror of ``thd_varlen_args``."""
    _fields_ = [
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_kv", ctypes.c_void_p),
        ("cu_seqlens_q_padded", ctypes.c_void_p),
        ("cu_seqlens_kv_padded", ctypes.c_void_p),
        ("mask_type", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_kv", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class ThdError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_LIB = None


def load(path=None):
    """Load (once) and return the ctypes handle of libthdattn.so."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build it with `python -m variable_length_packed_amd.build` "
            "(the attention path has no fallback)")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    argsp = ctypes.POINTER(ThdVarlenArgs)
    lib.thd_padding_mask.argtypes = [vp, i32, i32, vp, vp]
    lib.thd_padding_mask.restype = ctypes.c_int
    lib.thd_padding_masks.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.thd_padding_masks.restype = ctypes.c_int
    lib.thd_attn_fwd_workspace_size.argtypes = [argsp]
    lib.thd_attn_fwd_workspace_size.restype = sz
    lib.thd_attn_fwd.argtypes = [argsp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.thd_attn_fwd.restype = ctypes.c_int
    lib.thd_attn_fwd_noalloc.argtypes = [argsp, vp, vp, vp, vp, vp, vp]
    lib.thd_attn_fwd_noalloc.restype = ctypes.c_int
    lib.thd_attn_bwd_workspace_size.argtypes = [argsp]
    lib.thd_attn_bwd_workspace_size.restype = sz
    lib.thd_attn_bwd.argtypes = [argsp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.thd_attn_bwd.restype = ctypes.c_int
    lib.thd_attn_bwd_timed.argtypes = [argsp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                       ctypes.POINTER(vp)]
    lib.thd_attn_bwd_timed.restype = ctypes.c_int
    lib.thd_status_string.argtypes = [ctypes.c_int]
    lib.thd_status_string.restype = ctypes.c_char_p
    lib.thd_version.argtypes = []
    lib.thd_version.restype = ctypes.c_int
    if path is None:
        _LIB = lib
    return lib


def check(status, where):
    if status != 0:
        raise ThdError(status, where)
