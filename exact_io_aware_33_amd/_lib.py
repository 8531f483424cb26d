"""ctypes view of libfa's C ABI (include/fa.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_DTYPE_F32, FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_blocksparse", "fa_fwd_splitkv", "fa_fwd_splitkv_num_splits",
           "fa_merge_partials",
           "fa_fwd_splitkv_workspace_bytes", "fa_bwd_workspace_bytes", "fa_bwd",
           "fa_bwd_blocksparse", "fa_bwd_ex", "fa_bwd_noalloc", "fa_softmax_rows", "fa_layernorm_rows",
           "fa_status_string", "fa_last_error", "fa_abi_version")
FA_BWD_PRE, FA_BWD_MAIN, FA_BWD_DQ, FA_BWD_ALL = 1, 2, 4, 7
FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES = 16 << 20
FA_MERGE_MAX_PARTS = 64
ABI_VERSION = 4


class FaProblem(ctypes.Structure):
    """Mirror of fa_problem_t."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_n", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("key_lens", ctypes.c_void_p),
        ("dropout_p", ctypes.c_float),
        ("dropout_offset", ctypes.c_uint32),
        ("dropout_seed", ctypes.c_uint64),
        ("seqlen_k", ctypes.c_int32),
        ("fwd_query_tile", ctypes.c_int32),
        ("k_stride_b", ctypes.c_int64),
        ("k_stride_h", ctypes.c_int64),
        ("k_stride_n", ctypes.c_int64),
    ]


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libfa.so (built in-tree).  Raises if it is missing: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m exact_io_aware_33_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pp = ctypes.POINTER(FaProblem)
    lib.fa_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_blocksparse.argtypes = [pp, vp, i32, i64, vp, vp, vp, vp, vp, vp]
    lib.fa_fwd_blocksparse.restype = i32
    lib.fa_fwd_splitkv.argtypes = [pp, vp, i32, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = i32
    lib.fa_fwd_splitkv_num_splits.argtypes = [pp]
    lib.fa_fwd_splitkv_num_splits.restype = i32
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [pp, i32]
    lib.fa_fwd_splitkv_workspace_bytes.restype = sz
    lib.fa_merge_partials.argtypes = [pp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp]
    lib.fa_merge_partials.restype = i32
    lib.fa_bwd_workspace_bytes.argtypes = [pp]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_blocksparse.argtypes = [pp, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fa_bwd_blocksparse.restype = i32
    lib.fa_bwd_ex.argtypes = [pp, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                              ctypes.c_uint32, vp]
    lib.fa_bwd_ex.restype = i32
    lib.fa_bwd_noalloc.argtypes = [pp, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_softmax_rows.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, vp]
    lib.fa_softmax_rows.restype = i32
    lib.fa_layernorm_rows.argtypes = [i32, i64, i64, vp, i64, vp, vp, ctypes.c_float, i32, i64, vp, i64,
                                      vp, vp, vp]
    lib.fa_layernorm_rows.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i32
    if lib.fa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libfa ABI version {lib.fa_abi_version()} != {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FA_OK:
        lib = load()
        msg = lib.fa_last_error().decode() or lib.fa_status_string(status).decode()
        raise FaError(status, f"{lib.fa_status_string(status).decode()}: {msg}")
