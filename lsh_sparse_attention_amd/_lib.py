"""ctypes loader of liblsh.so (the C ABI declared in include/lsh.h).

Loading fails loudly if the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsh.so")

# Exported symbols, in header order.
SYMBOLS = ("lsh_status_string", "lsh_version", "lsh_workspace_bytes", "lsh_hash", "lsh_sort",
           "lsh_sort_noalloc", "lsh_attn_fwd", "lsh_combine", "lsh_attn_bwd", "lsh_attn_bwd_saved", "lsh_attn_bwd_rehash",
           "lsh_kernel_name", "lsh_profile_kernel", "lsh_ff_workspace_bytes", "lsh_ff_fwd", "lsh_ff_bwd")

KERNELS = ("hash", "sort_count", "sort_scatter", "prep", "attn_fwd", "combine", "bwd_dq", "bwd_dkv",
           "bwd_reduce", "tiles")

LSH_OK, LSH_ERR_INVALID, LSH_ERR_UNSUPPORTED, LSH_ERR_HIP = 0, 1, 2, 3
LSH_F32, LSH_BF16 = 0, 1
LSH_WS_SORT, LSH_WS_FWD, LSH_WS_BWD, LSH_WS_TRAIN, LSH_WS_REHASH = 0, 1, 2, 3, 4
LSH_FLAG_NO_BUCKET_MASK, LSH_FLAG_DUP_BY_BUCKET = 1, 2
LSH_SORT_NOALLOC_MAX_BYTES = 16 << 20


class Problem(ctypes.Structure):
    """Mirror of lsh_problem_t."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_hashes", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("chunk_len", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class FF(ctypes.Structure):
    """Mirror of lsh_ff_t."""
    _fields_ = [("rows", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("chunks", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class LshError(RuntimeError):
    def __init__(self, name: str, status: int, text: str):
        super().__init__(f"{name} failed: {text} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if liblsh.so is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m lsh_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32p, fp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
        pp = ctypes.POINTER(Problem)
        L.lsh_status_string.argtypes, L.lsh_status_string.restype = [ctypes.c_int], ctypes.c_char_p
        L.lsh_version.argtypes, L.lsh_version.restype = [], ctypes.c_int
        L.lsh_workspace_bytes.argtypes, L.lsh_workspace_bytes.restype = [pp, ctypes.c_int], sz
        L.lsh_hash.argtypes = [pp, vp, vp, i32p, vp]
        L.lsh_sort.argtypes = [pp, i32p, i32p, i32p, i32p, vp, sz, vp]
        L.lsh_sort_noalloc.argtypes = [pp, i32p, i32p, i32p, i32p, vp]
        L.lsh_attn_fwd.argtypes = [pp, vp, vp, i32p, i32p, i32p, vp, fp, vp, sz, vp]
        L.lsh_combine.argtypes = [pp, vp, vp, vp, fp, vp, fp, vp]
        L.lsh_attn_bwd.argtypes = [pp, vp, vp, vp, vp, fp, i32p, i32p, i32p, vp, vp, vp, sz, vp]
        L.lsh_attn_bwd_saved.argtypes = [pp, vp, vp, vp, vp, fp, vp, vp, vp, sz, vp]
        L.lsh_attn_bwd_rehash.argtypes = [pp, vp, vp, vp, vp, vp, fp, vp, vp, vp, sz, vp]
        L.lsh_kernel_name.argtypes, L.lsh_kernel_name.restype = [ctypes.c_int], ctypes.c_char_p
        L.lsh_profile_kernel.argtypes = [ctypes.c_int, vp, vp]
        fp_ = ctypes.POINTER(FF)
        L.lsh_ff_workspace_bytes.argtypes, L.lsh_ff_workspace_bytes.restype = [fp_, ctypes.c_int], sz
        L.lsh_ff_fwd.argtypes = [fp_, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lsh_ff_bwd.argtypes = [fp_, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        for name in ("lsh_hash", "lsh_sort", "lsh_sort_noalloc", "lsh_attn_fwd", "lsh_combine", "lsh_attn_bwd", "lsh_attn_bwd_saved",
                     "lsh_attn_bwd_rehash", "lsh_profile_kernel", "lsh_ff_fwd", "lsh_ff_bwd"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def check(name: str, status: int) -> None:
    if status != LSH_OK:
        raise LshError(name, status, lib().lsh_status_string(status).decode())
