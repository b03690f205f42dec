"""ctypes loader for libfa.so (built in-tree by exact_block_sparse_amd.build).

There is no fallback: if the library is missing or fails to load, importing the package
raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM", 4: "FA_ERR_LAYOUT",
    5: "FA_ERR_LIST", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_HIP", 8: "FA_ERR_ARG", 9: "FA_ERR_CAPACITY",
}
EXPORTS = ("fa_fwd", "fa_sparse_fwd", "fa_bwd_workspace_bytes", "fa_bwd_ds_workspace_bytes", "fa_bwd", "fa_attn_fwd",
           "fa_attn_fwd_visits", "fa_attn_bwd_workspace_bytes", "fa_attn_bwd_ds_workspace_bytes", "fa_attn_bwd",
           "fa_attn_bwd_noalloc", "fa_transpose_block_lists", "fa_make_block_lists",
           "fa_check_block_lists", "fa_status_str", "fa_last_error")


class Strides(ctypes.Structure):
    """fa_strides: element strides (b, h, n) of a logical [B, H, N, d] tensor."""
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class AttnDesc(ctypes.Structure):
    """fa_attn_desc: problem description of fa_attn_fwd / fa_attn_bwd (field order as in fa.h)."""
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("H_kv", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("causal", ctypes.c_int), ("scale", ctypes.c_float),
                ("cu_seqlens", ctypes.c_void_p), ("total", ctypes.c_int64), ("block_size", ctypes.c_int64),
                ("kv_offsets", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p), ("nnz", ctypes.c_int64),
                ("q_offsets", ctypes.c_void_p), ("q_indices", ctypes.c_void_p), ("dtype", ctypes.c_int),
                ("q_descale", ctypes.c_float), ("k_descale", ctypes.c_float), ("v_descale", ctypes.c_float)]


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str, call: str):
        self.status = status
        self.name = FA_STATUS.get(status, f"status {status}")
        super().__init__(f"{call}: {self.name}: {detail}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python exact_block_sparse_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    pi32 = ctypes.POINTER(ctypes.c_int32)
    S = Strides
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, S, S, S, S, i32, f32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_sparse_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, S, S, S, S,
                                  i64, vp, vp, i64, i32, f32, vp]
    lib.fa_sparse_fwd.restype = i32
    lib.fa_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_ds_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.fa_bwd_ds_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                           S, S, S, S, S, S, S, S, i32, f32, vp, ctypes.c_size_t, vp]
    lib.fa_bwd.restype = i32
    D = ctypes.POINTER(AttnDesc)
    sz = ctypes.c_size_t
    lib.fa_attn_fwd.argtypes = [D, vp, S, vp, S, vp, S, vp, S, vp, vp]
    lib.fa_attn_fwd.restype = i32
    lib.fa_attn_fwd_visits.argtypes = [D, vp, S, vp, S, vp, S, vp, S, vp, vp, vp]
    lib.fa_attn_fwd_visits.restype = i32
    lib.fa_attn_bwd_workspace_bytes.argtypes = [D]
    lib.fa_attn_bwd_workspace_bytes.restype = sz
    lib.fa_attn_bwd_ds_workspace_bytes.argtypes = [D]
    lib.fa_attn_bwd_ds_workspace_bytes.restype = sz
    lib.fa_attn_bwd.argtypes = [D, vp, S, vp, S, vp, S, vp, S, vp, S, vp, vp, S, vp, S, vp, S, vp, sz, vp]
    lib.fa_attn_bwd.restype = i32
    lib.fa_attn_bwd_noalloc.argtypes = [D, vp, S, vp, S, vp, S, vp, S, vp, S, vp, vp, S, vp, S, vp, S, vp]
    lib.fa_attn_bwd_noalloc.restype = i32
    lib.fa_transpose_block_lists.argtypes = [i64, pi32, pi32, i64, pi32, pi32]
    lib.fa_transpose_block_lists.restype = i32
    lib.fa_make_block_lists.argtypes = [i64, ctypes.c_int32, ctypes.c_int32, i32, i32, pi32, pi32, i64,
                                        ctypes.POINTER(ctypes.c_int64)]
    lib.fa_make_block_lists.restype = i32
    lib.fa_check_block_lists.argtypes = [pi32, pi32, i64, i64, i32]
    lib.fa_check_block_lists.restype = i32
    lib.fa_status_str.argtypes = [i32]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def check(status: int, call: str) -> None:
    if status != 0:
        raise FaError(status, lib.fa_last_error().decode(errors="replace"), call)
