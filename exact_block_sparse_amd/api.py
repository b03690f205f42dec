"""torch-facing wrappers: validate Python-side types, allocate outputs with torch, call the C ABI.

Tensors are logical [B, H, N, d] bf16 CUDA (HIP) tensors whose last dimension is
contiguous; (B, N, H, d) memory is passed as a permuted view. Outputs are allocated in
the same memory layout as the corresponding input. Calls are asynchronous on the current
torch stream of the tensors' device.
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from ._lib import FaError, Strides, check, lib

BLOCK = 128


def status_str(status: int) -> str:
    return lib.fa_status_str(int(status)).decode()


def _strides(t: torch.Tensor) -> Strides:
    if t.dim() != 4:
        raise ValueError(f"expected a 4-d [B, H, N, d] tensor, got shape {tuple(t.shape)}")
    if t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _check_inputs(*ts: torch.Tensor) -> None:
    dev = ts[0].device
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"expected bfloat16 tensors, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a GPU device")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if tuple(t.shape) != tuple(ts[0].shape):
            raise ValueError(f"shape mismatch {tuple(t.shape)} vs {tuple(ts[0].shape)}")


def _empty_like_layout(t: torch.Tensor) -> torch.Tensor:
    """An uninitialised tensor with t's shape and, if t is a permuted dense tensor, its layout."""
    order = sorted(range(t.dim()), key=lambda i: (-t.stride(i), i))
    p = t.permute(*order)
    if p.is_contiguous():
        inv = [0] * t.dim()
        for j, i in enumerate(order):
            inv[i] = j
        return torch.empty(p.shape, dtype=t.dtype, device=t.device).permute(*inv)
    return torch.empty(t.shape, dtype=t.dtype, device=t.device)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _scale(scale, d: int) -> float:
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False, scale: float | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Attention forward through ``fa_fwd``; returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N])."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    o = _empty_like_layout(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    with torch.cuda.device(q.device):
        st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d,
                        _strides(q), _strides(k), _strides(v), _strides(o), int(bool(causal)),
                        _scale(scale, d), _stream(q.device))
    check(st, "fa_fwd")
    return o, l


def _lists_to_device(offsets, indices, n_blocks: int, causal: bool, device):
    if isinstance(offsets, torch.Tensor) and offsets.device.type == "cuda":
        if offsets.dtype != torch.int32 or indices.dtype != torch.int32:
            raise TypeError("block lists must be int32")
        return offsets.contiguous(), indices.contiguous()
    off = np.ascontiguousarray(np.asarray(offsets.cpu() if isinstance(offsets, torch.Tensor) else offsets,
                                          dtype=np.int32))
    idx = np.ascontiguousarray(np.asarray(indices.cpu() if isinstance(indices, torch.Tensor) else indices,
                                          dtype=np.int32))
    check_block_lists(off, idx, n_blocks, causal)
    to = torch.from_numpy(off).to(device)
    ti = torch.from_numpy(idx if idx.size else np.zeros(1, np.int32)).to(device)
    return to, ti[: idx.size] if idx.size else ti


def sparse_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_offsets, kv_indices, *,
               causal: bool = True, scale: float | None = None, block_size: int = BLOCK,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Block-sparse forward through ``fa_sparse_fwd``.

    ``kv_offsets``/``kv_indices``: CSR block lists, int32, either host arrays (checked with
    fa_check_block_lists, then copied) or device tensors (passed as they are).
    """
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    nb = (N + block_size - 1) // block_size
    off, idx = _lists_to_device(kv_offsets, kv_indices, nb, causal, q.device)
    o = _empty_like_layout(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    with torch.cuda.device(q.device):
        st = lib.fa_sparse_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d,
                               _strides(q), _strides(k), _strides(v), _strides(o), int(block_size),
                               _ptr(off), _ptr(idx), int(idx.numel()), int(bool(causal)), _scale(scale, d),
                               _stream(q.device))
    check(st, "fa_sparse_fwd")
    return o, l


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib.fa_bwd_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, lse, do, *, causal: bool = False, scale: float | None = None, workspace=None):
    """Backward through ``fa_bwd``; returns (dQ, dK, dV) bf16 in the layouts of q, k, v."""
    _check_inputs(q, k, v, o, do)
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    B, H, N, d = q.shape
    dq, dk, dv = _empty_like_layout(q), _empty_like_layout(k), _empty_like_layout(v)
    need = bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device) if workspace is None else workspace
    with torch.cuda.device(q.device):
        st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, H, N, d, _strides(q), _strides(k), _strides(v), _strides(o), _strides(do),
                        _strides(dq), _strides(dk), _strides(dv), int(bool(causal)), _scale(scale, d),
                        _ptr(ws), ws.numel(), _stream(q.device))
    check(st, "fa_bwd")
    return dq, dk, dv


def make_block_lists(n_blocks: int, window: int = 8, stride: int = 16, causal: bool = True,
                     rule: str = "strided"):
    """The Flash-MSA window + strided block pattern from ``fa_make_block_lists`` (host int32 CSR)."""
    r = {"strided": 0, "fixed": 1}[rule]
    off = np.zeros(n_blocks + 1, dtype=np.int32)
    nnz = ctypes.c_int64(0)
    p32 = ctypes.POINTER(ctypes.c_int32)
    st = lib.fa_make_block_lists(n_blocks, window, stride, int(bool(causal)), r,
                                 off.ctypes.data_as(p32), None, 0, ctypes.byref(nnz))
    if st not in (0, 9):
        check(st, "fa_make_block_lists")
    idx = np.zeros(max(nnz.value, 1), dtype=np.int32)
    st = lib.fa_make_block_lists(n_blocks, window, stride, int(bool(causal)), r,
                                 off.ctypes.data_as(p32), idx.ctypes.data_as(p32), idx.size, ctypes.byref(nnz))
    check(st, "fa_make_block_lists")
    return off, idx[: nnz.value]


def check_block_lists(offsets, indices, n_blocks: int, causal: bool = True) -> None:
    """Raise FaError(FA_ERR_LIST) unless the host CSR lists are well formed."""
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    if off.size != n_blocks + 1:
        raise FaError(5, f"offsets has {off.size} entries, {n_blocks + 1} expected", "fa_check_block_lists")
    p32 = ctypes.POINTER(ctypes.c_int32)
    st = lib.fa_check_block_lists(off.ctypes.data_as(p32), idx.ctypes.data_as(p32) if idx.size else None,
                                  n_blocks, idx.size, int(bool(causal)))
    check(st, "fa_check_block_lists")
