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

from ._lib import AttnDesc, FaError, Strides, check, lib

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


def _check_tensor_arg(name: str, t, shape, device, dtype=torch.bfloat16) -> None:
    """A tensor the caller passes for the library to read or write (out, o, do): its dtype,
    device and shape must be the ones the call implies, and its last dimension contiguous;
    its other strides are passed to the library as they are. A wrong shape would otherwise
    make the kernels read or write past the end of its storage."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dim() and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous (stride 1)")


def _check_stats_arg(name: str, t, shape, device) -> None:
    """Per-row statistics (lse): fp32, contiguous, of the given shape, on the device."""
    _check_tensor_arg(name, t, shape, device, torch.float32)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(ws, need: int, device) -> tuple[torch.Tensor, int]:
    """The backward workspace: a new one of `need` bytes, or the caller's (a contiguous tensor
    on the device, its size counted in bytes)."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device), max(need, 1)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return ws, ws.numel() * ws.element_size()


def _bwd_workspace(ws, need: int, need_ds: int, store_ds, device) -> tuple[torch.Tensor, int]:
    """Workspace of a backward call. A caller's tensor is used as given (its size selects the
    schedule in the library). Otherwise store_ds=True asks for the stored-dS schedule (an
    error where it does not exist), False for recomputation, and None takes the stored-dS
    schedule when it exists and its workspace is at most a quarter of the device's memory
    and half of what is free."""
    if ws is not None:
        return _workspace(ws, need, device)
    if store_ds and not need_ds:
        raise ValueError("the stored-dS backward needs head dimension 128, bf16 and a non-empty problem")
    if store_ds is None:
        free, total = torch.cuda.mem_get_info(device)
        store_ds = 0 < need_ds <= min(total // 4, free // 2)
    return _workspace(None, need_ds if store_ds else need, device)


def _empty_like_layout(t: torch.Tensor, dtype=None) -> torch.Tensor:
    """An uninitialised tensor with t's shape and, if t is a permuted dense tensor, its layout."""
    dtype = t.dtype if dtype is None else dtype
    order = sorted(range(t.dim()), key=lambda i: (-t.stride(i), i))
    p = t.permute(*order)
    if p.is_contiguous():
        inv = [0] * t.dim()
        for j, i in enumerate(order):
            inv[i] = j
        return torch.empty(p.shape, dtype=dtype, device=t.device).permute(*inv)
    return torch.empty(t.shape, dtype=dtype, device=t.device)


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
    _check_tensor_arg("out", o, q.shape, q.device)
    _check_stats_arg("lse", l, (B, H, N), q.device)
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
    _check_tensor_arg("out", o, q.shape, q.device)
    _check_stats_arg("lse", l, (B, H, N), q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_sparse_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d,
                               _strides(q), _strides(k), _strides(v), _strides(o), int(block_size),
                               _ptr(off), _ptr(idx), int(idx.numel()), int(bool(causal)), _scale(scale, d),
                               _stream(q.device))
    check(st, "fa_sparse_fwd")
    return o, l


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib.fa_bwd_workspace_bytes(B, H, N, d))


def bwd_ds_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool = False) -> int:
    """Workspace with which ``fa_bwd`` stores dS instead of recomputing it (0: no such schedule)."""
    return int(lib.fa_bwd_ds_workspace_bytes(B, H, N, d, int(bool(causal))))


def bwd(q, k, v, o, lse, do, *, causal: bool = False, scale: float | None = None, workspace=None,
        store_ds: bool | None = None):
    """Backward through ``fa_bwd``; returns (dQ, dK, dV) bf16 in the layouts of q, k, v.
    ``store_ds`` picks the schedule when no workspace is given (see ``_bwd_workspace``)."""
    _check_inputs(q, k, v, o, do)
    B, H, N, d = q.shape
    _check_stats_arg("lse", lse, (B, H, N), q.device)
    dq, dk, dv = _empty_like_layout(q), _empty_like_layout(k), _empty_like_layout(v)
    ws, ws_bytes = _bwd_workspace(workspace, bwd_workspace_bytes(B, H, N, d),
                                  bwd_ds_workspace_bytes(B, H, N, d, causal), store_ds, q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, H, N, d, _strides(q), _strides(k), _strides(v), _strides(o), _strides(do),
                        _strides(dq), _strides(dk), _strides(dv), int(bool(causal)), _scale(scale, d),
                        _ptr(ws), ws_bytes, _stream(q.device))
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


# ----------------------------------------------------------------------------- general calls
def transpose_block_lists(offsets, indices, n_blocks: int):
    """Key-side form of host CSR block lists via ``fa_transpose_block_lists`` (host int32)."""
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    if off.size != n_blocks + 1:
        raise FaError(5, f"offsets has {off.size} entries, {n_blocks + 1} expected", "fa_transpose_block_lists")
    t_off = np.zeros(n_blocks + 1, dtype=np.int32)
    t_idx = np.zeros(max(idx.size, 1), dtype=np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    st = lib.fa_transpose_block_lists(n_blocks, off.ctypes.data_as(p32), idx.ctypes.data_as(p32) if idx.size else None,
                                      idx.size, t_off.ctypes.data_as(p32), t_idx.ctypes.data_as(p32))
    check(st, "fa_transpose_block_lists")
    return t_off, t_idx[: idx.size]


def _packed_strides(t: torch.Tensor) -> Strides:
    if t.dim() != 3:
        raise ValueError(f"expected a packed 3-d [total, heads, d] tensor, got shape {tuple(t.shape)}")
    if t.stride(2) != 1 and t.shape[2] > 1:
        raise ValueError("the head dimension must be contiguous (stride 1)")
    return Strides(0, t.stride(1), t.stride(0))


FP8 = getattr(torch, "float8_e4m3fn", None)


def _check_group(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, packed: bool, allow_fp8: bool = False) -> None:
    for t in (q, k, v):
        ok = t.dtype == torch.bfloat16 or (allow_fp8 and FP8 is not None and t.dtype == FP8)
        if not ok or t.dtype != q.dtype:
            raise TypeError(f"expected bfloat16{' or float8_e4m3fn' if allow_fp8 else ''} tensors of one dtype, "
                            f"got {q.dtype}, {k.dtype}, {v.dtype}")
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError("tensors must be on one GPU device")
    hd = 1
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"k and v shapes differ: {tuple(k.shape)} vs {tuple(v.shape)}")
    same = [i for i in range(q.dim()) if i != hd]
    if any(q.shape[i] != k.shape[i] for i in same):
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} differ outside the head axis")


def _desc(B, H, H_kv, N, d, causal, scale, cu=None, total=0, lists=None, fp8=False,
          descales=(1.0, 1.0, 1.0)) -> AttnDesc:
    x = AttnDesc()
    x.B, x.H, x.H_kv, x.N, x.d = B, H, H_kv, N, d
    x.causal, x.scale = int(bool(causal)), float(scale)
    x.dtype = 1 if fp8 else 0
    x.q_descale, x.k_descale, x.v_descale = (float(s) for s in descales)
    x.cu_seqlens = cu.data_ptr() if cu is not None else None
    x.total = int(total)
    if lists is not None:
        x.block_size = lists["block"]
        x.kv_offsets, x.kv_indices = lists["off"].data_ptr(), lists["idx"].data_ptr()
        x.nnz = lists["nnz"]
        if "t_off" in lists:
            x.q_offsets, x.q_indices = lists["t_off"].data_ptr(), lists["t_idx"].data_ptr()
    return x


def _seq_args(q: torch.Tensor, cu_seqlens, max_seqlen):
    """(packed, B, N, total, cu device tensor or None)."""
    if cu_seqlens is None:
        B, _, N, _ = q.shape
        return False, B, N, 0, None
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-d int32 tensor")
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with device cu_seqlens")
        cu = cu_seqlens.contiguous()
    else:
        host = np.asarray(cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens, dtype=np.int64)
        if host.ndim != 1 or host.size < 1 or host[0] != 0 or np.any(np.diff(host) < 0) or host[-1] > q.shape[0]:
            raise ValueError("cu_seqlens must start at 0, not decrease and end within the packed rows")
        if max_seqlen is None:
            max_seqlen = int(np.max(np.diff(host))) if host.size > 1 else 0
        cu = torch.from_numpy(host.astype(np.int32)).to(q.device)
    return True, int(cu.numel()) - 1, int(max_seqlen), int(q.shape[0]), cu


def _device_lists(kv_offsets, kv_indices, q_offsets, q_indices, n_blocks, causal, block_size, device, backward):
    """Device copies of the query-side (and, for the backward, key-side) block lists."""
    on_device = isinstance(kv_offsets, torch.Tensor) and kv_offsets.device.type == "cuda"
    nnz = int(kv_indices.numel()) if on_device else int(np.asarray(
        kv_indices.cpu() if isinstance(kv_indices, torch.Tensor) else kv_indices).size)
    off, idx = _lists_to_device(kv_offsets, kv_indices, n_blocks, causal, device)
    lists = dict(block=int(block_size), off=off, idx=idx, nnz=nnz)
    if backward:
        if q_offsets is None:
            if on_device:
                raise ValueError("pass q_offsets/q_indices with device lists (see transpose_block_lists)")
            host_off = np.asarray(kv_offsets.cpu() if isinstance(kv_offsets, torch.Tensor) else kv_offsets)
            host_idx = np.asarray(kv_indices.cpu() if isinstance(kv_indices, torch.Tensor) else kv_indices)
            q_offsets, q_indices = transpose_block_lists(host_off, host_idx, n_blocks)
        t_off, t_idx = _lists_to_device(q_offsets, q_indices, n_blocks, False, device)
        lists["t_off"], lists["t_idx"] = t_off, t_idx
    return lists


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             scale: float | None = None, cu_seqlens=None, max_seqlen: int | None = None,
             kv_offsets=None, kv_indices=None, block_size: int = BLOCK,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
             q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0):
    """General forward through ``fa_attn_fwd``: grouped K/V heads, packed sequences, block lists,
    bf16 or fp8 (``torch.float8_e4m3fn``, real value = code x descale) inputs.

    Fixed length: q [B, H, N, d], k and v [B, H_kv, N, d]; returns O (bf16) in q's layout and
    LSE [B, H, N]. Packed (``cu_seqlens`` given, int32 [B+1], host or device): q [total, H, d],
    k and v [total, H_kv, d]; returns O like q and LSE [H, total]. ``max_seqlen`` bounds every
    sequence's length (computed from host offsets when omitted).
    """
    return _attn_fwd(q, k, v, causal, scale, cu_seqlens, max_seqlen, kv_offsets, kv_indices, block_size, out, lse,
                     (q_descale, k_descale, v_descale), False)


def attn_fwd_visits(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, kv_offsets, kv_indices,
                    causal: bool = False, scale: float | None = None, cu_seqlens=None,
                    max_seqlen: int | None = None, block_size: int = BLOCK,
                    out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                    q_descale: float = 1.0, k_descale: float = 1.0, v_descale: float = 1.0):
    """Block-sparse ``attn_fwd`` through ``fa_attn_fwd_visits``: returns (O, LSE, visits), where
    visits is a uint8 tensor [B * H, nnz, 2] holding 1 at (b * H + h, e, half) for every half of
    list entry e that sequence b, head h took into its softmax, and 0 for skipped entries."""
    return _attn_fwd(q, k, v, causal, scale, cu_seqlens, max_seqlen, kv_offsets, kv_indices, block_size, out, lse,
                     (q_descale, k_descale, v_descale), True)


def _attn_fwd(q, k, v, causal, scale, cu_seqlens, max_seqlen, kv_offsets, kv_indices, block_size, out, lse,
              descales, want_visits):
    packed = cu_seqlens is not None
    _check_group(q, k, v, packed, allow_fp8=True)
    fp8 = q.dtype != torch.bfloat16
    d = q.shape[-1]
    H, H_kv = (q.shape[1], k.shape[1])
    pk, B, N, total, cu = _seq_args(q, cu_seqlens, max_seqlen)
    lists = None
    if kv_offsets is not None:
        nb = (N + block_size - 1) // block_size
        lists = _device_lists(kv_offsets, kv_indices, None, None, nb, causal, block_size, q.device, False)
    if out is None:
        o = _empty_like_layout(q, torch.bfloat16) if not pk else torch.empty(q.shape, dtype=torch.bfloat16,
                                                                              device=q.device)
    else:
        o = out
    lshape = (H, total) if pk else (B, H, N)
    l = torch.empty(lshape, dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor_arg("out", o, q.shape, q.device)
    _check_stats_arg("lse", l, lshape, q.device)
    S = _packed_strides if pk else _strides
    x = _desc(B, H, H_kv, N, d, causal, _scale(scale, d), cu, total, lists, fp8, descales)
    if want_visits:
        if lists is None:
            raise ValueError("attn_fwd_visits needs block lists (kv_offsets, kv_indices)")
        visits = torch.zeros((B * H, int(x.nnz), 2), dtype=torch.uint8, device=q.device)
        with torch.cuda.device(q.device):
            st = lib.fa_attn_fwd_visits(ctypes.byref(x), _ptr(q), S(q), _ptr(k), S(k), _ptr(v), S(v), _ptr(o), S(o),
                                        _ptr(l), _ptr(visits), _stream(q.device))
        check(st, "fa_attn_fwd_visits")
        return o, l, visits
    with torch.cuda.device(q.device):
        st = lib.fa_attn_fwd(ctypes.byref(x), _ptr(q), S(q), _ptr(k), S(k), _ptr(v), S(v), _ptr(o), S(o), _ptr(l),
                             _stream(q.device))
    check(st, "fa_attn_fwd")
    return o, l


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int, total: int | None = None) -> int:
    x = _desc(B, H, H, N, d, False, 1.0)
    if total is not None:
        x.cu_seqlens = 1   # any non-NULL value selects the packed layout; it is not read
        x.total = int(total)
    return int(lib.fa_attn_bwd_workspace_bytes(ctypes.byref(x)))


def attn_bwd_ds_workspace_bytes(B: int, H: int, N: int, d: int, *, causal: bool = False, total: int | None = None,
                                nnz: int | None = None) -> int:
    """Workspace with which ``fa_attn_bwd`` stores dS (``nnz``: block-sparse with that many
    list entries; ``total``: packed rows). 0 where that schedule does not exist."""
    x = _desc(B, H, H, N, d, causal, 1.0)
    if total is not None:
        x.cu_seqlens = 1   # any non-NULL value selects the packed layout; it is not read
        x.total = int(total)
    if nnz is not None:
        x.kv_offsets = 1   # likewise selects block-sparse mode
        x.block_size, x.nnz = BLOCK, int(nnz)
    return int(lib.fa_attn_bwd_ds_workspace_bytes(ctypes.byref(x)))


def attn_bwd(q, k, v, o, lse, do, *, causal: bool = False, scale: float | None = None, cu_seqlens=None,
             max_seqlen: int | None = None, kv_offsets=None, kv_indices=None, q_offsets=None, q_indices=None,
             block_size: int = BLOCK, workspace=None, store_ds: bool | None = None):
    """General backward through ``fa_attn_bwd``; returns (dQ like q, dK like k, dV like v).

    Arguments as in ``attn_fwd``; ``o`` and ``lse`` are its outputs. With host block lists
    the key-side lists are derived with ``transpose_block_lists`` when not given.
    ``store_ds`` picks the schedule when no workspace is given: True stores dS in the
    workspace (head dimension 128), False recomputes it in the dQ pass, None (default) stores
    it when that workspace is at most a quarter of the device's memory and half of what is free.
    """
    packed = cu_seqlens is not None
    _check_group(q, k, v, packed)
    d = q.shape[-1]
    H, H_kv = q.shape[1], k.shape[1]
    pk, B, N, total, cu = _seq_args(q, cu_seqlens, max_seqlen)
    lists = None
    if kv_offsets is not None:
        nb = (N + block_size - 1) // block_size
        lists = _device_lists(kv_offsets, kv_indices, q_offsets, q_indices, nb, causal, block_size, q.device, True)
    _check_tensor_arg("o", o, q.shape, q.device)
    _check_tensor_arg("do", do, q.shape, q.device)
    _check_stats_arg("lse", lse, (H, total) if pk else (B, H, N), q.device)
    if pk:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = _empty_like_layout(q), _empty_like_layout(k), _empty_like_layout(v)
    S = _packed_strides if pk else _strides
    x = _desc(B, H, H_kv, N, d, causal, _scale(scale, d), cu, total, lists)
    ws, ws_bytes = _bwd_workspace(workspace, int(lib.fa_attn_bwd_workspace_bytes(ctypes.byref(x))),
                                  int(lib.fa_attn_bwd_ds_workspace_bytes(ctypes.byref(x))), store_ds, q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_attn_bwd(ctypes.byref(x), _ptr(q), S(q), _ptr(k), S(k), _ptr(v), S(v), _ptr(o), S(o), _ptr(do),
                             S(do), _ptr(lse), _ptr(dq), S(dq), _ptr(dk), S(dk), _ptr(dv), S(dv), _ptr(ws),
                             ws_bytes, _stream(q.device))
    check(st, "fa_attn_bwd")
    return dq, dk, dv


NOALLOC_WORKSPACE_BYTES = 32 << 20   # FA_NOALLOC_WORKSPACE_BYTES of fa.h


def attn_bwd_noalloc(q, k, v, o, lse, do, *, causal: bool = False, scale: float | None = None, cu_seqlens=None,
                     max_seqlen: int | None = None, kv_offsets=None, kv_indices=None, q_offsets=None,
                     q_indices=None, block_size: int = BLOCK, dq=None, dk=None, dv=None):
    """Backward through ``fa_attn_bwd_noalloc``: the function of ``attn_bwd`` with the workspace
    the library owns (one per GPU), for callers that cannot allocate. Pass ``dq``, ``dk``, ``dv``
    (shaped like q, k, v), device ``cu_seqlens`` and device block lists to make the call
    allocate nothing on the Python side either; missing outputs are allocated here.
    Calls that overlap on one GPU share the library's workspace and race.
    """
    packed = cu_seqlens is not None
    _check_group(q, k, v, packed)
    d = q.shape[-1]
    H, H_kv = q.shape[1], k.shape[1]
    pk, B, N, total, cu = _seq_args(q, cu_seqlens, max_seqlen)
    lists = None
    if kv_offsets is not None:
        nb = (N + block_size - 1) // block_size
        lists = _device_lists(kv_offsets, kv_indices, q_offsets, q_indices, nb, causal, block_size, q.device, True)
    _check_tensor_arg("o", o, q.shape, q.device)
    _check_tensor_arg("do", do, q.shape, q.device)
    _check_stats_arg("lse", lse, (H, total) if pk else (B, H, N), q.device)
    new = (lambda t: torch.empty_like(t)) if pk else _empty_like_layout
    dq = new(q) if dq is None else dq
    dk = new(k) if dk is None else dk
    dv = new(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor_arg(name, t, like.shape, q.device)
    S = _packed_strides if pk else _strides
    x = _desc(B, H, H_kv, N, d, causal, _scale(scale, d), cu, total, lists)
    with torch.cuda.device(q.device):
        st = lib.fa_attn_bwd_noalloc(ctypes.byref(x), _ptr(q), S(q), _ptr(k), S(k), _ptr(v), S(v), _ptr(o), S(o),
                                     _ptr(do), S(do), _ptr(lse), _ptr(dq), S(dq), _ptr(dk), S(dk), _ptr(dv), S(dv),
                                     _stream(q.device))
    check(st, "fa_attn_bwd_noalloc")
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """Autograd over attn_fwd / attn_bwd: the forward keeps O and the LSE (not the score
    matrix), the backward hands them to the library's backward."""

    @staticmethod
    def forward(ctx, q, k, v, kw, bwd_kw):
        o, lse = attn_fwd(q, k, v, **kw)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.kw, ctx.bwd_kw = kw, bwd_kw
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        do = do if do.stride(-1) == 1 else do.contiguous()
        dq, dk, dv = attn_bwd(q, k, v, o, lse, do, **ctx.kw, **ctx.bwd_kw)
        return dq, dk, dv, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
              scale: float | None = None, cu_seqlens=None, max_seqlen: int | None = None, kv_offsets=None,
              kv_indices=None, q_offsets=None, q_indices=None, block_size: int = BLOCK,
              store_ds: bool | None = None) -> torch.Tensor:
    """O = softmax(Q K^T scale + mask) V with gradients for q, k and v (bf16), for training: the
    arguments of ``attn_fwd`` (dense, causal, grouped, packed, block-sparse); the backward runs
    ``attn_bwd`` with ``store_ds`` and, block-sparse, the key-side lists (derived when not
    given)."""
    kw = dict(causal=causal, scale=scale, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, kv_offsets=kv_offsets,
              kv_indices=kv_indices, block_size=block_size)
    bwd_kw = dict(q_offsets=q_offsets, q_indices=q_indices, store_ds=store_ds)
    return _Attention.apply(q, k, v, kw, bwd_kw)
