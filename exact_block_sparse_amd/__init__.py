"""MI355X-native tiled exact attention (dense, causal, block-sparse forward; backward from the
stored log-sum-exp), as a thin Python binding over the C ABI of libfa.so.

Every step of the computation runs in the library's gfx950 kernels; this module only
marshals torch tensors (device memory and the current stream) into the C calls. There is
no CPU or eager fallback: a missing library raises at import, a bad argument raises
``FaError`` with the library's status and detail.

    o, lse = fwd(q, k, v, causal=True)                   # q, k, v: bf16 [B, H, N, d] views
    o, lse = sparse_fwd(q, k, v, offsets, indices)       # Flash-MSA block lists (CSR, int32)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)   # dS kept in the workspace (store_ds=False: recomputed)
    offsets, indices = make_block_lists(n_blocks, window=8, stride=16)
    o, lse = attn_fwd(q, k, v, causal=True)              # k, v may have fewer heads (GQA/MQA)
    o, lse = attn_fwd(q, k, v, cu_seqlens=cu)            # packed [total, H, d] sequences
    o, lse, visits = attn_fwd_visits(q, k, v, kv_offsets=off, kv_indices=idx)   # + which listed tiles ran
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, kv_offsets=off, kv_indices=idx)   # sparse backward
    attn_bwd_noalloc(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv)   # library-owned workspace, no allocation
    o = attention(q, k, v, causal=True); o.backward(do)   # autograd over attn_fwd / attn_bwd
"""
from ._lib import EXPORTS, FA_STATUS, LIB_PATH, AttnDesc, FaError, Strides, lib
from .api import (NOALLOC_WORKSPACE_BYTES, attention, attn_bwd, attn_bwd_ds_workspace_bytes, attn_bwd_noalloc,
                  attn_bwd_workspace_bytes, attn_fwd, attn_fwd_visits, bwd, bwd_ds_workspace_bytes, bwd_workspace_bytes,
                  check_block_lists, fwd, make_block_lists, sparse_fwd, status_str, transpose_block_lists)

__all__ = ["attention", "fwd", "sparse_fwd", "bwd", "bwd_workspace_bytes", "bwd_ds_workspace_bytes", "attn_fwd", "attn_fwd_visits",
           "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_ds_workspace_bytes", "attn_bwd_noalloc",
           "NOALLOC_WORKSPACE_BYTES",
           "make_block_lists", "check_block_lists", "transpose_block_lists", "status_str", "FaError", "Strides",
           "AttnDesc", "lib", "LIB_PATH", "EXPORTS", "FA_STATUS"]
