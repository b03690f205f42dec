"""fa_attn_bwd_noalloc, the backward for callers that cannot allocate (its D workspace is a
device array the library owns, one per GPU), against fa_attn_bwd with a caller-owned
workspace too small for the stored-dS schedule: the same kernels on the same D values, so the
outputs must be equal bit for bit.
Two calls in a row, the second smaller, show that what the first left in the shared array
does not matter; a third covers grouped heads, packed sequences and block lists together.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import exact_block_sparse_amd as fa
    return fa


def _compare(fa, w, **kw):
    x = W.make_inputs(w)
    g = {n: t.to("cuda") for n, t in x.items() if isinstance(t, torch.Tensor)}
    fwd_kw = {k: v for k, v in kw.items() if k not in ("q_offsets", "q_indices")}   # key-side lists: backward only
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=w.causal, scale=w.scale, **fwd_kw)
    want = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=w.causal, scale=w.scale, store_ds=False,
                       **kw)
    outs = [torch.full_like(t, float("nan")) for t in want]
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = fa.attn_bwd_noalloc(g["q"], g["k"], g["v"], o, lse, g["do"], causal=w.causal, scale=w.scale,
                              dq=outs[0], dk=outs[1], dv=outs[2], **kw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before     # nothing allocated through torch either
    for name, a, b in zip(("dQ", "dK", "dV"), got, want):
        assert a.data_ptr() == outs[("dQ", "dK", "dV").index(name)].data_ptr()
        assert torch.equal(a, b), name


def test_noalloc_equals_workspace_backward_twice_second_smaller(fa):
    _compare(fa, W.small(2, 8, 1500, 128, causal=True, seed=60, H_kv=4, direction="bwd"))
    _compare(fa, W.small(1, 2, 300, 64, causal=False, seed=61, direction="bwd"))


def test_noalloc_packed_grouped_block_sparse(fa):
    w = W.small(H=4, d=128, causal=True, seed=62, H_kv=2, seqlens=(300, 700, 129), direction="bwd", sigma=0.5)
    nb = (700 + 127) // 128
    off, idx = fa.make_block_lists(nb, 1, 3, causal=True)
    t_off, t_idx = fa.transpose_block_lists(off, idx, nb)
    to = lambda a: torch.from_numpy(a).to("cuda")
    cu = torch.from_numpy(w.cu_seqlens().astype(np.int32)).to("cuda")
    _compare(fa, w, cu_seqlens=cu, max_seqlen=700, kv_offsets=to(off), kv_indices=to(idx), q_offsets=to(t_off),
             q_indices=to(t_idx))


def test_noalloc_refuses_problems_beyond_its_workspace(fa):
    # 2 x 16 heads x 131073 rows need more than the 32 MiB (4,194,304 head-row pairs): refused on the host
    x = fa.AttnDesc()
    x.B, x.H, x.H_kv, x.N, x.d, x.causal, x.scale = 2, 16, 16, 131072 + 1, 128, 1, 0.1
    assert fa.lib.fa_attn_bwd_workspace_bytes(ctypes.byref(x)) > fa.NOALLOC_WORKSPACE_BYTES
    s = fa.Strides(0, 0, 128)
    p = ctypes.c_void_p(256)
    st = fa.lib.fa_attn_bwd_noalloc(ctypes.byref(x), p, s, p, s, p, s, p, s, p, s, p, p, s, p, s, p, s, None)
    assert st == 6 and "library-owned" in fa.lib.fa_last_error().decode()
