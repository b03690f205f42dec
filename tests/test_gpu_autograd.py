"""attention(): autograd over attn_fwd / attn_bwd. Its gradients must be the library backward's
outputs bit for bit (the same calls on the same O and LSE), and match the oracle's backward."""
import sys

import pytest
import torch

import oracle
import workloads as W
from parity import TOL_OUT, assert_close

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


def leaves(x, names=("q", "k", "v")):
    return [x[n].to("cuda").detach().requires_grad_(True) for n in names]


@pytest.mark.parametrize("store_ds", [None, False])
def test_autograd_equals_library_backward_grouped_causal(fa, store_ds):
    w = W.small(2, 6, 333, 128, causal=True, seed=71, H_kv=2, direction="bwd", sigma=0.5)
    x = W.make_inputs(w)
    q, k, v = leaves(x)
    do = x["do"].to("cuda")
    o = fa.attention(q, k, v, causal=True, scale=w.scale, store_ds=store_ds)
    o.backward(do)
    o2, lse = fa.attn_fwd(q.detach(), k.detach(), v.detach(), causal=True, scale=w.scale)
    ref = fa.attn_bwd(q.detach(), k.detach(), v.detach(), o2, lse, do, causal=True, scale=w.scale,
                      store_ds=store_ds)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for name, g, r in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), ref):
        assert torch.equal(g, r), name
    dQ, dK, dV = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale)
    assert_close("dQ", q.grad, dQ, TOL_OUT)
    assert_close("dK", k.grad, dK, TOL_OUT)
    assert_close("dV", v.grad, dV, TOL_OUT)


def test_autograd_bnhd_views_packed_and_block_sparse(fa):
    # (B, N, H, d) memory as [B, H, N, d] views: the gradients land in the base tensors
    w = W.small(1, 2, 400, 128, causal=False, seed=72, layout="bnhd", direction="bwd")
    x = W.make_inputs(w)
    bases = [x[n].to("cuda").transpose(1, 2).contiguous().requires_grad_(True) for n in ("q", "k", "v")]
    q, k, v = (t.transpose(1, 2) for t in bases)
    o = fa.attention(q, k, v, causal=False, scale=w.scale)
    o.backward(x["do"].to("cuda"))
    torch.cuda.synchronize()
    dQ, dK, dV = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=False, scale=w.scale)
    for name, base, ref in zip(("dQ", "dK", "dV"), bases, (dQ, dK, dV)):
        assert_close(name, base.grad.transpose(1, 2), ref, TOL_OUT)

    # packed sequences with block lists, grouped heads
    lens = (300, 129, 520)
    w = W.small(H=4, d=128, causal=True, seed=73, H_kv=2, seqlens=lens, direction="bwd", sigma=0.5)
    x = W.make_inputs(w)
    q, k, v = leaves(x)
    cu = w.cu_seqlens()
    nb = (max(lens) + 127) // 128
    off, idx = oracle.block_lists(nb, 1, 3, True, "strided")
    o = fa.attention(q, k, v, causal=True, scale=w.scale, cu_seqlens=cu, kv_offsets=off, kv_indices=idx)
    o.backward(x["do"].to("cuda"))
    torch.cuda.synchronize()
    sp = dict(block=128, offsets=off, indices=idx)
    dQ, dK, dV, O, L = oracle.attention_backward_varlen(x["q"], x["k"], x["v"], x["do"], cu, causal=True,
                                                        scale=w.scale, sparse=sp, return_forward=True)
    assert_close("O", o.detach(), O, TOL_OUT)
    assert_close("dQ", q.grad, dQ, TOL_OUT)
    assert_close("dK", k.grad, dK, TOL_OUT)
    assert_close("dV", v.grad, dV, TOL_OUT)
