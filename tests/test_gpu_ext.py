"""GPU parity of the general entry points (fa_attn_fwd / fa_attn_bwd) against the fp64 oracle:
grouped K/V heads (GQA, MQA), packed variable-length sequences, and the block-sparse
backward with key-side lists; each alone and combined.

Small cases are compared element by element; the extension workloads are compared at
full size on sampled query rows (O, LSE, dQ) and sampled keys (dK, dV, summed over the
query heads of a group). Tolerances as everywhere: max-abs 2e-2 on O, dQ, dK, dV, 1e-3
on LSE.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import TOL_LSE, TOL_OUT, assert_close, assert_finite, f64, sample_rows

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


def dev(x):
    return {n: t.to("cuda") for n, t in x.items()}


def lists_for(n_blocks, window, stride, causal, rule="strided"):
    off, idx = oracle.block_lists(n_blocks, window, stride, causal, rule)
    return off, idx, dict(block=128, offsets=off, indices=idx)


# ----------------------------------------------------------------------------- grouped heads
GQA_FWD = [
    # B, H, H_kv, N, d, causal, layout
    (2, 8, 2, 300, 128, True, "bhnd"),
    (1, 6, 3, 200, 64, False, "bnhd"),
    (1, 4, 1, 129, 128, True, "bhnd"),      # multi-query
    (1, 4, 4, 100, 128, True, "bhnd"),      # H_kv = H through the general call
    (1, 8, 2, 513, 64, True, "bhnd"),
]


@pytest.mark.parametrize("case", GQA_FWD, ids=lambda c: "b{}h{}kv{}n{}d{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", c[6]))
def test_gqa_forward_small(fa, case):
    B, H, Hkv, N, d, causal, layout = case
    w = W.small(B, H, N, d, causal=causal, layout=layout, seed=11, H_kv=Hkv)
    x = W.make_inputs(w)
    g = dev(x)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(x["q"], x["k"], x["v"], causal=causal, scale=w.scale)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)


def test_gqa_with_shared_heads_equals_replicated_mha(fa):
    # grouping only changes which K/V head is read: the same numbers as plain multi-head
    # attention on K/V replicated over the group (same kernels, same order of work)
    w = W.small(1, 8, 700, 128, causal=True, seed=12, H_kv=2)
    g = dev(W.make_inputs(w))
    o1, l1 = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale)
    kr = g["k"].repeat_interleave(4, dim=1).contiguous()
    vr = g["v"].repeat_interleave(4, dim=1).contiguous()
    o2, l2 = fa.fwd(g["q"], kr, vr, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# dK and dV of a K/V head sum over its query heads, so they grow with the group; the
# multi-query case is drawn at sigma 0.5 to keep |dV| below 8, where bf16 output rounding
# (half an ulp is 1/32 from 8 up) would exceed the 2e-2 bound on its own.
GQA_BWD = [
    (1, 4, 2, 200, 128, True, 1.0),
    (2, 6, 3, 130, 64, False, 1.0),
    (1, 4, 1, 257, 128, True, 0.5),
    # three query heads per K/V head, causal, N = 130: the last key block sees one query
    # step per head (an odd number of masked steps), the first an odd number of unmasked ones
    (1, 6, 2, 130, 128, True, 0.5),
    (2, 6, 3, 300, 128, False, 1.0),
]


SCHEDULES = pytest.mark.parametrize("store_ds", [None, False], ids=["stored_ds", "recomputed"])


@SCHEDULES
@pytest.mark.parametrize("case", GQA_BWD, ids=lambda c: "b{}h{}kv{}n{}d{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else ""))
def test_gqa_backward_small(fa, case, store_ds):
    B, H, Hkv, N, d, causal, sigma = case
    w = W.small(B, H, N, d, causal=causal, seed=13, H_kv=Hkv, direction="bwd", sigma=sigma)
    x = W.make_inputs(w)
    g = dev(x)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=w.scale)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=causal, scale=w.scale,
                             store_ds=store_ds)
    torch.cuda.synchronize()
    assert tuple(dk.shape) == tuple(x["k"].shape)
    dQ, dK, dV = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=causal, scale=w.scale)
    assert_close("dQ", dq, dQ, TOL_OUT)
    assert_close("dK", dk, dK, TOL_OUT)
    assert_close("dV", dv, dV, TOL_OUT)


# ----------------------------------------------------------------------------- packed sequences
VARLEN = [
    # lengths, H, H_kv, d, causal
    ((37, 0, 263, 1, 399), 4, 2, 128, True),
    ((37, 0, 263, 1, 399), 2, 2, 128, False),
    ((128, 128, 128), 2, 1, 64, True),
    ((700,), 2, 2, 64, False),
    ((5, 300, 64, 129), 3, 3, 128, True),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "{}_h{}kv{}d{}{}".format(
    "-".join(map(str, c[0])), c[1], c[2], c[3], "c" if c[4] else ""))
def test_varlen_forward_small(fa, case):
    lens, H, Hkv, d, causal = case
    w = W.small(H=H, d=d, causal=causal, seed=14, H_kv=Hkv, seqlens=lens)
    x = W.make_inputs(w)
    g = dev(x)
    cu = w.cu_seqlens()
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=w.scale, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert tuple(lse.shape) == (H, w.total)
    O, L = oracle.attention_forward_varlen(x["q"], x["k"], x["v"], cu, causal=causal, scale=w.scale)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)


def test_varlen_single_sequence_equals_fixed_length(fa):
    # one packed sequence is the fixed-length problem with B = 1 in (B, N, H, d) memory
    w = W.small(H=4, d=128, causal=True, seed=15, seqlens=(1000,))
    g = dev(W.make_inputs(w))
    o1, l1 = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale, cu_seqlens=w.cu_seqlens())
    view = lambda t: t.unsqueeze(0).permute(0, 2, 1, 3)
    o2, l2 = fa.fwd(view(g["q"]), view(g["k"]), view(g["v"]), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[0].permute(1, 0, 2)) and torch.equal(l1, l2[0])


@pytest.mark.parametrize("case", [((37, 0, 200, 1), 4, 2, 128, True), ((64, 100), 2, 2, 64, False),
                                  ((129, 3, 256), 2, 1, 128, True), ((300, 1, 129), 4, 2, 128, False)],
                         ids=lambda c: "{}_h{}kv{}d{}{}".format("-".join(map(str, c[0])), c[1], c[2], c[3],
                                                                "c" if c[4] else ""))
@SCHEDULES
def test_varlen_backward_small(fa, case, store_ds):
    # sigma 0.5: a one-row sequence makes dV the plain sum of its query heads' dO, which at
    # sigma 1 reaches the 4..8 range where bf16 output rounding alone uses 0.016 of the 0.02
    lens, H, Hkv, d, causal = case
    w = W.small(H=H, d=d, causal=causal, seed=16, H_kv=Hkv, seqlens=lens, direction="bwd", sigma=0.5)
    x = W.make_inputs(w)
    g = dev(x)
    cu = w.cu_seqlens()
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=w.scale, cu_seqlens=cu)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=causal, scale=w.scale,
                             cu_seqlens=cu, store_ds=store_ds)
    torch.cuda.synchronize()
    dQ, dK, dV = oracle.attention_backward_varlen(x["q"], x["k"], x["v"], x["do"], cu, causal=causal,
                                                  scale=w.scale)
    assert_close("dQ", dq, dQ, TOL_OUT)
    assert_close("dK", dk, dK, TOL_OUT)
    assert_close("dV", dv, dV, TOL_OUT)


def test_varlen_device_offsets_and_trailing_rows(fa):
    # offsets as a device tensor with max_seqlen given; packed rows after the last sequence
    # are not part of any sequence and are left as they were
    w = W.small(H=2, d=64, causal=True, seed=17, seqlens=(100, 50, 30))
    x = W.make_inputs(w)
    pad = 20
    q, k, v = (torch.cat([x[n], torch.zeros(pad, *x[n].shape[1:], dtype=x[n].dtype)]).to("cuda") for n in "qkv")
    cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    o, lse = fa.attn_fwd(q, k, v, causal=True, scale=w.scale, cu_seqlens=cu, max_seqlen=100, out=out)
    torch.cuda.synchronize()
    O, L = oracle.attention_forward_varlen(x["q"], x["k"], x["v"], w.cu_seqlens(), causal=True, scale=w.scale)
    assert_close("O", o[: w.total], O, TOL_OUT)
    assert_close("LSE", lse[:, : w.total], L, TOL_LSE)
    assert bool((o[w.total:] == 7.0).all())


# ----------------------------------------------------------------------------- block-sparse backward
SPARSE_BWD = [
    # N, H, H_kv, d, causal, window, stride, rule
    (1000, 2, 2, 128, True, 1, 3, "strided"),
    (640, 2, 2, 64, False, 1, 2, "fixed"),
    (900, 4, 2, 128, True, 2, 4, "strided"),
    (256, 1, 1, 128, True, 0, 0, "strided"),
    # non-causal at head dimension 128 with grouped heads and a ragged end (the stored-dS
    # schedule's key-tail zeros and above-diagonal tiles)
    (700, 4, 2, 128, False, 1, 3, "strided"),
]


@pytest.mark.parametrize("case", SPARSE_BWD, ids=lambda c: "n{}h{}kv{}d{}{}w{}s{}{}".format(
    c[0], c[1], c[2], c[3], "c" if c[4] else "", c[5], c[6], c[7]))
@SCHEDULES
def test_sparse_backward_small(fa, case, store_ds):
    N, H, Hkv, d, causal, window, stride, rule = case
    w = W.small(1, H, N, d, causal=causal, seed=18, H_kv=Hkv, direction="bwd")
    x = W.make_inputs(w)
    g = dev(x)
    nb = (N + 127) // 128
    off, idx, sp = lists_for(nb, window, stride, causal, rule)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=w.scale, kv_offsets=off, kv_indices=idx)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=causal, scale=w.scale,
                             kv_offsets=off, kv_indices=idx, store_ds=store_ds)
    torch.cuda.synchronize()
    dQ, dK, dV, O, L = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=causal, scale=w.scale,
                                                 sparse=sp, return_forward=True)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)
    assert_close("dQ", dq, dQ, TOL_OUT)
    assert_close("dK", dk, dK, TOL_OUT)
    assert_close("dV", dv, dV, TOL_OUT)


def test_sparse_backward_with_full_lists_equals_dense(fa):
    # listing every causal block visits the same tiles in the same order as the dense kernels
    w = W.small(2, 3, 777, 128, causal=True, seed=19, direction="bwd")
    g = dev(W.make_inputs(w))
    nb = (777 + 127) // 128
    off, idx = fa.make_block_lists(nb, nb, 0, causal=True)
    o, lse = fa.fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale)
    d1 = fa.bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=True, scale=w.scale)
    d2 = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=True, scale=w.scale, kv_offsets=off,
                     kv_indices=idx)
    torch.cuda.synchronize()
    for a, b in zip(d1, d2):
        assert torch.equal(a, b)


def test_sparse_backward_hand_lists_with_empty_block(fa):
    # query block 1 lists nothing: its rows have no keys (O = 0, LSE = -inf, dQ = 0) and add
    # nothing to dK, dV; block 2 lists only block 0 (off-diagonal, fully allowed)
    N, d = 384, 128
    w = W.small(1, 2, N, d, causal=True, seed=20, direction="bwd")
    x = W.make_inputs(w)
    g = dev(x)
    off = np.array([0, 1, 1, 2], np.int32)
    idx = np.array([0, 0], np.int32)
    sp = dict(block=128, offsets=off, indices=idx)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale, kv_offsets=off, kv_indices=idx)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=True, scale=w.scale,
                             kv_offsets=off, kv_indices=idx)
    torch.cuda.synchronize()
    assert bool(torch.isneginf(lse[:, :, 128:256]).all())
    assert bool((dq[:, :, 128:256] == 0).all())
    assert_finite("dq", dq)
    dQ, dK, dV = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale, sparse=sp)
    assert_close("dQ", dq, dQ, TOL_OUT)
    assert_close("dK", dk, dK, TOL_OUT)
    assert_close("dV", dv, dV, TOL_OUT)


@SCHEDULES
@pytest.mark.parametrize("d", [64, 128])
def test_sparse_backward_lists_with_entries_above_the_diagonal(fa, d, store_ds):
    # Device lists in which query blocks also name key blocks above them: under causal
    # masking those entries are skipped, so in the key-side lists a skipped query block comes
    # before the diagonal one. The dK/dV pass must still take the diagonal steps with the
    # causal element mask (key block 2 is listed by query blocks 0 (skipped), 2 and 4).
    N = 128 * 5 - 30
    w = W.small(1, 2, N, d, causal=True, seed=23, direction="bwd", sigma=0.5)
    x = W.make_inputs(w)
    g = dev(x)
    lists = [[0, 2], [0, 1, 3], [1, 2], [0, 3, 4], [2, 4]]
    off = np.cumsum([0] + [len(l) for l in lists]).astype(np.int32)
    idx = np.array([k for l in lists for k in l], np.int32)
    t_off, t_idx = fa.transpose_block_lists(off, idx, 5)
    assert list(t_idx[t_off[2]:t_off[3]]) == [0, 2, 4]
    to = lambda a: torch.from_numpy(a).to("cuda")
    kw = dict(causal=True, scale=w.scale, kv_offsets=to(off), kv_indices=to(idx))
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], q_offsets=to(t_off), q_indices=to(t_idx),
                             store_ds=store_ds, **kw)
    torch.cuda.synchronize()
    sp = dict(block=128, offsets=off, indices=idx)
    dQ, dK, dV, O, L = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale,
                                                 sparse=sp, return_forward=True)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)
    assert_close("dQ", dq, dQ, TOL_OUT)
    assert_close("dK", dk, dK, TOL_OUT)
    assert_close("dV", dv, dV, TOL_OUT)


def test_wrappers_refuse_mis_shaped_outputs(fa):
    w = W.small(1, 2, 200, 128, causal=True, seed=24, direction="bwd")
    g = dev(W.make_inputs(w))
    short = torch.empty(1, 2, 199, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.fwd(g["q"], g["k"], g["v"], causal=True, out=short)
    with pytest.raises(ValueError):
        fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, lse=torch.empty(1, 2, 100, device="cuda"))
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True)
    with pytest.raises(ValueError):
        fa.attn_bwd(g["q"], g["k"], g["v"], o[:, :, :100], lse, g["do"], causal=True)
    with pytest.raises(TypeError):
        fa.bwd(g["q"], g["k"], g["v"], o, lse.double(), g["do"], causal=True)


@SCHEDULES
def test_sparse_varlen_gqa_together(fa, store_ds):
    lens = (300, 700, 129)
    w = W.small(H=4, d=128, causal=True, seed=21, H_kv=2, seqlens=lens, direction="bwd", sigma=0.5)
    x = W.make_inputs(w)
    g = dev(x)
    cu = w.cu_seqlens()
    nb = (max(lens) + 127) // 128
    off, idx, sp = lists_for(nb, 1, 3, True)
    kw = dict(causal=True, scale=w.scale, cu_seqlens=cu, kv_offsets=off, kv_indices=idx)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], store_ds=store_ds, **kw)
    torch.cuda.synchronize()
    dQ, dK, dV, O, L = oracle.attention_backward_varlen(x["q"], x["k"], x["v"], x["do"], cu, causal=True,
                                                        scale=w.scale, sparse=sp, return_forward=True)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)
    assert_close("dQ", dq, dQ, TOL_OUT)
    assert_close("dK", dk, dK, TOL_OUT)
    assert_close("dV", dv, dV, TOL_OUT)


def test_sparse_backward_is_deterministic(fa):
    w = W.small(1, 2, 1024, 128, causal=True, seed=22, direction="bwd")
    g = dev(W.make_inputs(w))
    off, idx = fa.make_block_lists(8, 1, 3, causal=True)
    kw = dict(causal=True, scale=w.scale, kv_offsets=off, kv_indices=idx)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw)
    a = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], **kw)
    b = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], **kw)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ----------------------------------------------------------------------------- full-size workloads
def test_workload_gqa_h32kv8_n32k(fa):
    w = W.WORKLOADS["gqa_h32kv8_n32k"]
    x = W.make_inputs(w)
    g = dev(x)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert_finite("o", o)
    rows = sample_rows(w.N, 256, np.random.default_rng(6), extra=16)[::4]
    for h in (0, 3, 4, 31):   # heads 0-3 share K/V head 0, head 4 starts K/V head 1
        O, L = oracle.attention_forward(x["q"][:, h:h + 1], x["k"][:, h // 4:h // 4 + 1],
                                        x["v"][:, h // 4:h // 4 + 1], causal=True, scale=w.scale, rows=rows)
        assert_close(f"O[h{h}]", o[0, h, rows], O[0, 0, rows], TOL_OUT)
        assert_close(f"LSE[h{h}]", lse[0, h, rows], L[0, 0, rows], TOL_LSE)


def test_workload_gqa_bwd_b2h32kv8_n8k(fa):
    w = W.WORKLOADS["gqa_bwd_b2h32kv8_n8k"]
    x = W.make_inputs(w)
    g = dev(x)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert_finite(n, t)
    b, hk = 1, 5
    rows = sample_rows(w.N, 1024, np.random.default_rng(8), extra=8)
    ref = oracle.backward_rows_dq(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale, b=b, h=4 * hk + 2,
                                  rows=rows)
    assert_close("dQ rows", dq[b, 4 * hk + 2, rows], np.stack([ref[int(r)] for r in rows]), TOL_OUT)
    keys = [w.N - 1, w.N - 60, w.N - 129, w.N - 200]
    acc = oracle.backward_keys_dkdv(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale, b=b, h_kv=hk,
                                    keys=keys, rows=range(min(keys), w.N))
    assert_close("dK keys", dk[b, hk, keys], np.stack([acc[j][0] for j in keys]), TOL_OUT)
    assert_close("dV keys", dv[b, hk, keys], np.stack([acc[j][1] for j in keys]), TOL_OUT)


def _seq(x, cu, s, heads):
    """(1, h, n, d) fp64 slices of packed tensors for sequence s and the given heads."""
    a, e = int(cu[s]), int(cu[s + 1])
    return {n: f64(t[a:e, heads]).transpose(1, 0, 2)[None] for n, t in x.items()}


def test_workload_varlen_h32_b16(fa):
    w = W.WORKLOADS["varlen_h32_b16"]
    x = W.make_inputs(w)
    g = dev(x)
    cu = w.cu_seqlens()
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale, cu_seqlens=cu, max_seqlen=w.N)
    torch.cuda.synchronize()
    assert_finite("o", o)
    rng = np.random.default_rng(7)
    for s in (0, 8, 13, 15):
        n = int(cu[s + 1] - cu[s])
        rows = sample_rows(n, 256, rng, extra=8)[::3]
        h = int(rng.integers(0, w.H))
        sx = _seq(x, cu, s, [h])
        O, L = oracle.attention_forward(sx["q"], sx["k"], sx["v"], causal=True, scale=w.scale, rows=rows)
        pr = cu[s] + rows
        assert_close(f"O[s{s}h{h}]", o[pr, h], O[0, 0, rows], TOL_OUT)
        assert_close(f"LSE[s{s}h{h}]", lse[h, pr], L[0, 0, rows], TOL_LSE)


def test_workload_varlen_bwd_h32_b16(fa):
    w = W.WORKLOADS["varlen_bwd_h32_b16"]
    x = W.make_inputs(w)
    g = dev(x)
    cu = w.cu_seqlens()
    kw = dict(causal=True, scale=w.scale, cu_seqlens=cu, max_seqlen=w.N)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], **kw)
    torch.cuda.synchronize()
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert_finite(n, t)
    # the shortest sequence whole (all its outputs), for two heads
    s = int(np.argmin(np.diff(cu)))
    heads = [0, 17]
    sx = _seq(x, cu, s, heads)
    dQ, dK, dV = oracle.attention_backward(sx["q"], sx["k"], sx["v"], sx["do"], causal=True, scale=w.scale)
    a, e = int(cu[s]), int(cu[s + 1])
    for j, h in enumerate(heads):
        assert_close(f"dQ[s{s}h{h}]", dq[a:e, h], dQ[0, j], TOL_OUT)
        assert_close(f"dK[s{s}h{h}]", dk[a:e, h], dK[0, j], TOL_OUT)
        assert_close(f"dV[s{s}h{h}]", dv[a:e, h], dV[0, j], TOL_OUT)
    # sampled dQ rows of a long sequence
    s = int(np.argmax(np.diff(cu)))
    sx = _seq(x, cu, s, [9])
    n = int(cu[s + 1] - cu[s])
    rows = sample_rows(n, 1024, np.random.default_rng(9), extra=8)
    ref = oracle.backward_rows_dq(sx["q"], sx["k"], sx["v"], sx["do"], causal=True, scale=w.scale, rows=rows)
    assert_close("dQ rows", dq[int(cu[s]) + rows, 9], np.stack([ref[int(r)] for r in rows]), TOL_OUT)


def test_workload_sparse_bwd_h16_n128k(fa):
    w = W.WORKLOADS["sparse_bwd_h16_n128k"]
    x = W.make_inputs(w)
    g = dev(x)
    nb = w.N // 128
    off, idx = fa.make_block_lists(nb, 8, 16, causal=True)
    t_off, t_idx = fa.transpose_block_lists(off, idx, nb)
    to = lambda a: torch.from_numpy(a).to("cuda")
    kw = dict(causal=True, scale=w.scale, kv_offsets=to(off), kv_indices=to(idx))
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw)
    dq, dk, dv = fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], q_offsets=to(t_off), q_indices=to(t_idx), **kw)
    torch.cuda.synchronize()
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert_finite(n, t)
    sp = dict(block=128, offsets=off, indices=idx)
    h = 11
    rows = sample_rows(w.N, 8192, np.random.default_rng(4), extra=8)
    ref = oracle.backward_rows_dq(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale, sparse=sp, h=h,
                                  rows=rows)
    assert_close("dQ rows", dq[0, h, rows], np.stack([ref[int(r)] for r in rows]), TOL_OUT)
    # keys of the last block (seen by one query block) and of a block 20 from the end (seen
    # through the window and the stride): only the query blocks the key-side lists name
    for kb in (nb - 1, nb - 20):
        keys = [kb * 128, kb * 128 + 77, kb * 128 + 127]
        qbs = oracle.transpose_lists(off, idx, nb)
        qblocks = qbs[1][qbs[0][kb]:qbs[0][kb + 1]]
        rows_k = np.concatenate([np.arange(q * 128, q * 128 + 128) for q in qblocks])
        acc = oracle.backward_keys_dkdv(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale, sparse=sp,
                                        h_kv=h, keys=keys, rows=rows_k)
        assert_close(f"dK[kb{kb}]", dk[0, h, keys], np.stack([acc[j][0] for j in keys]), TOL_OUT)
        assert_close(f"dV[kb{kb}]", dv[0, h, keys], np.stack([acc[j][1] for j in keys]), TOL_OUT)


# ----------------------------------------------------------------------------- fp8 (e4m3) inputs
def dequant(x, n):
    """fp64 values of an fp8 input: code x descale (exact)."""
    return x[n].to(torch.float64) * x[n + "_descale"]


def fp8_kw(x):
    return dict(q_descale=x["q_descale"], k_descale=x["k_descale"], v_descale=x["v_descale"])


FP8_CASES = [
    # B, H, H_kv, N, d, causal, layout
    (1, 2, 2, 300, 128, True, "bhnd"),
    (2, 2, 1, 257, 64, False, "bnhd"),
    (1, 4, 2, 64, 128, True, "bhnd"),
    (1, 1, 1, 1, 128, False, "bhnd"),
    (1, 2, 2, 640, 64, True, "bhnd"),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "b{}h{}kv{}n{}d{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "", c[6]))
def test_fp8_forward_small(fa, case):
    B, H, Hkv, N, d, causal, layout = case
    w = W.small(B, H, N, d, causal=causal, layout=layout, seed=30, H_kv=Hkv, dtype="fp8_e4m3")
    x = W.make_inputs(w)
    g = {n: x[n].to("cuda") for n in "qkv"}
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=causal, scale=w.scale, **fp8_kw(x))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    O, L = oracle.attention_forward(dequant(x, "q"), dequant(x, "k"), dequant(x, "v"), causal=causal,
                                    scale=w.scale)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)


def test_fp8_sparse_and_packed(fa):
    lens = (300, 700, 129)
    w = W.small(H=2, d=128, causal=True, seed=31, seqlens=lens, dtype="fp8_e4m3")
    x = W.make_inputs(w)
    g = {n: x[n].to("cuda") for n in "qkv"}
    cu = w.cu_seqlens()
    off, idx, sp = lists_for((max(lens) + 127) // 128, 1, 3, True)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale, cu_seqlens=cu, kv_offsets=off,
                         kv_indices=idx, **fp8_kw(x))
    torch.cuda.synchronize()
    O, L = oracle.attention_forward_varlen(dequant(x, "q"), dequant(x, "k"), dequant(x, "v"), cu, causal=True,
                                           scale=w.scale, sparse=sp)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)


@pytest.mark.parametrize("sparse", [False, True])
def test_fp8_negative_scale(fa, sparse):
    # the e4m3 Q codes get their sign bit flipped and the scale's magnitude is used
    w = W.small(1, 2, 300, 128, causal=True, seed=32, dtype="fp8_e4m3")
    x = W.make_inputs(w)
    g = {n: x[n].to("cuda") for n in "qkv"}
    sc = float(np.float32(-1.3 * w.scale))
    kw = {}
    sp = None
    if sparse:
        off, idx, sp = lists_for((300 + 127) // 128, 1, 2, True)
        kw = dict(kv_offsets=off, kv_indices=idx)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=sc, **kw, **fp8_kw(x))
    torch.cuda.synchronize()
    O, L = oracle.attention_forward(dequant(x, "q"), dequant(x, "k"), dequant(x, "v"), causal=True, scale=sc,
                                    sparse=sp)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)


def test_fp8_descales_scale_the_result(fa):
    # the same codes with V's descale doubled give exactly twice the output (a power of two);
    # doubling Q's descale and halving K's leaves the scores, so O and LSE are unchanged
    w = W.small(1, 2, 500, 128, causal=True, seed=32, dtype="fp8_e4m3")
    x = W.make_inputs(w)
    g = {n: x[n].to("cuda") for n in "qkv"}
    kw = fp8_kw(x)
    o1, l1 = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale, **kw)
    o2, l2 = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale,
                         **{**kw, "v_descale": 2 * kw["v_descale"]})
    o3, l3 = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale,
                         **{**kw, "q_descale": 2 * kw["q_descale"], "k_descale": kw["k_descale"] / 2})
    torch.cuda.synchronize()
    assert torch.equal(o2.float(), 2 * o1.float()) and torch.equal(l1, l2)
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_workload_fp8_h32_n32k(fa):
    w = W.WORKLOADS["fp8_h32_n32k"]
    x = W.make_inputs(w)
    g = {n: x[n].to("cuda") for n in "qkv"}
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], causal=True, scale=w.scale, **fp8_kw(x))
    torch.cuda.synchronize()
    assert_finite("o", o)
    rows = sample_rows(w.N, 256, np.random.default_rng(10), extra=16)[::4]
    for h in (0, 17, 31):
        sl = lambda n: dequant(x, n)[:, h:h + 1]
        O, L = oracle.attention_forward(sl("q"), sl("k"), sl("v"), causal=True, scale=w.scale, rows=rows)
        assert_close(f"O[h{h}]", o[0, h, rows], O[0, 0, rows], TOL_OUT)
        assert_close(f"LSE[h{h}]", lse[0, h, rows], L[0, 0, rows], TOL_LSE)


# ----------------------------------------------------------------------------- seeded random mix
def _random_case(rng):
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.integers(1, 4))
    causal = bool(rng.integers(0, 2))
    packed = bool(rng.integers(0, 2))
    lens = tuple(int(x) for x in rng.integers(0, 600, size=int(rng.integers(1, 4)))) if packed else None
    N = max(lens) if packed else int(rng.integers(1, 600))
    if packed and N == 0:
        lens, N = lens + (1,), max(1, N)
    B = len(lens) if packed else int(rng.integers(1, 3))
    sparse = bool(rng.integers(0, 2)) and N > 128
    window, stride = int(rng.integers(0, 3)), int(rng.integers(0, 5))
    return B, H, Hkv, N, d, causal, lens, sparse, window, stride


@pytest.mark.parametrize("seed", range(40))
def test_backward_seeded_random_mix(fa, seed):
    """Forty seeded draws over head dimension, grouping, causality, packed lengths (empty and
    one-row sequences included) and block lists; forward and both backward schedules against
    the oracle."""
    rng = np.random.default_rng(1000 + seed)
    B, H, Hkv, N, d, causal, lens, sparse, window, stride = _random_case(rng)
    sys.__stderr__.write(f"[case] B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} lens={lens} "
                         f"sparse={sparse} w={window} s={stride}\n")
    w = W.small(B, H, N, d, causal=causal, seed=40 + seed, H_kv=Hkv, seqlens=lens, direction="bwd", sigma=0.5)
    x = W.make_inputs(w)
    g = dev(x)
    kw = dict(causal=causal, scale=w.scale)
    sp = None
    if lens is not None:
        kw["cu_seqlens"] = w.cu_seqlens()
    if sparse:
        nb = (N + 127) // 128
        off, idx, sp = lists_for(nb, window, stride, causal)
        kw.update(kv_offsets=off, kv_indices=idx)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw)
    outs = {flag: fa.attn_bwd(g["q"], g["k"], g["v"], o, lse, g["do"], store_ds=flag, **kw)
            for flag in ((None, False) if d == 128 else (False,))}
    torch.cuda.synchronize()
    if lens is not None:
        dQ, dK, dV, O, L = oracle.attention_backward_varlen(x["q"], x["k"], x["v"], x["do"], w.cu_seqlens(),
                                                            causal=causal, scale=w.scale, sparse=sp,
                                                            return_forward=True)
    else:
        dQ, dK, dV, O, L = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=causal,
                                                     scale=w.scale, sparse=sp, return_forward=True)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)
    for dq, dk, dv in outs.values():
        assert_close("dQ", dq, dQ, TOL_OUT)
        assert_close("dK", dk, dK, TOL_OUT)
        assert_close("dV", dv, dV, TOL_OUT)


@pytest.mark.parametrize("seed", range(40))
def test_forward_seeded_random_mix(fa, seed):
    """Forty seeded draws for the forward (both layouts when not packed, scales other than
    1/sqrt(d) included) against the oracle's output and LSE."""
    rng = np.random.default_rng(2000 + seed)
    B, H, Hkv, N, d, causal, lens, sparse, window, stride = _random_case(rng)
    layout = "bhnd" if lens is not None or rng.integers(0, 2) else "bnhd"
    sys.__stderr__.write(f"[case] B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} lens={lens} "
                         f"sparse={sparse} w={window} s={stride} layout={layout}\n")
    w = W.small(B, H, N, d, causal=causal, seed=80 + seed, H_kv=Hkv, seqlens=lens, layout=layout)
    x = W.make_inputs(w)
    g = dev(x)
    scale = float(w.scale * rng.choice([1.0, 0.5, 2.0]))
    kw = dict(causal=causal, scale=scale)
    sp = None
    if lens is not None:
        kw["cu_seqlens"] = w.cu_seqlens()
    if sparse:
        nb = (N + 127) // 128
        off, idx, sp = lists_for(nb, window, stride, causal)
        kw.update(kv_offsets=off, kv_indices=idx)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw)
    torch.cuda.synchronize()
    if lens is not None:
        O, L = oracle.attention_forward_varlen(x["q"], x["k"], x["v"], w.cu_seqlens(), causal=causal, scale=scale,
                                               sparse=sp)
    else:
        O, L = oracle.attention_forward(x["q"], x["k"], x["v"], causal=causal, scale=scale, sparse=sp)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)


@pytest.mark.parametrize("seed", range(20))
def test_fp8_forward_seeded_random_mix(fa, seed):
    """Twenty seeded draws of the fp8 forward (head dimension, grouping, causality, packed
    lengths, block lists, layouts) against the oracle on the dequantized inputs."""
    rng = np.random.default_rng(3000 + seed)
    B, H, Hkv, N, d, causal, lens, sparse, window, stride = _random_case(rng)
    layout = "bhnd" if lens is not None or rng.integers(0, 2) else "bnhd"
    sys.__stderr__.write(f"[case] fp8 B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} lens={lens} "
                         f"sparse={sparse} w={window} s={stride} layout={layout}\n")
    w = W.small(B, H, N, d, causal=causal, seed=120 + seed, H_kv=Hkv, seqlens=lens, layout=layout,
                dtype="fp8_e4m3")
    x = W.make_inputs(w)
    g = {n: x[n].to("cuda") for n in "qkv"}
    kw = dict(causal=causal, scale=w.scale)
    sp = None
    if lens is not None:
        kw["cu_seqlens"] = w.cu_seqlens()
    if sparse:
        off, idx, sp = lists_for((N + 127) // 128, window, stride, causal)
        kw.update(kv_offsets=off, kv_indices=idx)
    o, lse = fa.attn_fwd(g["q"], g["k"], g["v"], **kw, **fp8_kw(x))
    torch.cuda.synchronize()
    if lens is not None:
        O, L = oracle.attention_forward_varlen(dequant(x, "q"), dequant(x, "k"), dequant(x, "v"), w.cu_seqlens(),
                                               causal=causal, scale=w.scale, sparse=sp)
    else:
        O, L = oracle.attention_forward(dequant(x, "q"), dequant(x, "k"), dequant(x, "v"), causal=causal,
                                        scale=w.scale, sparse=sp)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)


# ----------------------------------------------------------------------------- outputs in padded views
@pytest.mark.parametrize("sparse", [False, True])
def test_outputs_into_padded_views_touch_nothing_else(fa, sparse):
    # The epilogues stage each wave's rows in LDS and store whole rows: with O, dQ, dK, dV
    # as views into larger buffers (row stride d + 64, eight spare rows per head) the
    # results must match the oracle and the padding must keep its sentinel.
    B, H, N, d = 1, 2, 333, 128
    w = W.small(B, H, N, d, causal=True, seed=91, direction="bwd", sigma=0.5)
    x = W.make_inputs(w)
    q, k, v, do = (x[n].to("cuda") for n in ("q", "k", "v", "do"))
    sentinel = 7.0

    def padded():
        buf = torch.full((B, H, N + 8, d + 64), sentinel, dtype=torch.bfloat16, device="cuda")
        return buf, buf[:, :, :N, :d]

    def untouched(buf):
        return bool((buf[:, :, N:, :] == sentinel).all()) and bool((buf[:, :, :, d:] == sentinel).all())

    ob, o = padded()
    if sparse:
        off, idx = fa.make_block_lists(3, 1, 2, causal=True, rule="strided")
        o, lse = fa.attn_fwd(q, k, v, causal=True, scale=w.scale, kv_offsets=off, kv_indices=idx, out=o)
        sp = dict(block=128, window=1, stride=2, rule="strided")
    else:
        o, lse = fa.fwd(q, k, v, causal=True, scale=w.scale, out=o)
        sp = None
    (dqb, dq), (dkb, dk), (dvb, dv) = padded(), padded(), padded()
    kw = dict(kv_offsets=off, kv_indices=idx) if sparse else {}
    fa.attn_bwd_noalloc(q, k, v, o, lse, do, causal=True, scale=w.scale, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    for name, buf in (("O", ob), ("dQ", dqb), ("dK", dkb), ("dV", dvb)):
        assert untouched(buf), f"{name}: padding overwritten"
    dQ, dK, dV, O, L = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], causal=True, scale=w.scale,
                                                 sparse=sp, return_forward=True)
    assert_close("O", o, O, TOL_OUT)
    assert_close("LSE", lse, L, TOL_LSE)
    assert_close("dQ", dq, dQ, TOL_OUT)
    assert_close("dK", dk, dK, TOL_OUT)
    assert_close("dV", dv, dV, TOL_OUT)
