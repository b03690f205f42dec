"""Pins for the oracle's grouped-head, variable-length and key-side-list extensions.

Each is checked against something other than the oracle's own loop: torch CPU fp64
(scaled_dot_product_attention with grouped heads, autograd through a replicated or
masked formulation), whole-matrix brute force with an explicit mask, closed forms and
invariants. A wrong head mapping (h % H_kv instead of h // (H / H_kv)), a gradient that
is not summed over the group, a sequence boundary off by one, positions or block numbers
counted from the pack instead of the sequence, or a transposed list that is not the exact
converse fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (attention_backward, attention_backward_varlen, attention_forward,
                    attention_forward_varlen, block_lists, key_mask_from_lists, kv_head,
                    transpose_lists)

SDPA = torch.nn.functional.scaled_dot_product_attention


def t64(shape, g):
    return torch.randn(*shape, generator=g, dtype=torch.float64)


# ----------------------------------------------------------------------------- grouped heads
def test_kv_head_mapping_groups_consecutive_query_heads():
    assert [kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [kv_head(h, 6, 1) for h in range(6)] == [0] * 6
    assert [kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        kv_head(0, 6, 4)


@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 3), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_forward_matches_torch_sdpa_gqa(H, H_kv, causal):
    g = torch.Generator().manual_seed(40 + H + H_kv)
    B, n, d = 2, 37, 16
    Q, K, V = t64((B, H, n, d), g), t64((B, H_kv, n, d), g), t64((B, H_kv, n, d), g)
    scale = 0.3
    ref = SDPA(Q, K, V, is_causal=causal, scale=scale, enable_gqa=True)
    O, L = attention_forward(Q.numpy(), K.numpy(), V.numpy(), causal=causal, scale=scale)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)
    # LSE from the replicated formulation, whole-matrix
    Kr = K.repeat_interleave(H // H_kv, dim=1)
    S = scale * Q @ Kr.transpose(-1, -2)
    if causal:
        S = S.masked_fill(~torch.tril(torch.ones(n, n, dtype=torch.bool)), -math.inf)
    np.testing.assert_allclose(L, torch.logsumexp(S, -1).numpy(), atol=1e-12)


@pytest.mark.parametrize("H,H_kv", [(4, 2), (3, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_backward_matches_autograd_through_replication(H, H_kv, causal):
    g = torch.Generator().manual_seed(50 + H)
    B, n, d = 1, 29, 8
    Q, dO = t64((B, H, n, d), g), t64((B, H, n, d), g)
    K, V = t64((B, H_kv, n, d), g), t64((B, H_kv, n, d), g)
    scale = 0.45
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    G = H // H_kv
    S = scale * q @ k.repeat_interleave(G, dim=1).transpose(-1, -2)
    if causal:
        S = S.masked_fill(~torch.tril(torch.ones(n, n, dtype=torch.bool)), -math.inf)
    (torch.softmax(S, -1) @ v.repeat_interleave(G, dim=1)).backward(dO)
    dQ, dK, dV = attention_backward(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=causal, scale=scale)
    assert dK.shape == K.shape and dV.shape == V.shape
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, v.grad.numpy(), atol=1e-12)


def test_grouped_backward_group_invariants():
    r = np.random.default_rng(41)
    H, H_kv, n, d = 6, 2, 40, 8
    Q, dO = r.normal(size=(1, H, n, d)), r.normal(size=(1, H, n, d))
    K, V = r.normal(size=(1, H_kv, n, d)), r.normal(size=(1, H_kv, n, d))
    dQ, dK, dV = attention_backward(Q, K, V, dO, causal=True, scale=0.5)
    G = H // H_kv
    for kvh in range(H_kv):
        heads = range(kvh * G, (kvh + 1) * G)
        # each query row's probabilities sum to 1: dV of a K/V head collects all of its group's dO
        np.testing.assert_allclose(dV[0, kvh].sum(axis=0), sum(dO[0, h].sum(axis=0) for h in heads), atol=1e-12)
        # a common shift of all keys leaves every softmax unchanged
        np.testing.assert_allclose(dK[0, kvh].sum(axis=0), 0.0, atol=1e-12)


def test_multi_query_equals_each_head_alone():
    r = np.random.default_rng(42)
    H, n, d = 3, 33, 8
    Q = r.normal(size=(1, H, n, d))
    K, V = r.normal(size=(1, 1, n, d)), r.normal(size=(1, 1, n, d))
    O, L = attention_forward(Q, K, V, causal=True, scale=0.4)
    for h in range(H):
        o, l = attention_forward(Q[:, h:h + 1], K, V, causal=True, scale=0.4)
        np.testing.assert_array_equal(O[:, h:h + 1], o)
        np.testing.assert_array_equal(L[:, h:h + 1], l)


# ----------------------------------------------------------------------------- variable length
def block_diagonal_mask(cu, causal):
    T = int(cu[-1])
    m = np.zeros((T, T), dtype=bool)
    for s, e in zip(cu[:-1], cu[1:]):
        blk = np.ones((e - s, e - s), dtype=bool)
        m[s:e, s:e] = np.tril(blk) if causal else blk
    return m


def masked_dense(Q, K, V, mask, scale):
    """Whole-matrix attention over the packed tokens (one head), fully masked rows -> 0 / -inf."""
    S = np.where(mask, scale * (Q @ K.T), -np.inf)
    m = S.max(axis=1, keepdims=True)
    safe = np.where(np.isinf(m), 0.0, m)
    E = np.exp(S - safe)
    l = E.sum(axis=1, keepdims=True)
    P = np.divide(E, l, out=np.zeros_like(E), where=l > 0)
    with np.errstate(divide="ignore"):
        lse = np.where(l[:, 0] > 0, safe[:, 0] + np.log(l[:, 0]), -np.inf)
    return P @ V, lse


CU_CASES = [[0, 5, 5, 17, 18, 40], [0, 64], [0, 1, 2, 3], [0, 0, 23]]


@pytest.mark.parametrize("cu", CU_CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_forward_is_block_diagonal_attention(cu, causal):
    r = np.random.default_rng(43 + len(cu))
    T, H, H_kv, d = cu[-1], 4, 2, 8
    Q, K, V = r.normal(size=(T, H, d)), r.normal(size=(T, H_kv, d)), r.normal(size=(T, H_kv, d))
    mask = block_diagonal_mask(cu, causal)
    O, L = attention_forward_varlen(Q, K, V, cu, causal=causal, scale=0.35)
    assert O.shape == (T, H, d) and L.shape == (H, T)
    for h in range(H):
        o, lse = masked_dense(Q[:, h], K[:, h // 2], V[:, h // 2], mask, 0.35)
        np.testing.assert_allclose(O[:, h], o, atol=1e-12)
        np.testing.assert_allclose(L[h], lse, atol=1e-12)


def test_varlen_forward_matches_sdpa_on_padded_batch():
    g = torch.Generator().manual_seed(44)
    cu = [0, 7, 30, 31, 50]
    lens = np.diff(cu)
    B, Nmax, H, d = len(lens), int(lens.max()), 2, 16
    Qp, Kp, Vp = (t64((B, H, Nmax, d), g) for _ in range(3))
    pad = torch.zeros(B, 1, Nmax, Nmax, dtype=torch.bool)
    for b, n in enumerate(lens):
        pad[b, :, :n, :n] = torch.tril(torch.ones(n, n, dtype=torch.bool))
    pad[:, :, torch.arange(Nmax), torch.arange(Nmax)] |= True   # keep padding rows finite in SDPA
    ref = SDPA(Qp, Kp, Vp, attn_mask=pad, scale=0.25)
    pack = lambda X: np.concatenate([X[b, :, :n].numpy().transpose(1, 0, 2) for b, n in enumerate(lens)])
    O, _ = attention_forward_varlen(pack(Qp), pack(Kp), pack(Vp), cu, causal=True, scale=0.25)
    np.testing.assert_allclose(O, pack(ref), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_matches_autograd_on_masked_pack(causal):
    g = torch.Generator().manual_seed(45)
    cu = [0, 9, 10, 31]
    T, H, H_kv, d = cu[-1], 2, 1, 8
    Q, dO = t64((T, H, d), g), t64((T, H, d), g)
    K, V = t64((T, H_kv, d), g), t64((T, H_kv, d), g)
    mask = torch.from_numpy(block_diagonal_mask(cu, causal))
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    outs = []
    for h in range(H):
        S = (0.4 * q[:, h] @ k[:, 0].T).masked_fill(~mask, -math.inf)
        outs.append(torch.softmax(S, -1) @ v[:, 0])
    torch.stack(outs, 1).backward(dO)
    dQ, dK, dV = attention_backward_varlen(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), cu,
                                           causal=causal, scale=0.4)
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, v.grad.numpy(), atol=1e-12)


def test_varlen_sparse_counts_blocks_from_each_sequence_start():
    r = np.random.default_rng(46)
    cu = [0, 20, 57]   # block 8: sequence 1 starts mid-block in the pack
    T, H, d, blk = cu[-1], 1, 8, 8
    Q, K, V = (r.normal(size=(T, H, d)) for _ in range(3))
    sp = dict(block=blk, window=1, stride=3, rule="strided")
    O, L = attention_forward_varlen(Q, K, V, cu, causal=True, scale=0.5, sparse=sp)
    for s, e in zip(cu[:-1], cu[1:]):
        n = e - s
        off, idx = block_lists((n + blk - 1) // blk, 1, 3, True, "strided")
        mask = key_mask_from_lists(n, blk, off, idx, True)
        o, lse = masked_dense(Q[s:e, 0], K[s:e, 0], V[s:e, 0], mask, 0.5)
        np.testing.assert_allclose(O[s:e, 0], o, atol=1e-12)
        np.testing.assert_allclose(L[0, s:e], lse, atol=1e-12)


def test_varlen_rejects_inconsistent_offsets():
    X = np.zeros((5, 1, 4))
    for bad in ([0, 3], [1, 5], [0, 4, 3, 5]):
        with pytest.raises(ValueError):
            attention_forward_varlen(X, X, X, bad, causal=True, scale=1.0)


# ----------------------------------------------------------------------------- key-side lists
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rule", ["strided", "fixed"])
def test_transposed_lists_are_the_exact_converse(causal, rule):
    nb = 45
    off, idx = block_lists(nb, 3, 7, causal, rule)
    t_off, t_idx = transpose_lists(off, idx, nb)
    assert t_off[0] == 0 and t_off[-1] == len(idx) and np.all(np.diff(t_off) >= 0)
    fwd = {(q, int(k)) for q in range(nb) for k in idx[off[q]:off[q + 1]]}
    bwd = set()
    for k in range(nb):
        qs = t_idx[t_off[k]:t_off[k + 1]]
        assert np.all(np.diff(qs) > 0)
        bwd.update((int(q), k) for q in qs)
    assert fwd == bwd


def test_transposed_lists_closed_form_at_128k():
    # causal, window 8, strided 16: key block k is listed by q = k + t for t <= 8 or t % 16 == 0,
    # so its list has min(8, M) + 1 + floor(M / 16) entries, M = nb - 1 - k.
    nb = 1024
    off, idx = block_lists(nb, 8, 16, True, "strided")
    t_off, t_idx = transpose_lists(off, idx, nb)
    lens = np.diff(t_off)
    M = nb - 1 - np.arange(nb)
    np.testing.assert_array_equal(lens, np.minimum(8, M) + 1 + M // 16)
    assert int(lens.sum()) == 41436
    assert all(t_idx[t_off[k]] == k for k in range(nb))   # the diagonal block always comes first


# ----------------------------------------------------------------------------- sampled key gradients
@pytest.mark.parametrize("sparse", [None, dict(block=8, window=1, stride=3, rule="strided")])
def test_sampled_key_gradients_match_autograd(sparse):
    from oracle import backward_keys_dkdv, block_lists as bl
    g = torch.Generator().manual_seed(47)
    H, H_kv, n, d = 4, 2, 41, 8
    Q, dO = t64((1, H, n, d), g), t64((1, H, n, d), g)
    K, V = t64((1, H_kv, n, d), g), t64((1, H_kv, n, d), g)
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool))
    if sparse:
        off, idx = bl((n + 7) // 8, 1, 3, True, "strided")
        mask &= torch.from_numpy(key_mask_from_lists(n, 8, off, idx, True))
    S = (0.3 * q @ k.repeat_interleave(2, dim=1).transpose(-1, -2)).masked_fill(~mask, -math.inf)
    (torch.softmax(S, -1) @ v.repeat_interleave(2, dim=1)).backward(dO)
    keys = [0, 5, 17, 40]
    got = backward_keys_dkdv(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=True, scale=0.3, sparse=sparse,
                             h_kv=1, keys=keys)
    for j in keys:
        np.testing.assert_allclose(got[j][0], k.grad[0, 1, j].numpy(), atol=1e-12)
        np.testing.assert_allclose(got[j][1], v.grad[0, 1, j].numpy(), atol=1e-12)


# ----------------------------------------------------------------------------- fp8 inputs
def e4m3_by_definition(code: int) -> float:
    """OCP 8-bit e4m3 (E4M3FN): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
    holds the subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_fp8_e4m3_decode_matches_the_format_definition():
    # the oracle sees fp8 inputs as code x descale in fp64; pin the code decoding used for it
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    got = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = np.array([e4m3_by_definition(c) for c in range(256)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert want[~nan].max() == 448.0 and want[1] == 2.0 ** -9   # largest finite, smallest subnormal


def test_fp8_dequantisation_is_exact_in_fp64():
    # code (4 significant bits) x fp32 descale (24 bits) fits the 53-bit fp64 mantissa
    import workloads as W
    x = W.make_inputs(W.small(1, 2, 100, 64, seed=5, dtype="fp8_e4m3"))
    q = x["q"].to(torch.float64).numpy()
    deq = q * x["q_descale"]
    assert np.array_equal(deq / x["q_descale"], q)
    assert np.abs(q).max() <= 448.0


# ----------------------------------------------------------------------------- sampled query gradients
def _masked_autograd_dq(Q, K, V, dO, scale, mask, G):
    """dQ by torch fp64 autograd of softmax(scale Q K^T + mask) V with K, V replicated over
    groups of G query heads. Rows without any allowed key have P = 0 (and so dQ = 0): their
    scores are replaced by zeros and their probabilities multiplied by 0, which keeps the
    graph free of NaN."""
    q = Q.clone().requires_grad_(True)
    k = K.repeat_interleave(G, dim=1)
    v = V.repeat_interleave(G, dim=1)
    has = mask.any(-1, keepdim=True)
    S = (scale * q @ k.transpose(-1, -2)).masked_fill(~mask, -math.inf)
    S = torch.where(has, S, torch.zeros_like(S))
    P = torch.softmax(S, -1) * has
    (P @ v).backward(dO)
    return q.grad


@pytest.mark.parametrize("kind", ["dense", "causal", "lists", "rule"])
def test_sampled_query_gradients_match_autograd(kind):
    """backward_rows_dq (the dQ reference at sizes where the whole backward is too slow)
    against torch fp64 autograd, at a batch and query head other than (0, 0) of a grouped
    problem (H = 6 over H_kv = 2), for dense, causal and block-sparse masks; the explicit
    lists give one query block an empty list (its rows: dQ = 0) and one an entry above the
    diagonal (skipped under causal masking)."""
    from oracle import backward_rows_dq, block_lists as bl
    g = torch.Generator().manual_seed(53)
    B, H, H_kv, n, d, blk = 2, 6, 2, 43, 8, 8
    G = H // H_kv
    Q, dO = t64((B, H, n, d), g), t64((B, H, n, d), g)
    K, V = t64((B, H_kv, n, d), g), t64((B, H_kv, n, d), g)
    causal = kind != "dense"
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool)) if causal else torch.ones(n, n, dtype=torch.bool)
    sparse = None
    nb = (n + blk - 1) // blk
    if kind == "lists":
        # block 2 lists nothing; block 3 lists block 4 (above it: skipped) besides 1 and 3
        lists = {0: [0], 1: [0, 1], 2: [], 3: [1, 3, 4], 4: [2, 4], 5: [0, 5]}
        off = np.cumsum([0] + [len(lists[q]) for q in range(nb)]).astype(np.int64)
        idx = np.array([k for q in range(nb) for k in lists[q]], dtype=np.int64)
        sparse = dict(block=blk, offsets=off, indices=idx)
        mask &= torch.from_numpy(key_mask_from_lists(n, blk, off, idx, True))
        assert not mask[2 * blk:3 * blk].any()
    elif kind == "rule":
        off, idx = bl(nb, 1, 3, True, "strided")
        sparse = dict(block=blk, window=1, stride=3, rule="strided")
        mask &= torch.from_numpy(key_mask_from_lists(n, blk, off, idx, True))
    want = _masked_autograd_dq(Q, K, V, dO, 0.37, mask, G)
    rows = [0, 1, 7, 8, 16, 17, 23, 25, 31, 40, 42]
    for b, h in ((1, 4), (0, 5), (1, 2)):
        got = backward_rows_dq(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=causal, scale=0.37,
                               sparse=sparse, b=b, h=h, rows=rows)
        assert sorted(got) == rows
        for i in rows:
            np.testing.assert_allclose(got[i], want[b, h, i].numpy(), atol=1e-12, rtol=0)
    if kind == "lists":
        got = backward_rows_dq(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=True, scale=0.37,
                               sparse=sparse, b=1, h=4, rows=range(2 * blk, 3 * blk))
        assert all(np.all(got[i] == 0) for i in range(2 * blk, 3 * blk))


def test_sampled_query_gradients_agree_with_the_full_backward():
    """Same rows from backward_rows_dq and from attention_backward (grouped, causal, block
    rule): a mistake in either one's head mapping, scale or D fails here or above."""
    from oracle import backward_rows_dq
    g = torch.Generator().manual_seed(54)
    B, H, H_kv, n, d = 1, 4, 1, 37, 8
    Q, dO = t64((B, H, n, d), g), t64((B, H, n, d), g)
    K, V = t64((B, H_kv, n, d), g), t64((B, H_kv, n, d), g)
    sp = dict(block=8, window=1, stride=2, rule="strided")
    dQ, _, _ = attention_backward(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=True, scale=0.5, sparse=sp)
    for h in range(H):
        got = backward_rows_dq(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=True, scale=0.5, sparse=sp,
                               h=h, rows=range(n))
        np.testing.assert_allclose(np.stack([got[i] for i in range(n)]), dQ[0, h], atol=1e-12, rtol=0)
