"""Pins for the fp64 oracle: each test checks it against something other than itself.

Closed forms, a hand-worked case, brute force on tiny inputs, the online-softmax
recurrence of the pages, finite differences and a library routine (torch CPU fp64).
Chosen so that a dropped term, a wrong sign or index, a transposed operand, a wrong
causal boundary, a missing scale or a wrong logarithm base fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (KeySets, allowed_blocks, attention_backward, attention_forward,
                    block_lists, key_mask_from_lists, row_probabilities)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_4x4.json")


def rng(seed):
    return np.random.default_rng(seed)


def as_bhnd(x):
    return np.asarray(x, dtype=np.float64)[None, None]


# ----------------------------------------------------------------------------- brute force
def dense_reference(Q, K, V, scale, mask):
    """Whole-matrix attention written independently of the oracle's row loop."""
    S = scale * (Q @ K.T)
    S = np.where(mask, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    return P @ V, (m + np.log(l))[:, 0], P


def tril(n):
    return np.tril(np.ones((n, n), dtype=bool))


# ----------------------------------------------------------------------------- hand case
@pytest.fixture(scope="module")
def hand():
    with open(GOLDEN) as f:
        return json.load(f)


def hand_inputs():
    I = np.eye(4)
    return as_bhnd(I), as_bhnd(math.log(3.0) * I), as_bhnd(6.0 * I), as_bhnd(I)


@pytest.mark.parametrize("causal", [False, True])
def test_hand_4x4_forward(hand, causal):
    Q, K, V, _ = hand_inputs()
    O, L = attention_forward(Q, K, V, causal=causal, scale=1.0)
    ref = hand["causal" if causal else "noncausal"]
    np.testing.assert_allclose(O[0, 0], np.array(ref["O"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(L[0, 0], np.array(ref["LSE"]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_hand_4x4_backward(hand, causal):
    Q, K, V, dO = hand_inputs()
    dQ, dK, dV = attention_backward(Q, K, V, dO, causal=causal, scale=1.0)
    ref = hand["causal_bwd" if causal else "noncausal_bwd"]
    for got, name in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        np.testing.assert_allclose(got[0, 0], np.array(ref[name]), rtol=0, atol=1e-13, err_msg=name)


# ----------------------------------------------------------------------------- closed forms
def test_identical_keys_give_mean_of_v():
    r = rng(1)
    n, d = 37, 8
    q = r.normal(size=(n, d))
    k = np.tile(r.normal(size=(1, d)), (n, 1))
    v = r.normal(size=(n, d))
    scale = 0.3
    for causal in (False, True):
        O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=causal, scale=scale)
        for i in range(n):
            J = np.arange(i + 1) if causal else np.arange(n)
            s = scale * float(q[i] @ k[0])
            np.testing.assert_allclose(O[0, 0, i], v[J].mean(axis=0), atol=1e-13)
            assert abs(L[0, 0, i] - (s + math.log(len(J)))) < 1e-12


def test_one_hot_dominant_score_selects_its_v_row():
    r = rng(2)
    n, d = 64, 16
    scale = 0.25
    q = r.normal(size=(n, d))
    k = r.normal(size=(n, d)) * 0.1
    v = r.normal(size=(n, d))
    i, jstar = 40, 17
    k[jstar] = 40.0 * q[i] / float(q[i] @ q[i]) / scale    # s_{i,j*} = 40
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=False, scale=scale, rows=[i])
    others = scale * (np.delete(k, jstar, axis=0) @ q[i])
    bound = n * math.exp(-(40.0 - others.max()))
    assert bound < 1e-10
    np.testing.assert_allclose(O[0, 0, i], v[jstar], atol=bound * np.abs(v).max() * 4 + 1e-14)
    assert abs(L[0, 0, i] - 40.0) <= bound * 2 + 1e-13


def test_row_constant_shift_changes_only_lse():
    r = rng(3)
    n, d = 50, 12
    scale = 0.4
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    c = r.normal(size=n) * 3.0
    q2 = np.concatenate([q, (c / scale)[:, None]], axis=1)   # adds c_i to every score of row i
    k2 = np.concatenate([k, np.ones((n, 1))], axis=1)
    for causal in (False, True):
        O1, L1 = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=causal, scale=scale)
        O2, L2 = attention_forward(as_bhnd(q2), as_bhnd(k2), as_bhnd(v), causal=causal, scale=scale)
        np.testing.assert_allclose(O2, O1, atol=1e-12)
        np.testing.assert_allclose(L2[0, 0], L1[0, 0] + c, atol=1e-12)


def test_permutation_equivariance_noncausal():
    r = rng(4)
    n, d = 45, 10
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=False, scale=0.3)
    pk = r.permutation(n)
    O2, L2 = attention_forward(as_bhnd(q), as_bhnd(k[pk]), as_bhnd(v[pk]), causal=False, scale=0.3)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)
    pq = r.permutation(n)
    O3, L3 = attention_forward(as_bhnd(q[pq]), as_bhnd(k), as_bhnd(v), causal=False, scale=0.3)
    np.testing.assert_allclose(O3[0, 0], O[0, 0][pq], atol=1e-13)
    np.testing.assert_allclose(L3[0, 0], L[0, 0][pq], atol=1e-13)


def test_probability_rows_sum_to_one_long_row():
    r = rng(5)
    s = r.normal(size=131072) * 3.0
    p, m, l = row_probabilities(s)
    assert abs(p.sum() - 1.0) < 1e-12
    assert m == s.max()
    assert np.all(p >= 0)


def test_lse_and_output_bounds():
    r = rng(6)
    n, d = 80, 16
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    scale = 0.5
    for causal in (False, True):
        O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=causal, scale=scale)
        for i in range(n):
            J = np.arange(i + 1) if causal else np.arange(n)
            s = scale * (k[J] @ q[i])
            assert s.max() - 1e-12 <= L[0, 0, i] <= s.max() + math.log(len(J)) + 1e-12
            assert np.all(O[0, 0, i] >= v[J].min(axis=0) - 1e-12)
            assert np.all(O[0, 0, i] <= v[J].max(axis=0) + 1e-12)


def test_causal_row_zero():
    r = rng(7)
    n, d = 20, 8
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=True, scale=0.7)
    np.testing.assert_allclose(O[0, 0, 0], v[0], atol=1e-15)
    assert abs(L[0, 0, 0] - 0.7 * float(q[0] @ k[0])) < 1e-14


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (64, 16), (130, 32)])
def test_matches_dense_matrix_path(causal, n, d):
    r = rng(100 + n)
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    mask = tril(n) if causal else np.ones((n, n), dtype=bool)
    O_ref, L_ref, _ = dense_reference(q, k, v, scale, mask)
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=causal, scale=scale)
    np.testing.assert_allclose(O[0, 0], O_ref, atol=1e-12)
    np.testing.assert_allclose(L[0, 0], L_ref, atol=1e-12)


def test_multi_head_batch_indexing():
    r = rng(8)
    B, H, n, d = 2, 3, 20, 8
    Q, K, V = (r.normal(size=(B, H, n, d)) for _ in range(3))
    O, L = attention_forward(Q, K, V, causal=True, scale=0.35)
    for b in range(B):
        for h in range(H):
            O_ref, L_ref, _ = dense_reference(Q[b, h], K[b, h], V[b, h], 0.35, tril(n))
            np.testing.assert_allclose(O[b, h], O_ref, atol=1e-12)
            np.testing.assert_allclose(L[b, h], L_ref, atol=1e-12)


# ----------------------------------------------------------------------------- page recurrence
def online_softmax_forward(q, k, v, scale, block, causal):
    """The tiled loop of "Flash MSA Attention Kernel Implementation..." (section "The
    Flash Core: Tiling Over the Memory Hierarchy"): per query block, a running max m,
    a running sum l and a rescaled output, normalised at the end. Written here in fp64
    as an independent cross-check of the plain definition."""
    n, d = q.shape
    out = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for q0 in range(0, n, block):
        qb = q[q0:q0 + block]
        rows = np.arange(q0, min(n, q0 + block))
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        o = np.zeros((len(rows), v.shape[1]))
        for k0 in range(0, n, block):
            s = scale * (qb @ k[k0:k0 + block].T)
            if causal:
                cols = np.arange(k0, min(n, k0 + block))
                s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            safe = np.where(np.isinf(m_new), 0.0, m_new)
            alpha = np.exp(m - safe)
            p = np.exp(s - safe[:, None])
            l = alpha * l + p.sum(axis=1)
            o = alpha[:, None] * o + p @ v[k0:k0 + block]
            m = m_new
        out[q0:q0 + block] = o / l[:, None]
        lse[q0:q0 + block] = m + np.log(l)
    return out, lse


@pytest.mark.parametrize("block", [1, 3, 16, 128, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_online_softmax_recurrence(block, causal):
    r = rng(9)
    n, d = 200, 16
    q, k, v = (r.normal(size=(n, d)) * 1.5 for _ in range(3))
    O_rec, L_rec = online_softmax_forward(q, k, v, 0.25, block, causal)
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=causal, scale=0.25)
    np.testing.assert_allclose(O[0, 0], O_rec, atol=1e-12)
    np.testing.assert_allclose(L[0, 0], L_rec, atol=1e-12)


# ----------------------------------------------------------------------------- library
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    g = torch.Generator().manual_seed(10)
    B, H, n, d = 2, 2, 96, 32
    Q, K, V = (torch.randn(B, H, n, d, generator=g, dtype=torch.float64) for _ in range(3))
    scale = 0.21
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool)) if causal else torch.ones(n, n, dtype=torch.bool)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    lse_ref = torch.logsumexp((scale * Q @ K.transpose(-1, -2)).masked_fill(~mask, -math.inf), dim=-1)
    O, L = attention_forward(Q.numpy(), K.numpy(), V.numpy(), causal=causal, scale=scale)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(L, lse_ref.numpy(), atol=1e-12)


def test_accepts_bf16_tensors_exactly():
    g = torch.Generator().manual_seed(11)
    Q, K, V = (torch.randn(1, 1, 33, 8, generator=g).to(torch.bfloat16) for _ in range(3))
    O, L = attention_forward(Q, K, V, causal=True, scale=0.5)
    O2, L2 = attention_forward(Q.double().numpy(), K.double().numpy(), V.double().numpy(),
                               causal=True, scale=0.5)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


# ----------------------------------------------------------------------------- backward
def loss_grad_fd(Q, K, V, dO, scale, causal, h=1e-6):
    def loss(q, k, v):
        O, _ = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=causal, scale=scale)
        return float(np.sum(O[0, 0] * dO))
    grads = []
    for which in range(3):
        args = [Q.copy(), K.copy(), V.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*g.shape):
            a_p = [x.copy() for x in args]
            a_m = [x.copy() for x in args]
            a_p[which][idx] += h
            a_m[which][idx] -= h
            g[idx] = (loss(*a_p) - loss(*a_m)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    r = rng(12)
    n, d = 7, 4
    Q, K, V, dO = (r.normal(size=(n, d)) for _ in range(4))
    scale = 0.7
    fd = loss_grad_fd(Q, K, V, dO, scale, causal)
    got = attention_backward(as_bhnd(Q), as_bhnd(K), as_bhnd(V), as_bhnd(dO), causal=causal, scale=scale)
    for g_fd, g, name in zip(fd, got, ("dQ", "dK", "dV")):
        np.testing.assert_allclose(g[0, 0], g_fd, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_fp64(causal):
    g = torch.Generator().manual_seed(13)
    B, H, n, d = 1, 2, 48, 16
    Q, K, V, dO = (torch.randn(B, H, n, d, generator=g, dtype=torch.float64) for _ in range(4))
    scale = 0.3
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    S = scale * q @ k.transpose(-1, -2)
    if causal:
        S = S.masked_fill(~torch.tril(torch.ones(n, n, dtype=torch.bool)), -math.inf)
    O = torch.softmax(S, dim=-1) @ v
    O.backward(dO)
    dQ, dK, dV = attention_backward(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=causal, scale=scale)
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, v.grad.numpy(), atol=1e-12)


def test_backward_invariants():
    r = rng(14)
    n, d = 60, 8
    Q, K, V, dO = (r.normal(size=(1, 1, n, d)) for _ in range(4))
    for causal in (False, True):
        dQ, dK, dV = attention_backward(Q, K, V, dO, causal=causal, scale=0.4)
        # softmax is unchanged by a common shift of all keys, so the key gradients sum to 0
        np.testing.assert_allclose(dK[0, 0].sum(axis=0), 0.0, atol=1e-12)
        # every probability row sums to 1, so the value gradients sum to the output gradients
        np.testing.assert_allclose(dV[0, 0].sum(axis=0), dO[0, 0].sum(axis=0), atol=1e-12)


# ----------------------------------------------------------------------------- block-sparse rule
def test_block_list_closed_form_and_totals():
    nb = 1024
    off, idx = block_lists(nb, window=8, stride=16, causal=True, rule="strided")
    lens = np.diff(off)
    expect = np.array([min(q, 8) + 1 + q // 16 for q in range(nb)])
    assert np.array_equal(lens, expect)
    assert int(off[-1]) == 41436 and int(lens.max()) == 72
    for q in range(nb):
        ks = idx[off[q]:off[q + 1]]
        assert np.all(np.diff(ks) > 0) and ks[-1] == q and ks[0] >= 0
    off2, _ = block_lists(nb, window=8, stride=16, causal=True, rule="fixed")
    assert int(off2[-1]) == 41884 and int(np.diff(off2).max()) == 73


def test_block_rule_direct_definition():
    nb, w, st = 70, 3, 5
    for q in range(nb):
        ks = allowed_blocks(q, nb, w, st, causal=True, rule="strided")
        direct = [k for k in range(nb) if k <= q and (q - k <= w or (q - k) % st == 0)]
        assert ks == direct
        ks = allowed_blocks(q, nb, w, st, causal=True, rule="fixed")
        assert ks == [k for k in range(nb) if k <= q and (q - k <= w or k % st == 0)]


def sparse_mask_direct(n, block, w, st, causal=True):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    qb, kb = i // block, j // block
    m = ((qb - kb >= 0) & (qb - kb <= w)) | ((qb - kb) % st == 0)
    if causal:
        m &= j <= i
    return m


def test_sparse_forward_matches_masked_dense():
    r = rng(15)
    block, w, st = 8, 2, 3
    n, d = 8 * 13 + 5, 8            # ragged last block
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    sp = dict(block=block, window=w, stride=st, rule="strided")
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=True, scale=0.4, sparse=sp)
    mask = sparse_mask_direct(n, block, w, st)
    O_ref, L_ref, _ = dense_reference(q, k, v, 0.4, mask)
    np.testing.assert_allclose(O[0, 0], O_ref, atol=1e-12)
    np.testing.assert_allclose(L[0, 0], L_ref, atol=1e-12)
    # the same mask through the explicit-list path and the list-to-mask helper
    off, idx = block_lists((n + block - 1) // block, w, st, causal=True)
    assert np.array_equal(key_mask_from_lists(n, block, off, idx, causal=True), mask)
    O2, L2 = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=True, scale=0.4,
                               sparse=dict(block=block, offsets=off, indices=idx))
    np.testing.assert_allclose(O2, O, atol=0)
    np.testing.assert_allclose(L2, L, atol=0)


def test_sparse_with_full_window_equals_causal_dense():
    r = rng(16)
    n, d, block = 96, 8, 16
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    sp = dict(block=block, window=n // block, stride=0, rule="strided")
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=True, scale=0.3, sparse=sp)
    O2, L2 = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=True, scale=0.3)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)


def test_empty_list_gives_zero_output_and_minus_inf_lse():
    r = rng(17)
    n, d, block = 32, 4, 8
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    off = np.array([0, 1, 1, 2, 3], dtype=np.int32)      # Q-block 1 lists nothing
    idx = np.array([0, 0, 3], dtype=np.int32)
    sp = dict(block=block, offsets=off, indices=idx)
    O, L = attention_forward(as_bhnd(q), as_bhnd(k), as_bhnd(v), causal=True, scale=0.5, sparse=sp)
    assert np.all(O[0, 0, 8:16] == 0) and np.all(np.isneginf(L[0, 0, 8:16]))
    assert np.all(np.isfinite(L[0, 0, :8])) and np.all(np.isfinite(L[0, 0, 16:]))
    dQ, dK, dV = attention_backward(as_bhnd(q), as_bhnd(k), as_bhnd(v), as_bhnd(q), causal=True,
                                    scale=0.5, sparse=sp)
    assert np.all(dQ[0, 0, 8:16] == 0)
    assert np.all(np.isfinite(dQ)) and np.all(np.isfinite(dK)) and np.all(np.isfinite(dV))


def test_sparse_backward_matches_autograd_with_mask():
    g = torch.Generator().manual_seed(18)
    n, d, block = 40, 8, 8
    Q, K, V, dO = (torch.randn(1, 1, n, d, generator=g, dtype=torch.float64) for _ in range(4))
    mask = torch.from_numpy(sparse_mask_direct(n, block, 1, 3))
    q, k, v = (t.clone().requires_grad_(True) for t in (Q, K, V))
    S = (0.5 * q @ k.transpose(-1, -2)).masked_fill(~mask, -math.inf)
    (torch.softmax(S, -1) @ v).backward(dO)
    sp = dict(block=block, window=1, stride=3, rule="strided")
    dQ, dK, dV = attention_backward(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), causal=True,
                                    scale=0.5, sparse=sp)
    np.testing.assert_allclose(dQ, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, v.grad.numpy(), atol=1e-12)


def test_keysets_sparse_rows_are_sorted_and_causal():
    ks = KeySets(1000, True, dict(block=128, window=2, stride=4, rule="strided"))
    for i in (0, 127, 128, 600, 999):
        J = ks.keys(i)
        assert np.all(np.diff(J) > 0) and J.max() == i
