"""Host-side model of where the stored-dS backward puts and finds each dS tile.

With a large enough workspace the dK/dV pass writes, for every step it takes (64 query rows
of one query head against its 128-key block), the step's dS into half `half` of the tile
numbered for its (key block, query block) pair, and the dQ pass reads, for every step it
takes (64 keys of a key block against its 128-row query block), both query halves of that
pair's tile. The numbering: dense non-causal kb * nqb + qb, dense causal
kb * nqb - kb (kb - 1) / 2 + qb - kb, block-sparse the pair's key-side list entry (the dQ
pass looks it up per query-side entry, as ds_pos_kernel does). This model walks both passes'
steps as the kernels order them (the dK/dV pass: the diagonal steps of each query head
first under causal masking, then the others) and checks, over dense, grouped, packed and
block-sparse cases (hand lists with out-of-range, above-diagonal and empty entries
included), that every write stays inside its region and that every tile half the dQ pass
needs (rows inside the sequence) was written, by the step of the same pair of blocks.
"""
import numpy as np
import pytest

import exact_block_sparse_amd as fa

BLK, STEP = 128, 64


def cdiv(a, b):
    return -(-a // b)


def clamp(x, nnz):
    return min(max(int(x), 0), nnz)


def dkdv_writes(L, N, G, hk, causal, kblk, lists=None):
    """{(query head, tile, half): (key block, query block, 64-row half of the query block)}
    written by the dK/dV workgroup of K/V head hk and key block kblk in a sequence of L rows
    (N: the longest one). The value comes from the rows the step computes (as the kernel
    derives them for its loads), the key from the store address."""
    out = {}
    if kblk * BLK >= L:
        return out
    nqbt = cdiv(N, BLK)
    nsteps = cdiv(L, STEP)
    t0 = 2 * kblk if causal else 0
    diag = 0
    if lists is None:
        per = nsteps - t0
        m_per = min(2, per) if causal else 0
    else:
        q_off, q_idx = lists
        nnz = len(q_idx)
        lo = clamp(q_off[kblk], nnz)
        hi = max(clamp(q_off[kblk + 1], nnz), lo)
        per = 2 * (hi - lo)
        m_per = 0
        if causal:
            e = lo
            while e < hi and q_idx[e] < kblk:
                e += 1
            if e < hi and q_idx[e] == kblk:
                m_per, diag = 2, e - lo
    u_per = per - m_per
    runs = [(True, gq) for gq in range(G)] + [(False, gq) for gq in range(G)]
    for masked, gq in runs:
        for j in range(m_per if masked else u_per):
            if lists is None:
                s = t0 + (j if masked else m_per + j)
                r0 = s * STEP                                   # the step's first row
                qb, half = s >> 1, s & 1                        # store address
                tile = kblk * nqbt - kblk * (kblk - 1) // 2 + qb - kblk if causal else kblk * nqbt + qb
            else:
                e = diag if masked else (j >> 1) + (1 if m_per and (j >> 1) >= diag else 0)
                r0 = int(q_idx[lo + e]) * BLK + (j & 1) * STEP  # the step's first row
                tile, half = lo + e, j & 1                      # store address
            key = (hk * G + gq, tile, half)
            assert key not in out, f"tile half {key} written twice"
            out[key] = (kblk, r0 // BLK, (r0 // STEP) & 1)
    return out


def positions(kv_off, kv_idx, q_off, q_idx, nb):
    """ds_pos_kernel: the key-side entry of every query-side entry, or -1."""
    nnz = len(kv_idx)
    pos = np.full(nnz, -1, np.int64)
    for qb in range(nb):
        lo = clamp(kv_off[qb], nnz)
        hi = max(clamp(kv_off[qb + 1], nnz), lo)
        for e in range(lo, hi):
            kb = int(kv_idx[e])
            if 0 <= kb < nb:
                a, z = clamp(q_off[kb], nnz), max(clamp(q_off[kb + 1], nnz), clamp(q_off[kb], nnz))
                hits = [i for i in range(a, z) if q_idx[i] == qb]
                pos[e] = hits[0] if hits else -1
    return pos


def dq_reads(L, N, h, causal, qb, lists=None, pos=None):
    """[(query head, tile, query half, key block)] the dQ workgroup of (h, qb) needs."""
    out = []
    q0 = qb * BLK
    if q0 >= L:
        return out
    nqbt = cdiv(N, BLK)
    qlast = min(q0 + BLK - 1, L - 1)
    halves = [qh for qh in (0, 1) if q0 + STEP * qh < L]
    if lists is None:
        nsteps = cdiv(L, STEP)
        if causal:
            nsteps = min(nsteps, qlast // STEP + 1)
        for t in range(nsteps):
            kb = t >> 1
            tile = kb * nqbt - kb * (kb - 1) // 2 + qb - kb if causal else kb * nqbt + qb
            out += [(h, tile, qh, kb) for qh in halves]
    else:
        kv_off, kv_idx = lists
        nnz = len(kv_idx)
        nkb = cdiv(L, BLK)
        lo = clamp(kv_off[qb], nnz)
        hi = max(clamp(kv_off[qb + 1], nnz), lo)
        for t in range(2 * (hi - lo)):
            e = lo + (t >> 1)
            kb, ps = int(kv_idx[e]), int(pos[e])
            if kb < 0 or kb >= nkb or (causal and kb > qb) or ps < 0 or ps >= nnz:
                continue
            kt0 = kb * BLK + STEP * (t & 1)
            if kt0 >= L or (causal and kt0 > qlast):
                continue
            out += [(h, ps, qh, kb) for qh in halves]
    return out


def check(lens, H, Hkv, causal, kv_lists=None):
    N = max(lens)
    G = H // Hkv
    nb = cdiv(N, BLK)
    if kv_lists is None:
        tiles = nb * (nb + 1) // 2 if causal else nb * nb
        q_lists = pos = None
    else:
        kv_off, kv_idx = (np.asarray(a, np.int32) for a in kv_lists)
        t_off, t_idx = fa.transpose_block_lists(kv_off, kv_idx, nb)
        q_lists = (t_off, t_idx)
        tiles = len(kv_idx)
        pos = positions(kv_off, kv_idx, t_off, t_idx, nb)
    needed = 0
    for b, L in enumerate(lens):
        written = {}
        for hk in range(Hkv):
            for kblk in range(nb):
                w = dkdv_writes(L, N, G, hk, causal, kblk, q_lists)
                assert not set(w) & set(written)
                written.update(w)
        for (hq, tile, half) in written:
            assert 0 <= hq < H and 0 <= tile < tiles and half in (0, 1)
        for h in range(H):
            for qb in range(nb):
                for hq, tile, qh, kb in dq_reads(L, N, h, causal, qb, None if kv_lists is None else
                                                 (kv_off, kv_idx), pos):
                    needed += 1
                    assert (hq, tile, qh) in written, f"sequence {b}: tile half {(hq, tile, qh)} never written"
                    assert written[(hq, tile, qh)] == (kb, qb, qh), "the tile half holds other blocks or rows"
    return needed


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens,H,Hkv", [((1,), 1, 1), ((64,), 2, 2), ((65,), 1, 1), ((128,), 2, 1),
                                        ((700,), 4, 2), ((1000,), 3, 1), ((37, 0, 263, 1, 399), 4, 2),
                                        ((300, 1, 129), 6, 2)])
def test_dense_layout(lens, H, Hkv, causal):
    assert check(lens, H, Hkv, causal) > 0 or max(lens) == 0


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N,window,stride,rule", [(1000, 1, 3, 0), (900, 2, 4, 0), (640, 1, 2, 1), (256, 0, 0, 0),
                                                  (128 * 37 + 5, 8, 16, 0)])
def test_block_sparse_layout_generated_lists(N, window, stride, rule, causal):
    nb = cdiv(N, BLK)
    off, idx = fa.make_block_lists(nb, window, stride, causal=causal, rule=("strided", "fixed")[rule])
    assert check((N,), 4, 2, causal, (off, idx)) > 0
    assert check((N, N // 2 + 3, 1), 2, 1, causal, (off, idx)) > 0


def test_block_sparse_layout_hand_lists():
    # query blocks naming key blocks above them (skipped under causal masking, and placed
    # before the diagonal entry in the key-side lists), an empty list, every block of block 4
    lists = [[0, 2], [0, 1, 3], [], [0, 3, 4], [0, 1, 2, 3, 4]]
    off = np.cumsum([0] + [len(l) for l in lists]).astype(np.int32)
    idx = np.array([k for l in lists for k in l], np.int32)
    for causal in (True, False):
        assert check((128 * 5 - 30,), 2, 1, causal, (off, idx)) > 0
        assert check((128 * 5 - 30, 200), 4, 4, causal, (off, idx)) > 0
