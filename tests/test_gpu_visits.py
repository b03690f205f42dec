"""Visit log of the block-sparse forward (fa_attn_fwd_visits): every query block takes into
its softmax exactly the key tiles its list names, less those the kernels must skip.

"How Does Flash-MSA Sparse Attention Work", section "How Flash-MSA Sparse Attention Works":
a query block walks its index list and nothing else, and only listed blocks that the causal
mask leaves enter its online softmax. The expected log is derived here from the lists alone
(host logic, independent of the kernels and of the oracle): half `half` of entry e of query
block qb is taken iff the entry's key block is inside the sequence, not above qb under causal
masking, and its first key 128 * block + 64 * half is inside the sequence and (causal) not
after the query block's last row. The log must equal that bit for bit, and the outputs must
equal those of fa_attn_fwd bit for bit. Both sparse kernels are covered: the one loading
straight into LDS (bf16, head dimension 128) and the register-staged one (head dimension 64
and fp8), at small sizes with hand-made and generated lists and at the 128K workload.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

BLOCK = 128


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


def expected_visits(off, idx, lens, H, N, causal):
    """uint8 [B * H, nnz, 2]: 1 where the kernels must take the half-block into the softmax."""
    off = np.asarray(off, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    nnz = idx.size
    exp = np.zeros((len(lens) * H, nnz, 2), dtype=np.uint8)
    nqb = (N + BLOCK - 1) // BLOCK
    for b, L in enumerate(lens):
        nkb = (L + BLOCK - 1) // BLOCK
        for qb in range(nqb):
            if qb * BLOCK >= L:
                continue
            lo = min(max(int(off[qb]), 0), nnz)
            hi = min(max(int(off[qb + 1]), lo), nnz)
            qlast = min(qb * BLOCK + BLOCK - 1, L - 1)
            for e in range(lo, hi):
                kb = int(idx[e])
                if kb < 0 or kb >= nkb or (causal and kb > qb):
                    continue
                for half in (0, 1):
                    kt0 = kb * BLOCK + 64 * half
                    if kt0 < L and not (causal and kt0 > qlast):
                        exp[b * H:(b + 1) * H, e, half] = 1
    return exp


def check_log(fa, q, k, v, off, idx, lens, N, causal, **kw):
    o, lse, vis = fa.attn_fwd_visits(q, k, v, kv_offsets=off, kv_indices=idx, causal=causal, **kw)
    o2, lse2 = fa.attn_fwd(q, k, v, kv_offsets=off, kv_indices=idx, causal=causal, **kw)
    torch.cuda.synchronize()
    host = lambda a: a.cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a)
    exp = expected_visits(host(off), host(idx), lens, q.shape[1], N, causal)
    got = vis.cpu().numpy()
    assert got.shape == exp.shape
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{len(bad)} log entries differ, first (row, entry, half) {bad[:5].tolist()}"
    assert exp.sum() > 0
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "the logging call changed the outputs"
    return exp


def inputs(B, H, N, d, seed, H_kv=None, packed=None):
    w = W.small(B, H, N, d, seed=seed, H_kv=H_kv, seqlens=packed)
    return {n: t.to("cuda") for n, t in W.make_inputs(w).items()}


@pytest.mark.parametrize("B,H,N,d,causal,window,stride", [
    (2, 3, 700, 128, True, 1, 2),
    (1, 2, 1000, 64, True, 2, 3),
    (1, 2, 640, 128, False, 1, 2),
    (1, 4, 128 * 9 + 5, 128, True, 2, 4),
])
def test_visits_generated_lists(fa, B, H, N, d, causal, window, stride):
    x = inputs(B, H, N, d, seed=N + d)
    nb = (N + BLOCK - 1) // BLOCK
    off, idx = fa.make_block_lists(nb, window, stride, causal=causal)
    check_log(fa, x["q"], x["k"], x["v"], off, idx, [N] * B, N, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_visits_device_lists_with_skipped_entries(fa, d, causal):
    # Five query blocks over a sequence that ends 37 rows into block 4. Block 0: an entry
    # past the last key block and a negative one; block 1: nothing; block 2: an entry above
    # the diagonal; block 3: its diagonal and block 0; block 4 (ragged): all of 0..4, whose
    # second half is past the sequence end. The last offset lies past nnz (clamped).
    N = 128 * 4 + 37
    x = inputs(1, 2, N, d, seed=11)
    off = torch.tensor([0, 3, 3, 6, 8, 16], dtype=torch.int32, device="cuda")
    idx = torch.tensor([0, 7, -1, 0, 2, 3, 0, 3, 0, 1, 2, 3, 4], dtype=torch.int32, device="cuda")
    exp = check_log(fa, x["q"], x["k"], x["v"], off, idx, [N], N, causal)
    assert exp[:, 1].sum() == 0 and exp[:, 2].sum() == 0       # out of range / negative
    assert exp[:, 5].sum() == (0 if causal else 2 * 2)         # key block 3 above query block 2
    assert exp[0, 12].tolist() == [1, 0]                       # second half past the end


def test_visits_packed_grouped(fa):
    lens = [300, 129, 700]
    N = max(lens)
    x = inputs(len(lens), 4, N, 128, seed=5, H_kv=2, packed=lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    nb = (N + BLOCK - 1) // BLOCK
    off, idx = fa.make_block_lists(nb, 1, 2, causal=True)
    check_log(fa, x["q"], x["k"], x["v"], off, idx, lens, N, True, cu_seqlens=cu, max_seqlen=N)


def test_visits_fp8(fa):
    w = W.small(1, 2, 800, 128, seed=6, dtype="fp8_e4m3")
    x = W.make_inputs(w)
    q, k, v = (x[n].to("cuda") for n in "qkv")
    nb = (800 + BLOCK - 1) // BLOCK
    off, idx = fa.make_block_lists(nb, 1, 3, causal=True)
    check_log(fa, q, k, v, off, idx, [800], 800, True, q_descale=x["q_descale"], k_descale=x["k_descale"],
              v_descale=x["v_descale"])


def test_visits_sparse_workload_full_size(fa):
    w = W.WORKLOADS["sparse_h16_n128k"]
    x = {n: t.to("cuda") for n, t in W.make_inputs(w).items()}
    nb = (w.N + BLOCK - 1) // BLOCK
    off, idx = fa.make_block_lists(nb, w.sparse["window"], w.sparse["stride"], causal=w.causal,
                                   rule=w.sparse["rule"])
    exp = check_log(fa, x["q"], x["k"], x["v"], off, idx, [w.N], w.N, w.causal, scale=w.scale)
    # every listed entry of this pattern is in range and at or below the diagonal
    assert exp.sum() == w.H * 2 * len(idx)
