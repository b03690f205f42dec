"""Oracle: the block-sparse (Flash-MSA) key-block pattern, written from the pages.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module; only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` do.

Sources ("How Does Flash-MSA Sparse Attention Work", section "How Flash-MSA Sparse
Attention Works"): the sequence is cut into blocks; the mask is applied inside the
tile loop, per block or through a precomputed index list; the named patterns include
a local window of +-W positions and the fixed "strided" pattern of Child et al. (2019).

Reading taken here (the pages give no formula):
* granularity is the block (128 tokens for the 128K workload), so the pattern is a
  set of allowed K-blocks for every Q-block;
* with causal masking the window is the blocks [q - window, q] clipped at 0;
* "strided" (default): keep K-blocks k <= q with (q - k) divisible by ``stride``
  (Child-style strided attention counted back from the query block);
  "fixed" (alternative reading): keep K-blocks k <= q with k divisible by ``stride``;
* without causal masking the window is symmetric, [q - window, q + window], and the
  strided set extends both ways (|q - k| divisible by the stride / k divisible);
* the final list for a Q-block is the sorted union of the two sets, without repeats.
"""
from __future__ import annotations

import numpy as np


def allowed_blocks(q: int, n_blocks: int, window: int, stride: int, causal: bool = True,
                   rule: str = "strided") -> list[int]:
    """Sorted K-block indices that Q-block ``q`` may attend to."""
    if rule not in ("strided", "fixed"):
        raise ValueError(f"unknown rule {rule!r}")
    allowed = set()
    hi = q if causal else n_blocks - 1
    # local window
    for k in range(max(0, q - window), min(hi, q + window) + 1):
        allowed.add(k)
    # strided / fixed columns
    if stride > 0:
        for k in range(0, hi + 1):
            if rule == "strided":
                if abs(q - k) % stride == 0:
                    allowed.add(k)
            else:
                if k % stride == 0:
                    allowed.add(k)
    return sorted(allowed)


def block_lists(n_blocks: int, window: int, stride: int, causal: bool = True,
                rule: str = "strided"):
    """The pattern as per-Q-block sorted lists in CSR form: (offsets[n+1], indices[nnz]), int32."""
    offsets = [0]
    indices: list[int] = []
    for q in range(n_blocks):
        ks = allowed_blocks(q, n_blocks, window, stride, causal, rule)
        indices.extend(ks)
        offsets.append(len(indices))
    return np.asarray(offsets, dtype=np.int32), np.asarray(indices, dtype=np.int32)


def key_mask_from_lists(n: int, block: int, offsets, indices, causal: bool) -> np.ndarray:
    """Dense boolean (n, n) mask [query, key] allowed by block lists (and causality).

    Only for small n: it materialises the whole matrix. A key j is allowed for query i
    iff j's block is listed for i's block and, with causal masking, j <= i.
    """
    n_blocks = (n + block - 1) // block
    m = np.zeros((n, n), dtype=bool)
    for qb in range(n_blocks):
        r0, r1 = qb * block, min(n, (qb + 1) * block)
        for t in range(int(offsets[qb]), int(offsets[qb + 1])):
            kb = int(indices[t])
            m[r0:r1, kb * block:min(n, (kb + 1) * block)] = True
    if causal:
        m &= np.tril(np.ones((n, n), dtype=bool))
    return m


def transpose_lists(offsets, indices, n_blocks: int):
    """The same pattern seen from the key side, in CSR form: for every K-block, the
    ascending Q-blocks whose lists name it. The backward's dK/dV pass walks these
    (page 3's FAQ on training: the backward reuses the forward's tiling and masking).
    """
    off = np.asarray(offsets, dtype=np.int64)
    idx = np.asarray(indices, dtype=np.int64)
    per_key: list[list[int]] = [[] for _ in range(n_blocks)]
    for q in range(n_blocks):
        for t in range(int(off[q]), int(off[q + 1])):
            per_key[int(idx[t])].append(q)
    t_off = [0]
    t_idx: list[int] = []
    for k in range(n_blocks):
        t_idx.extend(sorted(per_key[k]))
        t_off.append(len(t_idx))
    return np.asarray(t_off, dtype=np.int32), np.asarray(t_idx, dtype=np.int32)
