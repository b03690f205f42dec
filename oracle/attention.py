"""Oracle: plain fp64 CPU attention, one query row at a time.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module; only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` do.
It shares no code with the HIP library and imports nothing from it.

What it computes. The tiled method on the pages is exact: the online softmax is the
same function as the ordinary softmax ("Flash MSA Attention Kernel Implementation: A
Practical Guide for Production AI", FAQ on numeric precision; "How to Use Flash MSA
Kernels for Long Context", section "Why Most People Get Long-Context Wrong"). So this
oracle is the plain definition of attention, softmax(Q K^T * scale + mask) V
(page 1, section "Why Standard Attention Broke"), written out per query row i:

* the allowed key set J_i: all keys, minus keys j > i under causal masking
  (page 1, section "Code: A Complete Flash Attention Forward Kernel in CUDA": a key
  position past the query position is masked), minus keys whose block is not listed
  for i's block in block-sparse mode (page 3, section "How Flash-MSA Sparse Attention
  Works"). Masked keys are left out of the sum, which is what a -inf score does
  (page 1, section "Optimization Tricks That Actually Matter", and its NaN FAQ: -inf,
  not 0);
* s_j = scale * (q_i . k_j) for j in J_i; m = max s; e_j = exp(s_j - m); l = sum e;
  P_ij = e_j / l; O_i = sum_j P_ij v_j; LSE_i = m + ln l (natural log; page 1's
  forward kernel keeps the max and the sum per query for the backward, page 3's sketch
  keeps their log-sum-exp);
* an empty J_i (only possible with an empty block list) gives O_i = 0, LSE_i = -inf.

Backward (page 1, section "The Backward Pass: The Real Beast"): P is recomputed from
the row statistics; dP_ij = dO_i . v_j; D_i = sum_j P_ij dP_ij; dS_ij = P_ij (dP_ij - D_i);
and, by the chain rule through S = scale * Q K^T (the page's sketch leaves the scale
out of the dQ and dK lines), dQ_i = scale * sum_j dS_ij k_j, dK_j += scale * dS_ij q_i,
dV_j += P_ij dO_i. The backward uses this module's own fp64 forward.

Grouped key/value heads (page 1, FAQ on grouped-query and multi-query attention: the
tiling is unchanged, the K and V heads are replicated over fewer copies): K and V may
have H_kv heads with H divisible by H_kv; query head h reads key/value head
h // (H / H_kv), so consecutive query heads share one K/V head (the replication reading
taken here; H_kv = 1 is multi-query attention). In the backward a K/V head's gradient is
the sum of the gradients its query heads send it, as the chain rule gives for a shared
input.

Variable-length batches (page 1, section "The Production Pipeline: From Kernel to Service",
on request batching: padding tokens are masked out of every tile's softmax; "How to Use
Flash MSA Kernels for Long Context", FAQ on flash-batch inference, which points to a
variable-length entry point): sequences of
different lengths are packed one after another along the token axis, sequence b being
rows cu_seqlens[b] .. cu_seqlens[b+1] - 1; each sequence attends only to itself, exactly
as if it were run alone. ``attention_forward_varlen`` and ``attention_backward_varlen``
do just that, sequence by sequence.

All arithmetic is float64. Inputs may be bf16 torch tensors or numpy arrays; they are
upcast exactly. Arrays are logical (B, H, N, d); K and V are (B, H_kv, N, d).
"""
from __future__ import annotations

import math

import numpy as np

from .block_rule import allowed_blocks


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


class KeySets:
    """Allowed key indices J_i for each query row i of one head.

    ``sparse`` is either None (dense), a rule dict {block, window, stride, rule} from
    which the oracle builds its own block sets, or explicit block lists
    {block, offsets, indices} given as test inputs.
    """

    def __init__(self, n: int, causal: bool, sparse: dict | None = None):
        self.n = n
        self.causal = causal
        self.sparse = sparse
        self._blocks = None
        if sparse is not None:
            self.block = int(sparse["block"])
            nb = (n + self.block - 1) // self.block
            if "offsets" in sparse:
                off = np.asarray(sparse["offsets"]).astype(np.int64)
                idx = np.asarray(sparse["indices"]).astype(np.int64)
                self._blocks = [sorted(set(int(k) for k in idx[off[q]:off[q + 1]]))
                                for q in range(nb)]
            else:
                self._blocks = [allowed_blocks(q, nb, int(sparse["window"]), int(sparse["stride"]),
                                               causal, sparse.get("rule", "strided"))
                                for q in range(nb)]
        self._cache_q = None
        self._cache_keys = None

    def keys(self, i: int) -> np.ndarray:
        n = self.n
        hi = i + 1 if self.causal else n
        if self._blocks is None:
            return np.arange(0, hi, dtype=np.int64)
        qb = i // self.block
        if self._cache_q != qb:
            parts = [np.arange(kb * self.block, min(n, (kb + 1) * self.block), dtype=np.int64)
                     for kb in self._blocks[qb] if 0 <= kb * self.block < n]
            self._cache_keys = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
            self._cache_q = qb
        ks = self._cache_keys
        if self.causal:
            ks = ks[ks < hi]
        return ks


def row_scores(q: np.ndarray, K: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s_j = scale * (q . k_j) for the allowed keys."""
    return scale * (K[keys] @ q)


def row_probabilities(s: np.ndarray):
    """Softmax of one score row: returns (P, m, l). Empty rows give (empty, -inf, 0)."""
    if s.size == 0:
        return s.copy(), -math.inf, 0.0
    m = float(np.max(s))
    e = np.exp(s - m)
    l = float(np.sum(e))
    return e / l, m, l


def forward_row(q, K, V, keys, scale):
    """(O_i, LSE_i) for one query row, as defined in the module docstring."""
    s = row_scores(q, K, keys, scale)
    p, m, l = row_probabilities(s)
    if keys.size == 0:
        return np.zeros(V.shape[1], dtype=np.float64), -math.inf
    return p @ V[keys], m + math.log(l)


def kv_head(h: int, H: int, H_kv: int) -> int:
    """The key/value head query head ``h`` reads: h // (H / H_kv)."""
    if H_kv <= 0 or H % H_kv:
        raise ValueError(f"H={H} is not a multiple of H_kv={H_kv}")
    return h // (H // H_kv)


def attention_forward(Q, K, V, *, causal: bool, scale: float, sparse: dict | None = None,
                      rows=None, heads=None):
    """O (B,H,N,d) and LSE (B,H,N) in fp64. K and V may have H_kv heads (grouped).

    ``rows``: optional iterable of query rows to compute (others are left NaN).
    ``heads``: optional iterable of (b, h) pairs to compute (others are left NaN).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    scale = float(scale)
    O = np.full((B, H, N, V.shape[-1]), np.nan)
    LSE = np.full((B, H, N), np.nan)
    row_list = range(N) if rows is None else sorted(set(int(r) for r in rows))
    head_list = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    ks = KeySets(N, causal, sparse)
    for (b, h) in head_list:
        g = kv_head(h, H, H_kv)
        Kb, Vb, Qb = K[b, g], V[b, g], Q[b, h]
        for i in row_list:
            O[b, h, i], LSE[b, h, i] = forward_row(Qb[i], Kb, Vb, ks.keys(i), scale)
    return O, LSE


def attention_backward(Q, K, V, dO, *, causal: bool, scale: float, sparse: dict | None = None,
                       heads=None, return_forward: bool = False):
    """dQ (B,H,N,d), dK and dV (B,H_kv,N,d) in fp64, from the oracle's own forward.

    With grouped heads, dK and dV of a K/V head sum over the query heads that read it.
    ``heads`` limits the query heads computed; K/V heads none of them reads stay NaN.
    """
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    scale = float(scale)
    dQ = np.full(Q.shape, np.nan)
    dK = np.full(K.shape, np.nan)
    dV = np.full(V.shape, np.nan)
    O = np.full(Q.shape[:3] + (V.shape[-1],), np.nan)
    LSE = np.full((B, H, N), np.nan)
    head_list = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for (b, h) in head_list:
        g = kv_head(h, H, H_kv)
        dK[b, g] = 0.0
        dV[b, g] = 0.0
    ks = KeySets(N, causal, sparse)
    for (b, h) in head_list:
        g = kv_head(h, H, H_kv)
        Qb, Kb, Vb, dOb = Q[b, h], K[b, g], V[b, g], dO[b, h]
        dKb = dK[b, g]   # views: the group's query heads add into the same K/V head
        dVb = dV[b, g]
        for i in range(N):
            keys = ks.keys(i)
            s = row_scores(Qb[i], Kb, keys, scale)
            p, m, l = row_probabilities(s)
            if keys.size == 0:
                dQ[b, h, i] = 0.0
                O[b, h, i] = 0.0
                LSE[b, h, i] = -math.inf
                continue
            O[b, h, i] = p @ Vb[keys]
            LSE[b, h, i] = m + math.log(l)
            dp = Vb[keys] @ dOb[i]                 # dP_ij = dO_i . v_j
            Di = float(p @ dp)                      # D_i = sum_j P_ij dP_ij
            ds = p * (dp - Di)                      # dS_ij = P_ij (dP_ij - D_i)
            dQ[b, h, i] = scale * (ds @ Kb[keys])   # dQ_i = scale * sum_j dS_ij k_j
            dKb[keys] += scale * np.outer(ds, Qb[i])  # dK_j += scale * dS_ij q_i
            dVb[keys] += np.outer(p, dOb[i])          # dV_j += P_ij dO_i
    if return_forward:
        return dQ, dK, dV, O, LSE
    return dQ, dK, dV


def backward_rows_dq(Q, K, V, dO, *, causal, scale, sparse=None, b=0, h=0, rows=()):
    """dQ for selected query rows of one head (each row needs only its own keys)."""
    g = kv_head(h, Q.shape[1], K.shape[1])
    Q, K, V, dO = _f64(Q[b, h]), _f64(K[b, g]), _f64(V[b, g]), _f64(dO[b, h])
    N = Q.shape[0]
    ks = KeySets(N, causal, sparse)
    out = {}
    for i in rows:
        keys = ks.keys(int(i))
        s = row_scores(Q[i], K, keys, scale)
        p, _, _ = row_probabilities(s)
        if keys.size == 0:
            out[int(i)] = np.zeros(Q.shape[1])
            continue
        dp = V[keys] @ dO[i]
        ds = p * (dp - float(p @ dp))
        out[int(i)] = scale * (ds @ K[keys])
    return out


def _segments(cu_seqlens, total: int):
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    if cu.size < 1 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at the token count and not decrease")
    return [(int(cu[b]), int(cu[b + 1])) for b in range(cu.size - 1)]


def attention_forward_varlen(Q, K, V, cu_seqlens, *, causal: bool, scale: float,
                             sparse: dict | None = None, rows=None):
    """Packed variable-length forward: Q (T,H,d), K and V (T,H_kv,d) -> O (T,H,d), LSE (H,T).

    Sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1 and attends only to itself (causal
    positions and block numbers count from its own first row). ``rows``: optional packed
    row indices to compute (others left NaN).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    T, H, d = Q.shape
    O = np.full((T, H, V.shape[-1]), np.nan)
    LSE = np.full((H, T), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    for (s, e) in _segments(cu_seqlens, T):
        if e == s:
            continue
        local = None if want is None else [r - s for r in sorted(want) if s <= r < e]
        if local is not None and not local:
            continue
        q = Q[s:e].transpose(1, 0, 2)[None]
        k = K[s:e].transpose(1, 0, 2)[None]
        v = V[s:e].transpose(1, 0, 2)[None]
        o, lse = attention_forward(q, k, v, causal=causal, scale=scale, sparse=sparse, rows=local)
        O[s:e] = o[0].transpose(1, 0, 2)
        LSE[:, s:e] = lse[0]
    return O, LSE


def attention_backward_varlen(Q, K, V, dO, cu_seqlens, *, causal: bool, scale: float,
                              sparse: dict | None = None, return_forward: bool = False):
    """Packed variable-length backward: dQ (T,H,d), dK and dV (T,H_kv,d), per sequence."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    T, H, d = Q.shape
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    O = np.zeros((T, H, V.shape[-1]))
    LSE = np.full((H, T), -math.inf)
    for (s, e) in _segments(cu_seqlens, T):
        if e == s:
            continue
        tr = lambda x: x[s:e].transpose(1, 0, 2)[None]
        dq, dk, dv, o, lse = attention_backward(tr(Q), tr(K), tr(V), tr(dO), causal=causal, scale=scale,
                                                sparse=sparse, return_forward=True)
        dQ[s:e] = dq[0].transpose(1, 0, 2)
        dK[s:e] = dk[0].transpose(1, 0, 2)
        dV[s:e] = dv[0].transpose(1, 0, 2)
        O[s:e] = o[0].transpose(1, 0, 2)
        LSE[:, s:e] = lse[0]
    if return_forward:
        return dQ, dK, dV, O, LSE
    return dQ, dK, dV


def backward_keys_dkdv(Q, K, V, dO, *, causal: bool, scale: float, sparse: dict | None = None, b: int = 0,
                       h_kv: int = 0, keys=(), rows=None):
    """dK and dV of selected keys of K/V head ``h_kv`` (summed over the query heads that read
    it), for checks at sizes where the whole backward is too slow.

    Every query row i that may see a selected key contributes scale * dS_ij q_i to dK_j and
    P_ij dO_i to dV_j; P_ij and D_i need i's whole row. ``rows``: the query rows to visit
    (default all); rows that cannot see any selected key add nothing, so a superset is fine.
    Returns {key: (dK_j, dV_j)}.
    """
    B, H, N, d = Q.shape
    H_kv = K.shape[1]
    G = H // H_kv
    if kv_head(0, H, H_kv) != 0:   # validates the grouping
        raise ValueError("bad head grouping")
    Kb, Vb = _f64(K[b, h_kv]), _f64(V[b, h_kv])
    want = sorted(set(int(j) for j in keys))
    acc = {j: (np.zeros(K.shape[-1]), np.zeros(V.shape[-1])) for j in want}
    ks = KeySets(N, causal, sparse)
    row_list = range(N) if rows is None else sorted(set(int(r) for r in rows))
    for h in range(h_kv * G, (h_kv + 1) * G):
        Qh, dOh = _f64(Q[b, h]), _f64(dO[b, h])
        for i in row_list:
            J = ks.keys(i)
            hit = np.intersect1d(J, want, assume_unique=True)
            if hit.size == 0:
                continue
            s = row_scores(Qh[i], Kb, J, scale)
            p, _, _ = row_probabilities(s)
            dp = Vb[J] @ dOh[i]
            Di = float(p @ dp)
            pos = np.searchsorted(J, hit)
            for j, t in zip(hit, pos):
                ds = p[t] * (dp[t] - Di)
                acc[int(j)][0][:] += scale * ds * Qh[i]
                acc[int(j)][1][:] += p[t] * dOh[i]
    return acc
