"""Seeded synthetic workloads shared by the oracle tests, the GPU parity tests and the bench.

This module holds only shapes and random draws. It contains none of the attention
arithmetic: neither the oracle nor the HIP path puts any of its own logic here.

The five workloads follow the benchmark shapes used for this attention path: a small
dense head (N=512, d=64), a 7B-like causal layer (32 heads, head dim 128, the shape
of the H100 latency table in "Flash MSA Attention Kernel Implementation: A Practical
Guide for Production AI", section "Measuring What Matters: Performance Benchmarks"),
the 32K-token long-context case of that page's section "Why Standard Attention
Broke", a 128K-token block-sparse case (the 128K context of "How Does Flash-MSA
Sparse Attention Work", section "Flash-MSA vs Standard Attention Benchmark") and a
causal backward. The pages measure on private models and data; seeded Gaussian
tensors of these shapes stand in for them.

Five more cover the extensions: grouped K/V heads at the 32K shape and at the
backward's shape (32 query heads over 8 K/V heads, the replication of the first page's
GQA FAQ), a packed batch of variable-length sequences forward and backward (the first
page's request batching in its production pipeline; the pages give no length mix, so 16 lengths are drawn
uniformly from [256, 8192] with a seeded numpy generator), the backward of the
128K block-sparse case (the third page's FAQ on training), and the 32K case with fp8
(e4m3) inputs (the second page's FAQ on FP16 vs FP8): Q, K, V are drawn as for the bf16
case, then each tensor gets the usual per-tensor scaling, descale = amax / 448, and is
stored as e4m3 codes of x / descale (torch's round-to-nearest-even conversion).

Drawing procedure (the pages name no RNG): a CPU ``torch.Generator`` seeded with the
workload's seed draws Q, K, V and then dO, in that order, each as float32
``randn`` over the *physical* shape (so a (B,N,H,d) workload is laid out that way in
memory), multiplied by sigma and rounded to bfloat16 (round-to-nearest-even).
K and V have H_kv heads when the workload groups them. Packed workloads draw
[total, H, d] (and [total, H_kv, d]) tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    key: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    layout: str = "bhnd"          # physical layout: "bhnd" or "bnhd"
    sigma: float = 1.0
    seed: int = 0
    direction: str = "fwd"        # "fwd", "sparse_fwd", "bwd" or "sparse_bwd"
    sparse: dict | None = field(default=None, hash=False)
    H_kv: int | None = None       # key/value heads (None: H)
    seqlens: tuple | None = None  # packed variable-length sequences (N is then the longest)
    dtype: str = "bf16"           # "bf16" or "fp8_e4m3" (forward only)

    @property
    def hkv(self) -> int:
        return self.H if self.H_kv is None else self.H_kv

    @property
    def packed(self) -> bool:
        return self.seqlens is not None

    @property
    def total(self) -> int:
        return int(sum(self.seqlens)) if self.packed else self.B * self.N

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32: the exact value the GPU receives."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    def describe(self) -> str:
        heads = f"H={self.H}" + (f" H_kv={self.hkv}" if self.hkv != self.H else "")
        if self.dtype != "bf16":
            heads = f"{self.dtype} {heads}"
        if self.packed:
            s = (f"B={self.B} {heads} packed total={self.total} max_len={self.N} d={self.d} "
                 f"{'causal' if self.causal else 'non-causal'} sigma={self.sigma}")
        else:
            s = (f"B={self.B} {heads} N={self.N} d={self.d} "
                 f"{'causal' if self.causal else 'non-causal'} layout={self.layout} sigma={self.sigma}")
        if self.sparse:
            s += (f" block={self.sparse['block']} window=±{self.sparse['window']} blocks"
                  f" stride={self.sparse['stride']} ({self.sparse['rule']})")
        return f"{self.direction} {s}"


# The block-sparse pattern: causal, restricted to a local window of 8 blocks and a
# strided set keeping every 16th K-block counted back from the query block.
SPARSE_128K = dict(block=128, window=8, stride=16, rule="strided")

def length_mix(count: int, lo: int, hi: int, seed: int) -> tuple:
    """``count`` sequence lengths drawn uniformly from [lo, hi] by a seeded numpy generator."""
    return tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, size=count))


VARLEN_MIX = length_mix(16, 256, 8192, 7)

WORKLOADS = {
    "dense_n512_d64": Workload("dense_n512_d64", 1, 1, 512, 64, False, "bhnd", 1.0, 1, "fwd"),
    "causal_b4h32_n4k_bnhd": Workload("causal_b4h32_n4k_bnhd", 4, 32, 4096, 128, True, "bnhd", 1.0, 2, "fwd"),
    "causal_h32_n32k": Workload("causal_h32_n32k", 1, 32, 32768, 128, True, "bhnd", 0.5, 3, "fwd"),
    "sparse_h16_n128k": Workload("sparse_h16_n128k", 1, 16, 131072, 128, True, "bhnd", 1.0, 4,
                                 "sparse_fwd", SPARSE_128K),
    "bwd_b2h32_n8k": Workload("bwd_b2h32_n8k", 2, 32, 8192, 128, True, "bhnd", 1.0, 5, "bwd"),
    # extensions: grouped heads, packed variable-length sequences, block-sparse backward
    "gqa_h32kv8_n32k": Workload("gqa_h32kv8_n32k", 1, 32, 32768, 128, True, "bhnd", 0.5, 6, "fwd", H_kv=8),
    "gqa_bwd_b2h32kv8_n8k": Workload("gqa_bwd_b2h32kv8_n8k", 2, 32, 8192, 128, True, "bhnd", 1.0, 8, "bwd",
                                     H_kv=8),
    "varlen_h32_b16": Workload("varlen_h32_b16", len(VARLEN_MIX), 32, max(VARLEN_MIX), 128, True, "packed", 1.0,
                               7, "fwd", seqlens=VARLEN_MIX),
    "varlen_bwd_h32_b16": Workload("varlen_bwd_h32_b16", len(VARLEN_MIX), 32, max(VARLEN_MIX), 128, True,
                                   "packed", 1.0, 9, "bwd", seqlens=VARLEN_MIX),
    "sparse_bwd_h16_n128k": Workload("sparse_bwd_h16_n128k", 1, 16, 131072, 128, True, "bhnd", 1.0, 4,
                                     "sparse_bwd", SPARSE_128K),
    "fp8_h32_n32k": Workload("fp8_h32_n32k", 1, 32, 32768, 128, True, "bhnd", 0.5, 10, "fwd", dtype="fp8_e4m3"),
}

FP8_MAX = 448.0   # largest finite e4m3 value


def to_fp8(x: torch.Tensor):
    """(e4m3 codes, descale) of an fp32 tensor with per-tensor scaling descale = amax / 448."""
    amax = float(x.abs().max())
    descale = float(torch.tensor(amax / FP8_MAX if amax > 0 else 1.0, dtype=torch.float32))
    return (x / descale).to(torch.float8_e4m3fn), descale
ORDER = list(WORKLOADS)
# the five benchmark configurations (the rest are the extensions)
BENCHMARK_CONFIGS = ("dense_n512_d64", "causal_b4h32_n4k_bnhd", "causal_h32_n32k", "sparse_h16_n128k", "bwd_b2h32_n8k")


def physical_shape(w: Workload) -> tuple:
    if w.layout == "bhnd":
        return (w.B, w.H, w.N, w.d)
    if w.layout == "bnhd":
        return (w.B, w.N, w.H, w.d)
    raise ValueError(w.layout)


def to_logical(t: torch.Tensor, layout: str) -> torch.Tensor:
    """View a physical tensor as logical (B, H, N, d) without copying."""
    return t if layout == "bhnd" else t.permute(0, 2, 1, 3)


def draw(shape, seed: int, sigma: float = 1.0, count: int = 3, dtype=torch.bfloat16):
    """``count`` tensors of ``shape`` drawn in order from one seeded CPU generator."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for _ in range(count):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        out.append(x.to(dtype))
    return out


def make_inputs(w: Workload, with_grad: bool | None = None):
    """Q, K, V (and dO for backward workloads) as bf16 CPU tensors: logical (B,H,N,d) views
    (K, V with H_kv heads), or packed [total, heads, d] tensors for packed workloads."""
    if with_grad is None:
        with_grad = w.direction in ("bwd", "sparse_bwd")
    if w.packed:
        qs, kvs = (w.total, w.H, w.d), (w.total, w.hkv, w.d)
    else:
        qs = physical_shape(w)
        kvs = physical_shape(Workload(w.key, w.B, w.hkv, w.N, w.d, w.causal, w.layout))
    if w.dtype == "fp8_e4m3":
        raw = draw(qs, w.seed, w.sigma, 3, dtype=torch.float32) if qs == kvs else None
        if raw is None:
            g = torch.Generator(device="cpu").manual_seed(int(w.seed))
            raw = [torch.randn(s, generator=g, dtype=torch.float32) * w.sigma for s in (qs, kvs, kvs)]
        out = {}
        for n, x in zip("qkv", raw):
            code, ds = to_fp8(x)
            out[n] = code if w.packed else to_logical(code, w.layout)
            out[n + "_descale"] = ds
        return out
    if qs == kvs:
        ts = draw(qs, w.seed, w.sigma, 4 if with_grad else 3)
    else:
        g = torch.Generator(device="cpu").manual_seed(int(w.seed))
        ts = []
        for shape in (qs, kvs, kvs, qs)[: 4 if with_grad else 3]:
            x = torch.randn(shape, generator=g, dtype=torch.float32)
            if w.sigma != 1.0:
                x.mul_(w.sigma)
            ts.append(x.to(torch.bfloat16))
    if not w.packed:
        ts = [to_logical(t, w.layout) for t in ts]
    names = ["q", "k", "v", "do"]
    return dict(zip(names, ts))


def small(B=1, H=1, N=256, d=64, causal=False, layout="bhnd", sigma=1.0, seed=0,
          direction="fwd", sparse=None, H_kv=None, seqlens=None, dtype="bf16") -> Workload:
    """An ad-hoc small workload for tests (same drawing procedure)."""
    if seqlens is not None:
        seqlens = tuple(int(x) for x in seqlens)
        B, N, layout = len(seqlens), max(seqlens) if seqlens else 0, "packed"
    return Workload(f"small_b{B}h{H}n{N}d{d}", B, H, N, d, causal, layout, sigma, seed, direction, sparse,
                    H_kv, seqlens, dtype)
