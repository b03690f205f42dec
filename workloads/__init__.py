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

Drawing procedure (the pages name no RNG): a CPU ``torch.Generator`` seeded with the
workload's seed draws Q, K, V and then dO, in that order, each as float32
``randn`` over the *physical* shape (so a (B,N,H,d) workload is laid out that way in
memory), multiplied by sigma and rounded to bfloat16 (round-to-nearest-even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

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
    direction: str = "fwd"        # "fwd", "sparse_fwd" or "bwd"
    sparse: dict | None = field(default=None, hash=False)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32: the exact value the GPU receives."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    def describe(self) -> str:
        s = (f"B={self.B} H={self.H} N={self.N} d={self.d} "
             f"{'causal' if self.causal else 'non-causal'} layout={self.layout} sigma={self.sigma}")
        if self.sparse:
            s += (f" block={self.sparse['block']} window=±{self.sparse['window']} blocks"
                  f" stride={self.sparse['stride']} ({self.sparse['rule']})")
        return f"{self.direction} {s}"


# The block-sparse pattern: causal, restricted to a local window of 8 blocks and a
# strided set keeping every 16th K-block counted back from the query block.
SPARSE_128K = dict(block=128, window=8, stride=16, rule="strided")

WORKLOADS = {
    "dense_n512_d64": Workload("dense_n512_d64", 1, 1, 512, 64, False, "bhnd", 1.0, 1, "fwd"),
    "causal_b4h32_n4k_bnhd": Workload("causal_b4h32_n4k_bnhd", 4, 32, 4096, 128, True, "bnhd", 1.0, 2, "fwd"),
    "causal_h32_n32k": Workload("causal_h32_n32k", 1, 32, 32768, 128, True, "bhnd", 0.5, 3, "fwd"),
    "sparse_h16_n128k": Workload("sparse_h16_n128k", 1, 16, 131072, 128, True, "bhnd", 1.0, 4,
                                 "sparse_fwd", SPARSE_128K),
    "bwd_b2h32_n8k": Workload("bwd_b2h32_n8k", 2, 32, 8192, 128, True, "bhnd", 1.0, 5, "bwd"),
}
ORDER = list(WORKLOADS)


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
    """Q, K, V (and dO for backward workloads) as bf16 CPU tensors, logical (B,H,N,d) views."""
    if with_grad is None:
        with_grad = w.direction == "bwd"
    ts = draw(physical_shape(w), w.seed, w.sigma, 4 if with_grad else 3)
    ts = [to_logical(t, w.layout) for t in ts]
    names = ["q", "k", "v", "do"]
    return dict(zip(names, ts))


def small(B=1, H=1, N=256, d=64, causal=False, layout="bhnd", sigma=1.0, seed=0,
          direction="fwd", sparse=None) -> Workload:
    """An ad-hoc small workload for tests (same drawing procedure)."""
    return Workload(f"small_b{B}h{H}n{N}d{d}", B, H, N, d, causal, layout, sigma, seed, direction, sparse)
