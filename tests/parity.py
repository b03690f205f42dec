"""Comparison helpers for the GPU parity tests (HIP path vs the fp64 oracle).

Tolerances (max-abs, GPU output upcast to fp64 vs oracle fp64):
    O, dQ, dK, dV : 2e-2       LSE : 1e-3
Block lists must match exactly.
"""
from __future__ import annotations

import math

import numpy as np
import torch

TOL_OUT = 2e-2
TOL_LSE = 1e-3


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def stats(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(got - ref))
    fin = np.isfinite(ref)
    denom = np.maximum(np.abs(ref), 1e-6)
    return dict(
        max_abs=float(np.max(diff)) if diff.size else 0.0,
        mean_abs=float(np.mean(diff)) if diff.size else 0.0,
        max_ref=float(np.max(np.abs(ref[fin]))) if fin.any() else 0.0,
        max_rel=float(np.max((diff / denom)[fin])) if fin.any() else 0.0,
        n=int(diff.size),
    )


def assert_close(name: str, got, ref, tol: float, report: dict | None = None) -> dict:
    got = f64(got)
    ref = f64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU output"
    s = stats(got, ref)
    if report is not None:
        report[name] = s
    assert s["max_abs"] <= tol, f"{name}: max-abs error {s['max_abs']:.3e} > {tol:.1e} ({s})"
    return s


def assert_finite(name: str, t: torch.Tensor, allow_neg_inf: bool = False) -> None:
    x = t.detach().float()
    if allow_neg_inf:
        x = torch.where(torch.isneginf(x), torch.zeros_like(x), x)
    assert bool(torch.isfinite(x).all()), f"{name} has NaN/Inf"


def sample_rows(n: int, block: int, rng: np.random.Generator, extra: int = 32) -> np.ndarray:
    """First and last row of every block plus `extra` random rows (sorted, unique)."""
    rows = set()
    for b0 in range(0, n, block):
        rows.add(b0)
        rows.add(min(n, b0 + block) - 1)
    rows.update(int(r) for r in rng.integers(0, n, size=extra))
    return np.array(sorted(rows))


def scale_for(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))
