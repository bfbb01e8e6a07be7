"""Oracle of gradient clipping by the global p-norm, in float64 numpy.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg use
this module; the GPU library does not.

What is computed follows the DMuon Training Guide:
  * "Gradient Clipping": dmuon.clip_grad_norm_(optimizer, max_norm) clips
    the dedicated (Muon) gradients only, after their reduce and before
    momentum and Newton-Schulz; the default strategy is global p-norm
    clipping over the Muon gradients.
  * "Fused CUDA clip for regular / Muon / AdamW": several gradient groups
    ("buckets") are clipped in one pass, each with its own norm, clip
    coefficient and in-place scaling.

The pages leave the formula to PyTorch's clip_grad_norm_, which the same
section uses for the other parameters; this oracle takes its semantics,
with the norm evaluated exactly (float64) whatever the gradient dtype:
  total_b = (sum over the bucket's gradients of sum |g|^p)^(1/p)
            (p = inf: the largest |g| of the bucket)
  coef_b  = min(1, max_norm_b / (total_b + 1e-6))
  g      <- g * coef_b, rounded once to the gradient's dtype;
a NaN or Inf in a bucket makes its total and coefficient non-finite and
propagates into that bucket's gradients (no error is raised).
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

from .muon import round_to_bf16

EPS = 1e-6


def grad_norm(grads: Sequence[np.ndarray], p: float) -> float:
    """Global p-norm of a list of arrays, in float64."""
    if not grads:
        return 0.0
    if math.isinf(p):
        return float(max(float(np.max(np.abs(g))) if g.size else 0.0 for g in grads))
    total = sum(float(np.sum(np.abs(np.asarray(g, dtype=np.float64)) ** p)) for g in grads)
    return total ** (1.0 / p)


def clip_coefficient(total: float, max_norm: float) -> float:
    """min(1, max_norm / (total + eps)); a NaN stays NaN."""
    coef = max_norm / (total + EPS)
    return 1.0 if coef >= 1.0 else coef


def clip_grad_norm(grads: Sequence[np.ndarray], buckets: Sequence[int], max_norms: Sequence[float],
                   p: float = 2.0) -> Tuple[List[np.ndarray], List[float], List[float]]:
    """Per-bucket clipping.  Returns (clipped gradients in float64, before
    rounding), the per-bucket totals and the per-bucket coefficients."""
    nb = len(max_norms)
    totals, coefs = [], []
    for b in range(nb):
        members = [np.asarray(g, dtype=np.float64) for g, k in zip(grads, buckets) if k == b]
        t = grad_norm(members, p)
        totals.append(t)
        coefs.append(clip_coefficient(t, max_norms[b]))
    out = [np.asarray(g, dtype=np.float64) * coefs[k] for g, k in zip(grads, buckets)]
    return out, totals, coefs


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """The value a gradient of ``dtype`` holds after one rounding."""
    if dtype == "bf16":
        return round_to_bf16(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
