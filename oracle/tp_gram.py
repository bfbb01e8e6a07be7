"""Oracle of Newton-Schulz on a tensor-parallel sharded matrix, in float64 numpy.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg use
this module; the GPU library does not.

What is computed follows the DMuon FAQ, "Does DMuon work with Tensor
Parallelism?": under tensor parallelism a dedicated matrix stays split into
shards across the TP ranks, and the Gram Newton-Schulz iteration needs only
Gram matrices to be summed across the shards (an all-reduce whose size is the
square of the unsplit dimension), never the shards themselves.  The
iteration itself is the one of the Training Guide's "Hyperparameter Guide"
(ns_steps, ns_backend), as in ``oracle.muon``.

Readings where the page is silent:
  * a matrix U is split along one dimension into k contiguous shards; the
    Gram matrices are formed over the other, unsplit, dimension d: with
    ``split = 1`` the shards are column blocks U_i (d x n_i) and
    X_i = U_i; with ``split = 0`` they are row blocks (n_i x d) and
    X_i = U_i^T;
  * the Frobenius norm that normalises the NS input is that of the whole U:
    a scalar summed over the shards (X0_i = X_i / (||U||_F + eps));
  * Gram form: R = sum_i X0_i X0_i^T (the all-reduce), then on every rank the
    same d x d iteration (P = aI + bA + cA^2, Q <- P Q, A <- P A P) and the
    local product O_i = Q X0_i;
  * standard form: every iteration sums A = sum_i X_i X_i^T (one all-reduce
    per iteration), forms B = bA + cA^2 and updates X_i <- a X_i + B X_i
    locally;
  * O_i is returned in the shard's own orientation.
In exact arithmetic both forms equal the unsharded iteration on the
concatenated matrix, for either split and any d (the push-through identity
p(U U^T) U = U p(U^T U) covers a Gram formed over the longer side).

Every function works on float64 arrays and on object arrays of
fractions.Fraction (exact checks).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

from .muon import _coeff_table


def orient(shards: Sequence[np.ndarray], split: int) -> List[np.ndarray]:
    """X_i: each shard with the unsplit dimension as its rows."""
    if split not in (0, 1):
        raise ValueError("split must be 0 (row blocks) or 1 (column blocks)")
    xs = [s if split == 1 else s.T for s in shards]
    d = xs[0].shape[0]
    if any(x.shape[0] != d for x in xs):
        raise ValueError("shards differ in the unsplit dimension")
    return xs


def global_frobenius_norm(xs: Sequence[np.ndarray]) -> float:
    """||U||_F from the shards: the per-shard sums of squares, summed."""
    return math.sqrt(sum(float(np.sum(np.asarray(x, dtype=np.float64) ** 2)) for x in xs))


def _eye(d: int, like: np.ndarray) -> np.ndarray:
    e = np.zeros((d, d), dtype=like.dtype)
    one = 1 if like.dtype == object else like.dtype.type(1)
    for i in range(d):
        e[i, i] = one
    return e


def gram_sum(xs: Sequence[np.ndarray]) -> np.ndarray:
    """sum_i X_i X_i^T: each rank's partial Gram matrix, then their sum."""
    partial = [x @ x.T for x in xs]
    total = partial[0]
    for p in partial[1:]:
        total = total + p
    return total


def gram_form_sharded(x0s: Sequence[np.ndarray], ns_steps: int = 5, coeffs=None) -> List[np.ndarray]:
    """Gram form on normalised shards: one Gram sum, the d x d iteration,
    then O_i = Q X0_i on each shard."""
    table = _coeff_table(ns_steps, coeffs)
    if not table:
        return list(x0s)
    A = gram_sum(x0s)
    I = _eye(A.shape[0], A)
    Q = None
    for k, (a, b, c) in enumerate(table):
        P = a * I + b * A + c * (A @ A)
        Q = P if Q is None else P @ Q
        if k + 1 < len(table):
            A = P @ A @ P
    return [Q @ x for x in x0s]


def direct_form_sharded(x0s: Sequence[np.ndarray], ns_steps: int = 5, coeffs=None) -> List[np.ndarray]:
    """Standard form on normalised shards: a Gram sum every iteration, the
    d x d polynomial B, and the local update of each shard."""
    xs = list(x0s)
    for a, b, c in _coeff_table(ns_steps, coeffs):
        A = gram_sum(xs)
        B = b * A + c * (A @ A)
        xs = [a * x + B @ x for x in xs]
    return xs


def orthogonalize_sharded(shards: Sequence[np.ndarray], split: int, ns_steps: int = 5,
                          backend: str = "gram", coeffs=None, eps: float = 1e-7) -> List[np.ndarray]:
    """O_i for every shard of one matrix, in the shards' own orientation."""
    xs = orient(shards, split)
    s = 1.0 / (global_frobenius_norm(xs) + eps)
    x0s = [x * s for x in xs]
    if backend == "gram":
        os_ = gram_form_sharded(x0s, ns_steps, coeffs)
    elif backend == "direct":
        os_ = direct_form_sharded(x0s, ns_steps, coeffs)
    else:
        raise ValueError(backend)
    return [o if split == 1 else o.T for o in os_]


def split_matrix(u: np.ndarray, split: int, sizes: Sequence[int]) -> List[np.ndarray]:
    """Cut U into contiguous shards of the given sizes: column blocks for
    split = 1, row blocks for split = 0."""
    axis = 1 if split == 1 else 0
    if sum(sizes) != u.shape[axis]:
        raise ValueError("shard sizes do not add up")
    edges = np.cumsum([0, *sizes])
    if axis == 1:
        return [u[:, edges[i]:edges[i + 1]] for i in range(len(sizes))]
    return [u[edges[i]:edges[i + 1], :] for i in range(len(sizes))]


def join_shards(parts: Sequence[np.ndarray], split: int) -> np.ndarray:
    return np.concatenate(list(parts), axis=1 if split == 1 else 0)
