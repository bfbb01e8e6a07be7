"""Oracle of the owner-assignment planner, in plain Python.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg use
this module; the library does not.

What is computed follows the DMuon pages:
  * FAQ, "Why isn't DMuon just ZeRO-1?": every dedicated matrix has exactly
    one owner rank, which runs its whole Newton-Schulz step;
  * Training Guide, "Verify Parameter Assignment": the assignment of the
    dedicated parameters to the ranks is summarised by the per-rank loads
    and an imbalance figure.

The pages print neither the cost of a matrix nor the assignment rule; this
oracle takes these readings:
  * a matrix's cost is one of three models --
      "numel":      rows * cols;
      "ns_nominal": ns_steps * (4 m^2 n + 2 m^3), m = min(rows, cols),
                    n = max(rows, cols), the usual flop count of the
                    quintic iteration;
      "roofline":   the time the owner step takes at the device's peaks:
                    the multiply-add flops of the products the library runs
                    for that matrix (symmetric results counted once, the
                    form the backend picks) at the bf16 matrix-core peak,
                    plus the bytes of momentum and update at the HBM peak;
  * matrices are taken in decreasing cost (ties: lower index first) and each
    goes to the rank with the smallest load so far (ties: lower rank) -- the
    longest-processing-time-first greedy rule;
  * imbalance = max(load) / mean(load) - 1 (0 when every cost is 0).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

PEAK_BF16_FLOPS = 2516.6e12    # dense bf16 matrix-core peak of the device
PEAK_HBM_BYTES = 8.0e12        # HBM bandwidth of the device


def _mn(rows: int, cols: int) -> Tuple[int, int]:
    return min(rows, cols), max(rows, cols)


def executed_flops(rows: int, cols: int, ns_steps: int, backend: str) -> int:
    """Flops (2 per multiply-add) of the products of one NS call: symmetric
    d x d results count their upper triangle with the diagonal, m(m+1)/2
    entries; the Gram form is taken when backend is "gram" and n >= 2m."""
    m, n = _mn(rows, cols)
    K = ns_steps
    if K == 0:
        return 0
    sym = m * (m + 1)            # 2 * m(m+1)/2 entries: flops per unit of contraction
    if backend == "gram" and n >= 2 * m:
        total = sym * n                       # R = X0 X0^T
        for k in range(K):
            total += sym * m                  # P_k
            if k >= 1:
                total += sym * m              # Q <- P_k Q
            if k + 1 < K:
                total += 2 * sym * m          # T = P_k A, A <- T P_k
        total += 2 * m * n * m                # O = Q X0
        return total
    per_iter = sym * n + sym * m + 2 * m * n * m   # A = X X^T, B = bA + cA^2, X <- aX + BX
    return K * per_iter


def elementwise_bytes(rows: int, cols: int, param_bytes: int = 2, grad_bytes: int = 2) -> int:
    """Bytes of the momentum pass (grad in, fp32 momentum in and out, the NS
    input and its transpose out in bf16) and the update pass (param in and
    out, O in)."""
    e = rows * cols
    return e * (grad_bytes + 8 + 2 + 2) + e * (2 * param_bytes + 2)


def matrix_cost(rows: int, cols: int, model: str, ns_steps: int = 5, backend: str = "gram") -> float:
    m, n = _mn(rows, cols)
    if model == "numel":
        return float(rows * cols)
    if model == "ns_nominal":
        return float(ns_steps * (4 * m * m * n + 2 * m ** 3))
    if model == "roofline":
        return (executed_flops(rows, cols, ns_steps, backend) / PEAK_BF16_FLOPS
                + elementwise_bytes(rows, cols) / PEAK_HBM_BYTES)
    raise ValueError(model)


def assign_owners(costs: Sequence[float], nranks: int) -> Tuple[List[int], List[float]]:
    """Longest-processing-time-first greedy: returns (owner of each matrix,
    load of each rank)."""
    if nranks < 1:
        raise ValueError("nranks must be >= 1")
    order = sorted(range(len(costs)), key=lambda i: (-costs[i], i))
    loads = [0.0] * nranks
    owner = [-1] * len(costs)
    for i in order:
        r = min(range(nranks), key=lambda q: (loads[q], q))
        owner[i] = r
        loads[r] += costs[i]
    return owner, loads


def imbalance(loads: Sequence[float]) -> float:
    total = sum(loads)
    if total == 0:
        return 0.0
    return max(loads) / (total / len(loads)) - 1.0


def plan(shapes: Sequence[Tuple[int, int]], nranks: int, model: str = "ns_nominal", ns_steps: int = 5,
         backend: str = "gram"):
    """(owners, costs, loads, imbalance) of a list of (rows, cols)."""
    costs = [matrix_cost(r, c, model, ns_steps, backend) for r, c in shapes]
    owner, loads = assign_owners(costs, nranks)
    return owner, costs, loads, imbalance(loads)
