"""Pins of the owner-assignment oracle: a hand-worked greedy example, the
tight instance of Graham's bound for the longest-processing-time rule,
brute-force optima on tiny instances, bookkeeping invariants and the cost
models' closed forms; planted mistakes must fail a pin."""
import inspect
import itertools
import math
import types

import numpy as np
import pytest

from oracle import owners as owners_oracle


def _opt_makespan(costs, nranks):
    best = math.inf
    for assign in itertools.product(range(nranks), repeat=len(costs)):
        loads = [0.0] * nranks
        for c, r in zip(costs, assign):
            loads[r] += c
        best = min(best, max(loads))
    return best


def _pins(ow):
    # hand-worked: 7, 6, 5, 4, 3 on two ranks
    owner, loads = ow.assign_owners([7, 6, 5, 4, 3], 2)
    assert owner == [0, 1, 1, 0, 0] and loads == [14.0, 11.0]
    assert math.isclose(ow.imbalance(loads), 14 / 12.5 - 1, rel_tol=1e-15)

    # Graham's tight instance for two ranks: the greedy reaches 7 where 6 is optimal
    _, loads = ow.assign_owners([3, 3, 2, 2, 2], 2)
    assert max(loads) == 7 and _opt_makespan([3, 3, 2, 2, 2], 2) == 6

    # random tiny instances: never better than the optimum, never worse than
    # (4/3 - 1/(3 ranks)) times it
    rng = np.random.default_rng(3)
    for _ in range(60):
        n, r = int(rng.integers(1, 8)), int(rng.integers(1, 4))
        costs = [float(x) for x in rng.integers(1, 20, size=n)]
        owner, loads = ow.assign_owners(costs, r)
        opt = _opt_makespan(costs, r)
        assert opt <= max(loads) <= (4 / 3 - 1 / (3 * r)) * opt + 1e-12, (costs, r)
        # every matrix placed once; loads add up
        assert sorted(set(owner)) == sorted(set(owner) & set(range(r))) and -1 not in owner
        assert math.isclose(sum(loads), sum(costs), rel_tol=1e-15)
        for q in range(r):
            assert math.isclose(loads[q], sum(c for c, o in zip(costs, owner) if o == q), rel_tol=1e-15)

    # more ranks than matrices: each matrix alone, the largest on rank 0
    owner, loads = ow.assign_owners([2.0, 5.0, 3.0], 5)
    assert owner == [2, 0, 1] and loads == [5.0, 3.0, 2.0, 0.0, 0.0]

    # equal loads give no imbalance; no work gives none either
    assert ow.imbalance([4.0, 4.0, 4.0]) == 0.0 and ow.imbalance([0.0, 0.0]) == 0.0

    # nominal NS flops: 5 (4 m^2 n + 2 m^3); 256 x 512 gives 0.84 GFLOP, and
    # the orientation of the matrix does not matter
    assert ow.matrix_cost(256, 512, "ns_nominal", 5) == 838860800.0
    assert ow.matrix_cost(512, 256, "ns_nominal", 5) == 838860800.0
    assert ow.matrix_cost(3, 7, "numel") == 21.0

    # executed products, to leading order: the standard form 3 m^2 n + m^3
    # per iteration, the Gram form 3 m^2 n + 17 m^3 per five iterations
    m, n = 4096, 3 * 4096
    g = ow.executed_flops(m, n, 5, "gram")
    d = ow.executed_flops(m, n, 5, "direct")
    assert abs(g / (3 * m * m * n + 17 * m ** 3) - 1) < 1e-3
    assert abs(d / (5 * (3 * m * m * n + m ** 3)) - 1) < 1e-3
    # near-square matrices take the standard form under both backends
    assert ow.executed_flops(1000, 1500, 5, "gram") == ow.executed_flops(1000, 1500, 5, "direct")
    assert ow.executed_flops(64, 64, 0, "gram") == 0

    # roofline time: products at the matrix-core peak plus 20 bytes per
    # element at the HBM peak
    t = ow.matrix_cost(1024, 4096, "roofline", 5, "gram")
    assert math.isclose(t, ow.executed_flops(1024, 4096, 5, "gram") / 2516.6e12 + 20 * 1024 * 4096 / 8e12,
                        rel_tol=1e-14)


def test_owner_pins():
    _pins(owners_oracle)


MUTATIONS = {
    "ascending order": ("key=lambda i: (-costs[i], i)", "key=lambda i: (costs[i], i)"),
    "most loaded rank": ("r = min(range(nranks), key=lambda q: (loads[q], q))",
                         "r = max(range(nranks), key=lambda q: (loads[q], -q))"),
    "ties to the higher rank": ("key=lambda q: (loads[q], q))", "key=lambda q: (loads[q], -q))"),
    "max over min": ("return max(loads) / (total / len(loads)) - 1.0", "return max(loads) / min(loads) - 1.0"),
    "m and n swapped": ("float(ns_steps * (4 * m * m * n + 2 * m ** 3))", "float(ns_steps * (4 * n * n * m + 2 * n ** 3))"),
    "no elementwise time": ("+ elementwise_bytes(rows, cols) / PEAK_HBM_BYTES)", ")"),
    "Gram step without T and A": ("total += 2 * sym * m          # T = P_k A, A <- T P_k", "pass"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_owner_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(owners_oracle)
    assert old in src, name
    mod = types.ModuleType("owners_mutant")
    exec(compile(src.replace(old, new), "owners_mutant", "exec"), mod.__dict__)
    with pytest.raises(Exception):
        _pins(mod)
