"""Parity of the library's owner planner (dmuon_assign_owners, host code in
the C-ABI library) with the owner oracle: owners, costs, loads and the
imbalance must be identical -- integer decisions bit-exact, and the floating
costs too, since both sides form every cost from the exact integer count by
one rounding and add the loads in the same order."""
import numpy as np
import pytest

import dmuon_inputs as di
from oracle import owners as oow


@pytest.fixture(scope="module")
def dm():
    import matrix_optimizer_step_owned_amd as dm
    return dm


def _shape_sets():
    sets = {f"workload {w}": [(m.rows, m.cols) for m in di.workload(w).matrices] for w in range(5)}
    eight_b = []
    for _ in range(32):
        eight_b += [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096),
                    (4096, 14336)]
    sets["8B, 32 layers"] = eight_b
    rng = np.random.default_rng(9)
    sets["random, many ties"] = [(int(a), int(b)) for a, b in rng.choice([64, 128, 1000, 4096], size=(300, 2))]
    sets["random ragged"] = [(int(a), int(b)) for a, b in rng.integers(1, 20000, size=(500, 2))]
    sets["huge"] = [(1 << 24, 1 << 24), (1 << 24, 3), (5, 1 << 24)]
    return sets


@pytest.mark.parametrize("model", ["numel", "ns_nominal", "roofline"])
@pytest.mark.parametrize("backend", ["gram", "direct"])
def test_planner_matches_oracle(dm, model, backend):
    for name, shapes in _shape_sets().items():
        for nranks in (1, 2, 3, 8, 64, 1000):
            for ns_steps in (5, 1, 0):
                got = dm.dmuon_assign_owners(shapes, nranks, model, ns_steps=ns_steps, ns_backend=backend)
                owner, costs, loads, imb = oow.plan(shapes, nranks, model, ns_steps, backend)
                what = (name, nranks, ns_steps)
                assert got["owner"] == owner, what
                assert got["cost"] == costs, what
                assert got["loads"] == loads, what
                assert got["imbalance"] == imb, what


def test_planner_errors(dm):
    with pytest.raises(dm.DmuonError):
        dm.dmuon_assign_owners([(4, 4)], 0)
    with pytest.raises(dm.DmuonError):
        dm.dmuon_assign_owners([(0, 4)], 2)
    with pytest.raises(dm.DmuonError):
        dm.dmuon_assign_owners([(4, (1 << 24) + 1)], 2)
    with pytest.raises(dm.DmuonError):
        dm.dmuon_assign_owners([(4, 4)], 2, 7)
    with pytest.raises(dm.DmuonError):
        dm.dmuon_assign_owners([(4, 4)], 2, ns_steps=17)
    empty = dm.dmuon_assign_owners([], 4)
    assert empty["owner"] == [] and empty["loads"] == [0.0] * 4 and empty["imbalance"] == 0.0


def test_planner_balances_the_3b_stack(dm):
    """196 matrices over 8 owners: the NS-cost models balance flops to well
    under a percent; counting elements leaves the flops uneven."""
    shapes = [(m.rows, m.cols) for m in di.workload(2).matrices]
    flops = [oow.matrix_cost(r, c, "ns_nominal") for r, c in shapes]
    out = {}
    for model in ("numel", "ns_nominal", "roofline"):
        owner = dm.dmuon_assign_owners(shapes, 8, model)["owner"]
        per = [sum(f for f, o in zip(flops, owner) if o == q) for q in range(8)]
        out[model] = max(per) / (sum(per) / 8) - 1
    assert out["ns_nominal"] < 0.01
    assert out["roofline"] < 0.02
