"""Pins of the clipping oracle against values fixed by mathematics and by a
library routine (PyTorch's clip_grad_norm_ on float64 tensors), plus planted
mistakes that the pins must catch."""
import inspect
import math
import types

import numpy as np
import pytest

from oracle import clip as clip_oracle


def _pins(clip):
    rng = np.random.default_rng(5)

    # closed forms on constant arrays: N elements of value c
    n, c = 1000, -0.75
    g = [np.full(n, c)]
    for p, expect in ((2.0, abs(c) * math.sqrt(n)), (1.0, abs(c) * n), (math.inf, abs(c)),
                      (3.0, abs(c) * n ** (1.0 / 3.0))):
        assert math.isclose(clip.grad_norm(g, p), expect, rel_tol=1e-12), p

    # global over several arrays of different sizes: squares add
    a, b = np.full(10, 3.0), np.full(40, 0.5)
    assert math.isclose(clip.grad_norm([a, b], 2.0), math.sqrt(90.0 + 10.0), rel_tol=1e-14)

    # coefficient: max_norm / (total + 1e-6), clamped at 1, NaN kept
    assert clip.clip_coefficient(2.0, 1.0) == 1.0 / (2.0 + 1e-6)
    assert clip.clip_coefficient(0.5, 1.0) == 1.0
    assert math.isnan(clip.clip_coefficient(float("nan"), 1.0))

    # PyTorch's clip_grad_norm_ on float64 tensors, one bucket, several p
    import torch
    shapes = [(7, 5), (33,), (4, 4, 4)]
    for p in (2.0, 1.0, math.inf, 3.0):
        gs = [rng.standard_normal(s) * 10.0 ** rng.uniform(-2, 1) for s in shapes]
        params = []
        for x in gs:
            t = torch.nn.Parameter(torch.zeros(x.shape, dtype=torch.float64))
            t.grad = torch.from_numpy(x.copy())
            params.append(t)
        tot = float(torch.nn.utils.clip_grad_norm_(params, max_norm=0.3, norm_type=p))
        out, totals, _ = clip.clip_grad_norm(gs, [0] * len(gs), [0.3], p)
        assert math.isclose(totals[0], tot, rel_tol=1e-12), p
        for o, t in zip(out, params):
            assert np.allclose(o, t.grad.numpy(), rtol=1e-12, atol=0.0), p

    # below the threshold nothing changes, bit for bit
    gs = [rng.standard_normal(50) * 1e-3]
    out, totals, coefs = clip.clip_grad_norm(gs, [0], [10.0], 2.0)
    assert coefs[0] == 1.0 and np.array_equal(out[0], gs[0])

    # after clipping, the bucket's norm is max_norm * total / (total + eps)
    gs = [rng.standard_normal(300), rng.standard_normal((20, 20))]
    out, totals, _ = clip.clip_grad_norm(gs, [0, 0], [1.0], 2.0)
    assert math.isclose(clip.grad_norm(out, 2.0), totals[0] / (totals[0] + 1e-6), rel_tol=1e-12)

    # buckets are independent, and a NaN stays inside its bucket
    g0, g1 = rng.standard_normal(64) * 5, rng.standard_normal(64) * 5
    g0n = g0.copy()
    g0n[3] = float("nan")
    out, totals, coefs = clip.clip_grad_norm([g0n, g1], [0, 1], [1.0, 2.0], 2.0)
    assert np.isnan(out[0]).all() and math.isnan(totals[0])
    ref1, t1, _ = clip.clip_grad_norm([g1], [0], [2.0], 2.0)
    assert np.array_equal(out[1], ref1[0]) and totals[1] == t1[0]

    # an empty bucket has norm 0 and coefficient 1
    out, totals, coefs = clip.clip_grad_norm([g1], [1], [1.0, 1.0], 2.0)
    assert totals[0] == 0.0 and coefs[0] == 1.0


def test_clip_pins():
    _pins(clip_oracle)


MUTATIONS = {
    "no p-th root": ("return total ** (1.0 / p)", "return total"),
    "no clamp": ("return 1.0 if coef >= 1.0 else coef", "return coef"),
    "eps dropped": ("coef = max_norm / (total + EPS)", "coef = max_norm / total"),
    "per-array norm": ("t = grad_norm(members, p)", "t = max([grad_norm([m], p) for m in members] or [0.0])"),
    "inf-norm as sum": ("return float(max(float(np.max(np.abs(g))) if g.size else 0.0 for g in grads))",
                        "return float(sum(float(np.max(np.abs(g))) if g.size else 0.0 for g in grads))"),
    "wrong bucket coefficient": ("out = [np.asarray(g, dtype=np.float64) * coefs[k]",
                                 "out = [np.asarray(g, dtype=np.float64) * coefs[0]"),
    "abs dropped": ("np.abs(np.asarray(g, dtype=np.float64)) ** p", "np.asarray(g, dtype=np.float64) ** p"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_clip_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(clip_oracle)
    assert old in src, name
    mod = types.ModuleType("clip_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "clip_mutant", "exec"), mod.__dict__)
    with pytest.raises(Exception):
        _pins(mod)
