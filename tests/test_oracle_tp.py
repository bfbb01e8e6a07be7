"""Pins of the tensor-parallel (sharded) Newton-Schulz oracle: exact rational
equality with the unsharded standard form, float64 agreement with the
unsharded oracle for both splits and both forms, the diagonal closed form,
shard-order independence, and planted mistakes that the pins must catch."""
import inspect
import math
import types
from fractions import Fraction

import numpy as np
import pytest

from oracle import muon as orc
from oracle import tp_gram as tp_oracle


def _frac(a):
    out = np.empty(a.shape, dtype=object)
    for idx, v in np.ndenumerate(a):
        out[idx] = Fraction(v)
    return out


def _phi(x, K=5, abc=orc.DEFAULT_COEFFS):
    a, b, c = abc
    for _ in range(K):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _pins(tp):
    rng = np.random.default_rng(11)

    # exact rationals: both sharded forms equal the unsharded standard form
    # on a pre-scaled rational X0 (no square root involved), for both splits
    # and uneven shard sizes; coefficients as exact fractions
    abc = (Fraction(3, 1), Fraction(-4, 1), Fraction(2, 1))
    for split, shape, sizes in ((1, (3, 7), (3, 2, 2)), (0, (6, 3), (1, 4, 1)), (1, (2, 5), (5,))):
        u = _frac(rng.integers(-3, 4, size=shape).astype(float)) / 16
        x0 = u if split == 1 else u.T
        ref = orc.ns_direct(x0, 3, abc)
        ref = ref if split == 1 else ref.T
        for form in (tp.gram_form_sharded, tp.direct_form_sharded):
            parts = tp.orient(tp.split_matrix(u, split, sizes), split)
            got = form(parts, 3, abc)
            got = [g if split == 1 else g.T for g in got]
            assert np.array_equal(tp.join_shards(got, split), ref), (form.__name__, split, shape)

    # float64: equal to the unsharded oracle on the concatenated matrix, for
    # both splits, both backends, shards of different sizes and norms, and a
    # Gram formed over the longer side (split = 1 of a tall matrix)
    cases = [(1, (48, 160), (64, 16, 80)), (0, (160, 48), (100, 60)), (1, (96, 40), (10, 30)),
             (0, (40, 96), (7, 33)), (1, (32, 64), (64,))]
    for split, shape, sizes in cases:
        u = rng.standard_normal(shape)
        parts = tp.split_matrix(u, split, sizes)
        parts[0] = parts[0] * 30.0          # shards of very different norms
        u = tp.join_shards(parts, split)
        for backend in ("gram", "direct"):
            got = tp.join_shards(tp.orthogonalize_sharded(parts, split, 5, backend), split)
            ref = orc.orthogonalize(u, 5, "direct")
            err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
            assert err <= 1e-10, (split, shape, backend, err)

    # diagonal closed form through shards: U = [diag(d) | 0] cut into columns
    d = np.array([0.9, 0.5, 0.25, 0.05])
    u = np.zeros((4, 10))
    u[np.arange(4), np.arange(4)] = d
    parts = tp.split_matrix(u, 1, (2, 5, 3))
    o = tp.join_shards(tp.orthogonalize_sharded(parts, 1, 5, "gram"), 1)
    expect = np.zeros_like(u)
    expect[np.arange(4), np.arange(4)] = _phi(d / (np.linalg.norm(d) + 1e-7))
    assert np.allclose(o, expect, rtol=1e-13, atol=1e-15)

    # shard order does not matter: permuted shards give permuted outputs
    u = rng.standard_normal((24, 90))
    parts = tp.split_matrix(u, 1, (30, 20, 40))
    a = tp.orthogonalize_sharded(parts, 1, 5, "gram")
    b = tp.orthogonalize_sharded([parts[2], parts[0], parts[1]], 1, 5, "gram")
    for x, y in zip([a[2], a[0], a[1]], b):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-14)

    # the global norm is the norm of the whole matrix
    parts = [rng.standard_normal((5, 3)), rng.standard_normal((5, 9))]
    assert math.isclose(tp.global_frobenius_norm(parts), np.linalg.norm(np.hstack(parts)), rel_tol=1e-14)


def test_tp_pins():
    _pins(tp_oracle)


MUTATIONS = {
    "per-shard norm": ("s = 1.0 / (global_frobenius_norm(xs) + eps)\n    x0s = [x * s for x in xs]",
                       "x0s = [x / (global_frobenius_norm([x]) + eps) for x in xs]"),
    "first shard's Gram only": ("    for p in partial[1:]:\n        total = total + p\n", ""),
    "mean instead of sum": ("    return total\n\n\ndef gram_form_sharded", "    return total / len(partial)\n\n\ndef gram_form_sharded"),
    "Q applied to shard 0": ("return [Q @ x for x in x0s]", "return [Q @ x0s[0] for x in x0s]"),
    "local A in direct form": ("        xs = [a * x + B @ x for x in xs]",
                               "        xs = [a * x + (b * (x @ x.T) + c * (x @ x.T) @ (x @ x.T)) @ x for x in xs]"),
    "no transpose for row blocks": ("xs = [s if split == 1 else s.T for s in shards]", "xs = [s for s in shards]"),
    "no transpose back": ("return [o if split == 1 else o.T for o in os_]", "return list(os_)"),
    "A <- P A": ("A = P @ A @ P", "A = P @ A"),
    "Gram over the split side": ("partial = [x @ x.T for x in xs]", "partial = [x.T @ x for x in xs]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_tp_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(tp_oracle)
    assert old in src, name
    mod = types.ModuleType("tp_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "tp_mutant", "exec"), mod.__dict__)
    with pytest.raises(Exception):
        _pins(mod)
