"""Pins for the oracle: checks against facts fixed by the mathematics, not by
the oracle's own code.

Each ``pin_*`` takes an oracle module and raises AssertionError on mismatch,
so the same checks run on the real oracle (test_oracle_pins.py) and on copies
with a planted mistake (test_oracle_mutations.py).

The closed forms used:
  * the NS map acts on singular values only: for G = U diag(s) V^T the
    quintic iteration gives U diag(phi(s_hat)) V^T with s_hat = s/(||s||+eps)
    (||G||_F = ||s||_2) and phi the scalar polynomial p(x) = a x + b x^3 + c x^5
    composed once per iteration -- checked on diagonal inputs with a scalar
    loop and on general inputs through numpy's SVD;
  * the Gram form equals the direct form exactly in rational arithmetic;
  * NS commutes with transposition and with orthogonal changes of basis, is
    odd, and is invariant to positive scaling when eps = 0;
  * the momentum recurrence unrolled by hand;
  * the update rule's closed values.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)
EPS = 1e-7


def phi(x: float, table) -> float:
    """Scalar NS polynomial composed over the coefficient table."""
    for a, b, c in table:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _table(ns_steps, coeffs=None):
    if coeffs is None:
        return [QUINTIC] * ns_steps
    return [tuple(coeffs[3 * k:3 * k + 3]) for k in range(ns_steps)]


def _rel(a, b) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


# ---------------------------------------------------------------------------

def pin_bf16_rounding(orc):
    """round_to_bf16 agrees with torch's float32 -> bfloat16 cast (RNE)."""
    import torch
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
        # exact ties between two bf16 neighbours, both parities
        # (odd multiples of 2**-8 in [1, 2): halfway between bf16 neighbours)
        (2 * np.arange(128, 256, dtype=np.float64) + 1) * 2.0 ** -8,
        -(2 * np.arange(128, 256, dtype=np.float64) + 1) * 2.0 ** -3,
        # subnormal range of bf16 / fp32
        np.array([2.0 ** -130, 3 * 2.0 ** -134, 1.5 * 2.0 ** -133, 2.0 ** -126, 0.0, -0.0]),
    ]).astype(np.float32).astype(np.float64)
    ours = orc.round_to_bf16(vals)
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


def pin_diagonal_closed_form(orc):
    """Diagonal (and diagonal-transposed) inputs against the scalar polynomial,
    for both backends, several step counts and a per-step coefficient table."""
    rng = np.random.default_rng(2)
    custom = [3.0, -3.2, 1.2, 2.0, -1.5, 0.5, 1.5, -0.5, 0.0]
    cases = [(5, 9, 5, None), (9, 5, 5, None), (6, 6, 3, None), (4, 7, 3, custom),
             (7, 4, 1, None), (3, 8, 2, None)]
    for rows, cols, k, coeffs in cases:
        m = min(rows, cols)
        d = rng.uniform(0.05, 1.0, m) * rng.choice([-1.0, 1.0], m)
        g = np.zeros((rows, cols))
        g[np.arange(m), np.arange(m)] = d
        nrm = math.sqrt(float(np.sum(d * d)))
        expect = np.zeros((rows, cols))
        for i in range(m):
            expect[i, i] = phi(d[i] / (nrm + EPS), _table(k, coeffs))
        for backend in ("direct", "gram"):
            o = orc.orthogonalize(g, k, backend, coeffs, EPS)
            assert o.shape == g.shape
            err = float(np.max(np.abs(o - expect)))
            assert err < 1e-12, (rows, cols, k, backend, err)


def pin_known_scalar_values(orc):
    """1x1 inputs: one step of the default quintic at 1 gives a+b+c = 0.701;
    five steps give phi_5(1), computed here in exact rationals."""
    one = np.array([[1.0]])
    o1 = orc.orthogonalize(one, 1, "direct", None, 0.0)
    assert abs(o1[0, 0] - 0.701) < 1e-15
    x = Fraction(1)
    fa, fb, fc = (Fraction(str(v)) for v in QUINTIC)
    for _ in range(5):
        x = fa * x + fb * x ** 3 + fc * x ** 5
    for backend in ("direct", "gram"):
        o5 = orc.orthogonalize(one, 5, backend, None, 0.0)
        assert abs(o5[0, 0] - float(x)) < 1e-14, (backend, o5[0, 0], float(x))


def pin_svd_closed_form(orc):
    """General tiny inputs: U diag(phi(s_hat)) V^T from numpy's SVD."""
    rng = np.random.default_rng(3)
    for rows, cols in [(5, 8), (8, 5), (6, 6), (3, 11), (12, 4), (1, 6)]:
        g = rng.standard_normal((rows, cols))
        u, s, vt = np.linalg.svd(g, full_matrices=False)
        sh = s / (np.linalg.norm(s) + EPS)
        expect = u @ np.diag([phi(v, _table(5)) for v in sh]) @ vt
        for backend in ("direct", "gram"):
            o = orc.orthogonalize(g, 5, backend, None, EPS)
            assert _rel(o, expect) < 1e-12, (rows, cols, backend, _rel(o, expect))


def pin_polar_band(orc):
    """Singular values driven into the band near 1: with every normalised
    singular value in [0.01, 1], O's singular values are phi_5 of them and O
    is within max|phi_5 - 1| of the polar factor U V^T in spectral norm."""
    rng = np.random.default_rng(4)
    grid = np.linspace(0.01, 1.0, 2001)
    vals = np.array([phi(v, _table(5)) for v in grid])
    lo, hi = float(vals.min()), float(vals.max())
    dev = float(np.max(np.abs(vals - 1.0)))
    assert 0.6 < lo < 0.7 and 1.1 < hi < 1.2     # the documented band of this quintic
    for rows, cols in [(6, 10), (10, 6), (7, 7)]:
        m = min(rows, cols)
        u, _ = np.linalg.qr(rng.standard_normal((rows, rows)))
        v, _ = np.linalg.qr(rng.standard_normal((cols, cols)))
        raw = rng.uniform(0.05, 1.0, m)
        shat = raw / np.linalg.norm(raw)          # normalised singular values
        assert shat.min() >= 0.01
        g = u[:, :m] @ np.diag(3.0 * shat) @ v[:, :m].T
        o = orc.orthogonalize(g, 5, "gram", None, 0.0)
        so = np.linalg.svd(o, compute_uv=False)
        assert np.allclose(np.sort(so), np.sort([phi(x, _table(5)) for x in shat]), atol=1e-12)
        assert lo - 1e-12 <= so.min() and so.max() <= hi + 1e-12
        polar = u[:, :m] @ v[:, :m].T
        assert np.linalg.norm(o - polar, 2) <= dev + 1e-12


def pin_gram_equals_direct_exact(orc):
    """Gram and direct forms give identical rational matrices."""
    F = Fraction
    cases = [
        (np.array([[F(1, 4), F(-1, 8), F(3, 16)],
                   [F(1, 8), F(1, 4), F(-1, 16)]], dtype=object), 5, None),
        (np.array([[F(1, 5), F(0), F(-1, 10), F(1, 10)],
                   [F(1, 10), F(1, 5), F(0), F(-1, 5)],
                   [F(0), F(-1, 10), F(3, 10), F(1, 10)]], dtype=object), 3,
         [F(3), F(-16, 5), F(6, 5), F(2), F(-3, 2), F(1, 2), F(3, 2), F(-1, 2), F(0)]),
    ]
    fq = [Fraction(str(v)) for v in QUINTIC]
    for x0, k, coeffs in cases:
        c = coeffs if coeffs is not None else fq
        d = orc.ns_direct(x0, k, c)
        g = orc.ns_gram(x0, k, c)
        assert d.shape == g.shape == x0.shape
        assert all(d[i, j] == g[i, j] for i in range(d.shape[0]) for j in range(d.shape[1]))
        assert any(d[i, j] != x0[i, j] for i in range(d.shape[0]) for j in range(d.shape[1]))


def pin_gram_equals_direct_fp64(orc):
    rng = np.random.default_rng(5)
    for rows, cols in [(16, 40), (40, 16), (24, 24), (64, 200)]:
        g = rng.standard_normal((rows, cols))
        a = orc.orthogonalize(g, 5, "direct", None, EPS)
        b = orc.orthogonalize(g, 5, "gram", None, EPS)
        assert _rel(a, b) < 1e-12, (rows, cols, _rel(a, b))


def pin_invariances(orc):
    rng = np.random.default_rng(6)
    for backend in ("direct", "gram"):
        for rows, cols in [(6, 9), (9, 6), (7, 7)]:
            g = rng.standard_normal((rows, cols))
            o = orc.orthogonalize(g, 5, backend, None, EPS)
            # transpose
            assert _rel(orc.orthogonalize(g.T.copy(), 5, backend, None, EPS), o.T) < 1e-12
            # orthogonal change of basis
            p, _ = np.linalg.qr(rng.standard_normal((rows, rows)))
            q, _ = np.linalg.qr(rng.standard_normal((cols, cols)))
            assert _rel(orc.orthogonalize(p @ g @ q.T, 5, backend, None, EPS), p @ o @ q.T) < 1e-11
            # odd map
            assert _rel(orc.orthogonalize(-g, 5, backend, None, EPS), -o) < 1e-14
            # scale invariance with eps = 0
            o0 = orc.orthogonalize(g, 5, backend, None, 0.0)
            assert _rel(orc.orthogonalize(37.5 * g, 5, backend, None, 0.0), o0) < 1e-12
            # zero steps: the normalised input
            assert _rel(orc.orthogonalize(g, 0, backend, None, EPS), g / (np.linalg.norm(g) + EPS)) < 1e-15
        # zero gradient: zero output, nothing non-finite
        z = orc.orthogonalize(np.zeros((5, 8)), 5, backend, None, EPS)
        assert np.all(z == 0.0)
        # rank one: G = x y^T -> phi(||G|| / (||G|| + eps)) G / ||G||
        x, y = rng.standard_normal(5), rng.standard_normal(8)
        g = np.outer(x, y)
        nrm = np.linalg.norm(g)
        expect = phi(nrm / (nrm + EPS), _table(5)) * g / nrm
        assert _rel(orc.orthogonalize(g, 5, backend, None, EPS), expect) < 1e-12
        # tiny norm: eps is added to the norm, not to its square
        t = 1e-7 * rng.standard_normal((4, 6)) / 5.0
        nt = np.linalg.norm(t)
        u, s, vt = np.linalg.svd(t, full_matrices=False)
        expect = u @ np.diag([phi(v / (nt + EPS), _table(5)) for v in s]) @ vt
        assert _rel(orc.orthogonalize(t, 5, backend, None, EPS), expect) < 1e-10


def pin_momentum_by_hand(orc):
    rng = np.random.default_rng(7)
    mu = 0.95
    g1, g2, g3 = (rng.standard_normal((3, 4)) for _ in range(3))
    m0 = np.zeros((3, 4))
    m1, u1 = orc.momentum_update(m0, g1, mu, True)
    assert np.allclose(m1, g1, rtol=0, atol=0)
    assert np.allclose(u1, 1.95 * g1, rtol=1e-15, atol=0)
    m2, u2 = orc.momentum_update(m1, g2, mu, True)
    assert np.allclose(m2, 0.95 * g1 + g2, rtol=1e-15, atol=1e-15)
    assert np.allclose(u2, 1.95 * g2 + 0.9025 * g1, rtol=1e-14, atol=1e-15)
    m3, u3 = orc.momentum_update(m2, g3, mu, True)
    assert np.allclose(m3, mu ** 2 * g1 + mu * g2 + g3, rtol=1e-14, atol=1e-15)
    # without Nesterov the NS input is the buffer itself
    n1, v1 = orc.momentum_update(m0, g1, mu, False)
    n2, v2 = orc.momentum_update(n1, g2, mu, False)
    assert np.array_equal(v1, g1) and np.allclose(v2, 0.95 * g1 + g2, rtol=1e-15, atol=1e-15)


def pin_update_rule(orc):
    # 256 x 512 at lr 0.02: effective lr 0.02 * 0.2 * sqrt(512)
    assert abs(orc.lr_scale(256, 512) * 0.02 - 0.0905096679918781) < 1e-15
    assert orc.lr_scale(3072, 1024) == orc.lr_scale(1024, 3072) == 0.2 * math.sqrt(3072)
    w = np.full((2, 3), 0.5)
    zero = np.zeros((2, 3))
    # decay alone uses the base lr: 0.5 * (1 - 0.02 * 0.1)
    assert np.allclose(orc.apply_update(w, zero, 0.02, 0.1), 0.5 * 0.998, rtol=1e-15, atol=0)
    one = np.ones((2, 3))
    assert np.allclose(orc.apply_update(zero, one, 0.02, 0.0), -0.02 * 0.2 * math.sqrt(3), rtol=1e-15, atol=0)
    # whole step with a zero gradient: only the decay moves W
    w2, m2, u2, o2 = orc.muon_step(w, zero, zero, lr=0.02, weight_decay=0.1)
    assert np.allclose(w2, 0.5 * 0.998, rtol=1e-15, atol=0) and np.all(o2 == 0)


def pin_step_rounds_bf16(orc):
    """A bf16 parameter step equals the float64 step rounded once."""
    rng = np.random.default_rng(8)
    w = orc.round_to_bf16(0.02 * rng.standard_normal((6, 10)))
    g = 1e-3 * rng.standard_normal((6, 10))
    w64, _, _, o = orc.muon_step(w, g, np.zeros_like(g), param_dtype="f32")
    wb, _, _, _ = orc.muon_step(w, g, np.zeros_like(g), param_dtype="bf16")
    assert np.array_equal(wb, orc.round_to_bf16(w64))
    assert not np.array_equal(wb, w)


ALL_PINS = [pin_bf16_rounding, pin_diagonal_closed_form, pin_known_scalar_values,
            pin_svd_closed_form, pin_polar_band, pin_gram_equals_direct_exact,
            pin_gram_equals_direct_fp64, pin_invariances, pin_momentum_by_hand,
            pin_update_rule, pin_step_rounds_bf16]
