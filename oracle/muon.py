"""Oracle of the owner-side Muon step, in float64 numpy.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the GPU library does not.

What is computed follows the DMuon documentation pages:
  * Training Guide, "Step 4: Create Optimizer": the dedicated (Muon) group runs
    momentum, then Newton-Schulz (NS), then the update, on the owner only.
  * Training Guide, "Hyperparameter Guide" table: lr 0.02 scaled per parameter
    by 0.2*sqrt(max(m, n)); momentum 0.95; ns_steps 5; ns_backend "gram"
    (default) or "direct"; Nesterov input is grad + mu*buf.
  * FAQ, "Why isn't DMuon just ZeRO-1?": NS needs the whole (m, n) matrix.
  * FAQ, "What related work should I cite?": the "gram" backend is Gram
    Newton-Schulz (Zhang, Amsel, Chen, Dao).

Where the pages are silent, this oracle takes these readings:
  * momentum is additive, buf <- mu*buf + grad, and the Nesterov input uses the
    updated buf; without Nesterov the NS input is buf itself;
  * the NS input is normalised by its Frobenius norm plus eps (1e-7);
  * the iteration is the odd quintic X <- aX + (bA + cA^2)X with A = X X^T,
    coefficients (3.4445, -4.7750, 2.0315) unless a table is given, and runs
    on the wide orientation (a tall matrix is transposed, orthogonalised and
    transposed back);
  * the Gram form keeps the iteration on the m x m Gram matrix R = X0 X0^T:
    each step forms P = aI + bA + cA^2, accumulates Q <- P Q, moves
    A <- P A P, and finally returns Q X0 -- equal to the direct form in exact
    arithmetic, since every matrix involved is a polynomial in R;
  * decoupled weight decay: W <- W (1 - lr*wd) - lr*0.2*sqrt(max(m,n))*O;
  * a bf16 parameter is written by one round-to-nearest-even of that value.

Every function is written for any numpy dtype that supports +, * and @ (float64
arrays, or object arrays of fractions.Fraction for exact checks).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)


def _coeff_table(ns_steps: int, coeffs: Optional[Sequence]) -> list:
    """(a, b, c) for each of the ns_steps iterations.

    ``coeffs`` is None (the default quintic for every step), one (a, b, c)
    triple, or a flat / nested table of ns_steps triples."""
    if coeffs is None:
        return [DEFAULT_COEFFS] * ns_steps
    flat = list(np.asarray(coeffs, dtype=object).reshape(-1))
    if len(flat) == 3:
        return [tuple(flat)] * ns_steps
    if len(flat) != 3 * ns_steps:
        raise ValueError("coefficient table must hold 3 or 3*ns_steps values")
    return [tuple(flat[3 * k:3 * k + 3]) for k in range(ns_steps)]


# --- momentum (Hyperparameter Guide: momentum, nesterov rows) ---------------

def momentum_update(buf, grad, mu, nesterov: bool = True):
    """buf <- mu*buf + grad; NS input = grad + mu*buf (Nesterov) or buf.

    Returns (new_buf, ns_input)."""
    new_buf = mu * buf + grad
    ns_input = grad + mu * new_buf if nesterov else new_buf
    return new_buf, ns_input


# --- normalisation -----------------------------------------------------------

def frobenius_norm(x) -> float:
    return math.sqrt(float(np.sum(np.asarray(x, dtype=np.float64) ** 2)))


def normalize(x, eps: float = 1e-7):
    """X0 = X / (||X||_F + eps)."""
    return x / (frobenius_norm(x) + eps)


# --- Newton-Schulz, direct form (ns_backend="direct") ------------------------

def ns_direct(x0, ns_steps: int = 5, coeffs=None):
    """ns_steps quintic iterations on a wide (m <= n) X0."""
    x = x0
    for a, b, c in _coeff_table(ns_steps, coeffs):
        A = x @ x.T
        B = b * A + c * (A @ A)
        x = a * x + B @ x
    return x


# --- Newton-Schulz, Gram form (ns_backend="gram") ----------------------------

def _identity_like(r):
    m = r.shape[0]
    eye = np.zeros((m, m), dtype=r.dtype)
    one = r.dtype.type(1) if r.dtype != object else 1
    for i in range(m):
        eye[i, i] = one
    return eye


def ns_gram(x0, ns_steps: int = 5, coeffs=None):
    """The same iteration carried on R = X0 X0^T; returns Q X0."""
    table = _coeff_table(ns_steps, coeffs)
    if not table:
        return x0
    R = x0 @ x0.T
    I = _identity_like(R)
    A = R
    Q = None
    for k, (a, b, c) in enumerate(table):
        P = a * I + b * A + c * (A @ A)
        Q = P if Q is None else P @ Q
        if k + 1 < len(table):
            A = P @ A @ P
    return Q @ x0


# --- whole orthogonalisation ---------------------------------------------------

def orthogonalize(u, ns_steps: int = 5, backend: str = "gram", coeffs=None,
                  eps: float = 1e-7):
    """O = NS(U): orient wide, normalise, iterate, orient back."""
    tall = u.shape[0] > u.shape[1]
    x = u.T if tall else u
    x0 = normalize(x, eps)
    if backend == "direct":
        o = ns_direct(x0, ns_steps, coeffs)
    elif backend == "gram":
        o = ns_gram(x0, ns_steps, coeffs)
    else:
        raise ValueError(backend)
    return o.T if tall else o


# --- update (Hyperparameter Guide: lr row; weight_decay of Step 4) ------------

def lr_scale(rows: int, cols: int) -> float:
    """Per-parameter lr multiplier 0.2*sqrt(max(m, n))."""
    return 0.2 * math.sqrt(max(rows, cols))


def apply_update(w, o, lr: float, weight_decay: float = 0.0):
    """W <- W*(1 - lr*wd) - lr*0.2*sqrt(max(m,n))*O, in float64."""
    rows, cols = w.shape
    return w * (1.0 - lr * weight_decay) - (lr * lr_scale(rows, cols)) * o


def round_to_bf16(x):
    """Nearest bfloat16 value (ties to even) of float64 ``x``, as float64.

    bf16 keeps 8 significant bits; below 2**-126 the spacing is fixed at
    2**-133.  Values past the bf16 range are not expected here."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)               # x = f * 2**e with 0.5 <= |f| < 1
    e = np.maximum(e, -125)          # subnormal range keeps the 2**-133 grid
    q = np.rint(np.ldexp(x, 8 - e))  # round half to even
    return np.ldexp(q, e - 8)


# --- one whole step for one matrix --------------------------------------------

def muon_step(w, grad, buf, *, lr=0.02, momentum=0.95, nesterov=True,
              ns_steps=5, weight_decay=0.0, ns_backend="gram", coeffs=None,
              eps=1e-7, param_dtype="f32") -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """One Muon step of one owned matrix.

    Returns (w_new, buf_new, ns_input, o), all float64; w_new is rounded to
    bf16 when param_dtype is "bf16"."""
    buf_new, u = momentum_update(buf, grad, momentum, nesterov)
    o = orthogonalize(u, ns_steps, ns_backend, coeffs, eps)
    w_new = apply_update(w, o, lr, weight_decay)
    if param_dtype == "bf16":
        w_new = round_to_bf16(w_new)
    return w_new, buf_new, u, o

