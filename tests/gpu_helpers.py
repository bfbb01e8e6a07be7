"""Helpers shared by the GPU tests: uploads of seeded inputs, read-back and
error measures.  No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def upload(raw: np.ndarray, dtype: str) -> torch.Tensor:
    """Seeded host array (float32, or uint16 bf16 bit patterns) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to(DEV)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (nb if nb > 0 else 1.0)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (normal range)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, min_exact: float = 0.999, what: str = "",
                      slack: np.ndarray | float = 0.0):
    """Every element within one bf16 ulp of the reference (plus ``slack``, the
    fp32 evaluation error of the kernel's arithmetic), and almost all equal."""
    diff = np.abs(got - ref)
    ulp = np.maximum(bf16_ulp(ref), bf16_ulp(got))
    bad = diff > ulp * (1 + 1e-12) + slack
    assert not bad.any(), (what, int(bad.sum()), float((diff / ulp).max()))
    exact = float(np.mean(got == ref))
    assert exact >= min_exact, (what, exact)


def check_param_step(got_new: np.ndarray, w_old: np.ndarray, ref_new_unrounded: np.ndarray,
                     param_dtype: str, ns_tol: float, ns_precision: str, what: str = "",
                     elementwise: bool = True) -> float:
    """Parameter change of one step against the oracle's change.

    fp32 parameters: relative error of (W_new - W_old) <= ns_tol.
    bf16 parameters: the stored value is the rounding of the kernel's fp32
    result, which moves each element by at most half a bf16 ulp; the allowed
    relative error is ns_tol plus that rounding's norm over the change's norm.
    With fp32 NS products the change is accurate far below a bf16 ulp, so
    additionally every element must sit within one ulp of the oracle's rounded
    value, 99 % of them equal (``elementwise``; large square matrices, whose
    near-singular directions the iteration amplifies, can hold single
    elements beyond that even when the NS output meets its tolerance).
    Returns the measured relative error."""
    d_ref = ref_new_unrounded - w_old
    err = rel(got_new - w_old, d_ref)
    if param_dtype == "f32":
        assert err <= ns_tol, (what, err)
        return err
    allow = float(np.linalg.norm(0.5 * bf16_ulp(got_new)) / np.linalg.norm(d_ref))
    assert err <= ns_tol + allow, (what, err, allow)
    if ns_precision == "f32" and elementwise:
        from oracle import muon as _orc
        # fp32 evaluation of the update, and the NS error itself, which near a
        # cancellation (W_new close to 0) can span several ulps of the result
        slack = 4 * 2.0 ** -24 * (np.abs(w_old) + np.abs(d_ref)) + 10 * ns_tol * np.abs(d_ref)
        assert_bf16_close(got_new, _orc.round_to_bf16(ref_new_unrounded), min_exact=0.99,
                          what=what, slack=slack)
    return err
