"""Plant plausible mistakes in a copy of the oracle and check that at least
one pin fails for each: the pins constrain every part of the oracle."""
import inspect
import types

import pytest

from oracle import muon as oracle_muon
from tests import oracle_pins

MUTATIONS = {
    "dropped A^2 term": ("B = b * A + c * (A @ A)", "B = b * A"),
    "X B instead of B X": ("x = a * x + B @ x", "x = a * x + x @ B"),
    "wrong sign of b": ("B = b * A + c * (A @ A)", "B = -b * A + c * (A @ A)"),
    "A = X^T X": ("A = x @ x.T", "A = x.T @ x if x.shape[0] == x.shape[1] else x @ x.T"),
    "gram: identity dropped": ("P = a * I + b * A + c * (A @ A)", "P = b * A + c * (A @ A)"),
    "gram: A <- P A": ("A = P @ A @ P", "A = P @ A"),
    "gram: final Q Q X0": ("return Q @ x0\n", "return Q @ Q @ x0\n"),
    "gram: last coefficients reused": ("for k, (a, b, c) in enumerate(table):",
                                       "for k, (a, b, c) in enumerate([table[0]] * len(table)):"),
    "eps under the square root": ("return x / (frobenius_norm(x) + eps)",
                                  "return x / math.sqrt(frobenius_norm(x) ** 2 + eps)"),
    "max-abs instead of Frobenius": ("return x / (frobenius_norm(x) + eps)",
                                     "return x / (float(np.max(np.abs(np.asarray(x, dtype=float)))) + eps)"),
    "nesterov on the old buffer": ("ns_input = grad + mu * new_buf if nesterov else new_buf",
                                   "ns_input = grad + mu * buf if nesterov else new_buf"),
    "EMA momentum": ("new_buf = mu * buf + grad", "new_buf = mu * buf + (1 - mu) * grad"),
    "lr scale on min(m, n)": ("return 0.2 * math.sqrt(max(rows, cols))", "return 0.2 * math.sqrt(min(rows, cols))"),
    "decay with the scaled lr": ("return w * (1.0 - lr * weight_decay)",
                                 "return w * (1.0 - lr * lr_scale(rows, cols) * weight_decay)"),
    "bf16 truncation": ("q = np.rint(np.ldexp(x, 8 - e))", "q = np.trunc(np.ldexp(x, 8 - e))"),
    "bf16 ties away from zero": ("q = np.rint(np.ldexp(x, 8 - e))",
                                 "q = np.sign(x) * np.floor(np.abs(np.ldexp(x, 8 - e)) + 0.5)"),
    "coefficients a/c swapped": ("for a, b, c in _coeff_table(ns_steps, coeffs):",
                                 "for c, b, a in _coeff_table(ns_steps, coeffs):"),
}


def _mutant(old: str, new: str) -> types.ModuleType:
    src = inspect.getsource(oracle_muon)
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a shape error from the mistake
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches: {name}"
