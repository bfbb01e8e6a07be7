"""Pins of the AdamW oracle: PyTorch's torch.optim.AdamW on float64 tensors
(a library routine with the same definition), the first-step and
constant-gradient closed forms, geometric decay of the moments under a zero
gradient, and scale invariance without eps; planted mistakes must fail."""
import inspect
import math
import types

import numpy as np
import pytest

from oracle import adamw as adamw_oracle


def _pins(ow):
    import torch
    rng = np.random.default_rng(21)

    # PyTorch's AdamW, several steps and hyperparameter sets
    for hp in (dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
               dict(lr=3e-2, beta1=0.8, beta2=0.95, eps=1e-3, weight_decay=0.0),
               dict(lr=5e-4, beta1=0.0, beta2=0.5, eps=1e-6, weight_decay=0.3)):
        p0 = rng.standard_normal((6, 5))
        t = torch.nn.Parameter(torch.from_numpy(p0.copy()))
        opt = torch.optim.AdamW([t], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                weight_decay=hp["weight_decay"])
        p, m, v = p0, np.zeros_like(p0), np.zeros_like(p0)
        for step in range(1, 6):
            g = rng.standard_normal(p0.shape) * 10.0 ** rng.uniform(-3, 1)
            t.grad = torch.from_numpy(g.copy())
            opt.step()
            p, m, v = ow.adamw_step(p, g, m, v, step, **hp)
            st = opt.state[t]
            assert np.allclose(p, t.detach().numpy(), rtol=1e-12, atol=1e-15), (hp, step)
            assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=0), (hp, step)
            assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=0), (hp, step)

    # first step from zero state: p (1 - lr wd) - lr g / (|g| + eps)
    lr, eps, wd = 1e-3, 1e-8, 0.01
    p0, g = rng.standard_normal(50), rng.standard_normal(50) * 1e-4
    p1, m1, v1 = ow.adamw_step(p0, g, 0 * p0, 0 * p0, 1, lr=lr, eps=eps, weight_decay=wd)
    assert np.allclose(p1, p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-13, atol=1e-18)
    assert np.allclose(m1, 0.1 * g, rtol=1e-15) and np.allclose(v1, 0.001 * g * g, rtol=1e-12)

    # constant gradient: every step moves by the first step's amount
    p, m, v = p0, 0 * p0, 0 * p0
    for step in range(1, 8):
        prev = p
        p, m, v = ow.adamw_step(p, g, m, v, step, lr=lr, eps=eps, weight_decay=0.0)
        assert np.allclose(prev - p, lr * g / (np.abs(g) + eps), rtol=1e-9, atol=1e-18), step

    # zero gradient after the first step: the moments decay geometrically
    p, m, v = ow.adamw_step(p0, g, 0 * p0, 0 * p0, 1)
    m1, v1 = m, v
    for step in range(2, 6):
        p, m, v = ow.adamw_step(p, 0 * g, m, v, step)
        assert np.allclose(m, 0.9 ** (step - 1) * m1, rtol=1e-13)
        assert np.allclose(v, 0.999 ** (step - 1) * v1, rtol=1e-13)

    # without eps the step does not depend on the gradient's scale
    a = ow.adamw_step(p0, g, 0 * p0, 0 * p0, 1, eps=0.0, weight_decay=0.0)[0]
    b = ow.adamw_step(p0, 1e3 * g, 0 * p0, 0 * p0, 1, eps=0.0, weight_decay=0.0)[0]
    assert np.allclose(a, b, rtol=1e-14)


def test_adamw_pins():
    _pins(adamw_oracle)


MUTATIONS = {
    "no bias correction": ("m_hat = m_new / (1.0 - beta1 ** step)", "m_hat = m_new"),
    "bias correction one step late": ("v_hat = v_new / (1.0 - beta2 ** step)", "v_hat = v_new / (1.0 - beta2 ** (step + 1))"),
    "eps under the root": ("(np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps)"),
    "coupled decay": ("p = p * (1.0 - lr * weight_decay)", "g = g + weight_decay * p"),
    "betas swapped": ("m_new = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g",
                      "m_new = beta2 * np.asarray(m, dtype=np.float64) + (1.0 - beta2) * g"),
    "|g| for g^2": ("(1.0 - beta2) * (g * g)", "(1.0 - beta2) * np.abs(g)"),
    "decay with lr^2": ("p = p * (1.0 - lr * weight_decay)", "p = p * (1.0 - lr * lr * weight_decay)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_adamw_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(adamw_oracle)
    assert old in src, name
    mod = types.ModuleType("adamw_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "adamw_mutant", "exec"), mod.__dict__)
    with pytest.raises(Exception):
        _pins(mod)


def test_adamw_defaults_are_the_pages():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "pages_hyperparameters.json")) as f:
        pages = json.load(f)
    d = adamw_oracle.DEFAULTS
    assert d["lr"] == pages["adamw_lr"] and [d["beta1"], d["beta2"]] == pages["adamw_betas"]
    assert d["weight_decay"] == pages["adamw_weight_decay"] and d["eps"] == pages["adamw_eps"]
