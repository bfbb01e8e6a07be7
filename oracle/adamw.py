"""Oracle of the AdamW step of the symmetric (non-Muon) parameters, in float64 numpy.

TEST INFRASTRUCTURE ONLY: the tests and the benchmark's CPU-baseline leg use
this module; the GPU library does not.

What is computed follows the DMuon Training Guide:
  * "Step 4: Create Optimizer": the optimizer's second group (symmetric
    parameters) runs standard AdamW on all ranks, with adamw_lr 1e-3,
    adamw_betas (0.9, 0.999), adamw_weight_decay 0.01, adamw_eps 1e-8;
  * "Semantic Param Groups": each user group may carry its own AdamW lr,
    weight decay, betas and eps;
  * "Step 5: Training Loop": optimizer.step() runs AdamW on the routed
    parameters after the Muon group.

"Standard AdamW" is read as PyTorch's torch.optim.AdamW with its defaults
(no amsgrad, no maximize), step t counted from 1:
  p <- p * (1 - lr * wd)                       (decoupled weight decay)
  m <- beta1 * m + (1 - beta1) * g
  v <- beta2 * v + (1 - beta2) * g^2
  p <- p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
with m and v starting at zero.  A bf16 parameter is written by one
round-to-nearest-even of that value; m and v are kept in float64 here (the
library keeps them in fp32).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .muon import round_to_bf16

DEFAULTS = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def adamw_step(p, g, m, v, step: int, lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
               eps: float = 1e-8, weight_decay: float = 0.01) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One AdamW step of one tensor at step number ``step`` (>= 1).
    Returns (p_new, m_new, v_new) in float64."""
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m_new = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * (g * g)
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m_new, v_new


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """The value a parameter of ``dtype`` holds after one rounding."""
    if dtype == "bf16":
        return round_to_bf16(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
