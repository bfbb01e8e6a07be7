"""Seeded synthetic inputs for the owner-side Muon step.

This module is shared by the oracle's tests and by the GPU path's tests and
benchmark.  It holds workload descriptions (shapes, dtypes, distributions,
step counts, hyperparameters) and seeded random generators, and nothing of
the optimizer's own arithmetic.

Workloads
---------
The pages (DMuon Training Guide and Integration Recipes) train Llama-style
decoder stacks; the Integration Recipes page loads Llama-3.2-3B in bf16.  No
weights or data are used here: every tensor is drawn from a seeded normal
distribution with the shapes of those models' projection matrices, stored
PyTorch-Linear style as (out_features, in_features).

Seeding
-------
Every tensor has its own stream: ``numpy.random.SeedSequence([seed, cfg,
matrix, kind, step])`` feeding PCG64, drawn in float64 and rounded to the
storage dtype (float32: numpy's round-to-nearest-even cast; bfloat16: round
the float32 value to nearest, ties to even).  The rounded values are the
exact inputs of both the GPU path and the oracle.

For full-size benchmark runs, where drawing billions of values on the host is
too slow, ``torch_normal_`` fills a device tensor from a seeded torch
generator instead; those inputs have the same distributions but are not the
numpy streams.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# tensor kinds, used as one coordinate of the seed
KIND_PARAM = 0
KIND_GRAD = 1
KIND_GRAD_SCALE = 2
KIND_SHAPE = 3

# quintic coefficients of the small single-matrix workload (the pages print
# none; this workload fixes them)
QUINTIC = (3.4445, -4.7750, 2.0315)


@dataclasses.dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int
    cols: int


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a batch of owned matrices and how to fill it."""
    index: int
    name: str
    matrices: Tuple[MatrixSpec, ...]
    param_dtype: str            # "f32" | "bf16"
    grad_dtype: str             # "f32" | "bf16"
    steps: int
    ns_precisions: Tuple[str, ...]   # NS modes exercised: "bf16" and/or "f32"
    ns_backends: Tuple[str, ...]     # "gram" and/or "direct"
    lr: float = 0.02
    momentum: float = 0.95
    nesterov: bool = True
    ns_steps: int = 5
    weight_decay: float = 0.0
    param_std: float = 0.02
    grad_std: float = 1e-3
    grad_lognormal_sigma: float = 0.0   # per-matrix log-normal grad scale

    @property
    def numel(self) -> int:
        return sum(m.rows * m.cols for m in self.matrices)

    def hparams(self, ns_backend: Optional[str] = None,
                ns_precision: Optional[str] = None) -> dict:
        return dict(lr=self.lr, momentum=self.momentum, nesterov=self.nesterov,
                    ns_steps=self.ns_steps, weight_decay=self.weight_decay,
                    ns_backend=ns_backend or self.ns_backends[0],
                    ns_precision=ns_precision or self.ns_precisions[0],
                    ns_coeffs=None, eps=1e-7)


def decoder_layer(hidden: int, ffn: int, q_heads: int, kv_heads: int,
                  head_dim: int, prefix: str = "") -> List[MatrixSpec]:
    """The seven projection matrices of one Llama-style decoder layer."""
    q = q_heads * head_dim
    kv = kv_heads * head_dim
    return [
        MatrixSpec(prefix + "q_proj", q, hidden),
        MatrixSpec(prefix + "k_proj", kv, hidden),
        MatrixSpec(prefix + "v_proj", kv, hidden),
        MatrixSpec(prefix + "o_proj", hidden, q),
        MatrixSpec(prefix + "gate_proj", ffn, hidden),
        MatrixSpec(prefix + "up_proj", ffn, hidden),
        MatrixSpec(prefix + "down_proj", hidden, ffn),
    ]


RAGGED_SHAPES = ((128, 2048), (2048, 128), (512, 4096), (4096, 512),
                 (1024, 1024), (4096, 4096), (14336, 4096))


def ragged_shape_draw(seed: int = 0, count: int = 96) -> List[int]:
    """Shape indices of the ragged batch: uniform over RAGGED_SHAPES."""
    return [int(i) for i in np.random.default_rng(seed).integers(0, len(RAGGED_SHAPES), count)]


def _layers(n_layers: int, **kw) -> Tuple[MatrixSpec, ...]:
    out: List[MatrixSpec] = []
    for layer in range(n_layers):
        out += decoder_layer(prefix=f"layers.{layer}.", **kw)
    return tuple(out)


_L3B = dict(hidden=3072, ffn=8192, q_heads=24, kv_heads=8, head_dim=128)
_L8B = dict(hidden=4096, ffn=14336, q_heads=32, kv_heads=8, head_dim=128)


def workload(index: int, seed: int = 0) -> Workload:
    """The five synthetic workloads, by index (0 is the small oracle-sized one)."""
    if index == 0:
        return Workload(0, "single fp32 256x512", (MatrixSpec("w", 256, 512),),
                        "f32", "f32", steps=1, ns_precisions=("bf16", "f32"),
                        ns_backends=("gram", "direct"), grad_std=1e-2)
    if index == 1:
        return Workload(1, "3B decoder layer (hidden 3072, ffn 8192, 24q/8kv x128)",
                        _layers(1, **_L3B), "bf16", "bf16", steps=10,
                        ns_precisions=("bf16",), ns_backends=("gram",))
    if index == 2:
        return Workload(2, "3B 28-layer stack (196 matrices)", _layers(28, **_L3B),
                        "bf16", "bf16", steps=5, ns_precisions=("bf16",),
                        ns_backends=("gram", "direct"))
    if index == 3:
        return Workload(3, "8B layers 0-3 (hidden 4096, ffn 14336, 32q/8kv x128)",
                        _layers(4, **_L8B), "bf16", "bf16", steps=5,
                        ns_precisions=("bf16",), ns_backends=("gram",),
                        weight_decay=0.1)
    if index == 4:
        idx = ragged_shape_draw(seed)
        mats = tuple(MatrixSpec(f"m{i}", *RAGGED_SHAPES[k]) for i, k in enumerate(idx))
        return Workload(4, "ragged 96 matrices", mats, "bf16", "bf16", steps=3,
                        ns_precisions=("bf16", "f32"), ns_backends=("gram",),
                        grad_lognormal_sigma=1.0)
    raise ValueError(f"no workload {index}")


N_WORKLOADS = 5


# ---------------------------------------------------------------------------
# rounding of generated values to their storage dtype
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.
    NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """Round float64 draws to the storage dtype.

    Returns (raw, exact): ``raw`` is the array to upload (float32, or uint16
    bf16 bit patterns) and ``exact`` its values as float64."""
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# seeded streams
# ---------------------------------------------------------------------------

def rng_for(seed: int, cfg: int, mat: int, kind: int, step: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, mat, kind, step])))


def grad_scale(w: Workload, mat: int, seed: int = 0) -> float:
    """Per-matrix gradient standard deviation (log-normal spread if asked)."""
    if w.grad_lognormal_sigma <= 0:
        return w.grad_std
    z = rng_for(seed, w.index, mat, KIND_GRAD_SCALE, 0).standard_normal()
    return w.grad_std * math.exp(w.grad_lognormal_sigma * z)


def param_init(w: Workload, mat: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Initial parameter of matrix ``mat``: N(0, param_std^2), storage-rounded."""
    s = w.matrices[mat]
    x = rng_for(seed, w.index, mat, KIND_PARAM, 0).standard_normal((s.rows, s.cols))
    return to_storage(w.param_std * x, w.param_dtype)


def grad_at(w: Workload, mat: int, step: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Gradient of matrix ``mat`` at step ``step`` (fresh draw every step)."""
    s = w.matrices[mat]
    x = rng_for(seed, w.index, mat, KIND_GRAD, step).standard_normal((s.rows, s.cols))
    return to_storage(grad_scale(w, mat, seed) * x, w.grad_dtype)


def normal_matrix(rows: int, cols: int, std: float, dtype: str, seed: int,
                  tag: Sequence[int] = ()) -> Tuple[np.ndarray, np.ndarray]:
    """A free-standing seeded normal matrix for unit tests of single stages."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99, *tag])))
    return to_storage(std * rng.standard_normal((rows, cols)), dtype)


def torch_normal_(t, std: float, seed: int) -> None:
    """Fill a (device) torch tensor in place from a seeded torch generator,
    N(0, std^2), for benchmark-size inputs."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    if t.dtype in (torch.float32,):
        t.normal_(0.0, std, generator=g)
    else:
        tmp = torch.empty(t.shape, dtype=torch.float32, device=t.device)
        tmp.normal_(0.0, std, generator=g)
        t.copy_(tmp)
