"""Test infrastructure: a plain, slow CPU oracle of the owner-side Muon step.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The GPU library never imports, calls or links it, and it
shares no code with the GPU library.
"""
from .muon import (  # noqa: F401
    DEFAULT_COEFFS,
    momentum_update,
    frobenius_norm,
    normalize,
    ns_direct,
    ns_gram,
    orthogonalize,
    lr_scale,
    apply_update,
    round_to_bf16,
    muon_step,
)
