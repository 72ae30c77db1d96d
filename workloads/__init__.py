"""Seeded synthetic inputs shared by the oracle's tests, the GPU tests and the
benchmark.

This package holds shapes, hyperparameters and random-number recipes only;
none of the Muon / Newton-Schulz arithmetic lives here.  Both the fp64
oracle and the HIP path read their inputs from it.
"""
from .synth import (  # noqa: F401
    BY_NAME,
    CONFIGS,
    OP_CONFIGS,
    Config,
    c4_shapes,
    grad_np,
    param_np,
    powerlaw_basis_np,
    grad_torch,
    param_torch,
    seed_words,
)
