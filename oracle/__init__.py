"""fp64 CPU oracle for the per-owner Muon step and its element-wise companions
(gradient clipping, AdamW) -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path
(``newton_schulz_06_amd``) never imports, links or calls it, and the two share
no code: the only module both sides read is ``workloads`` (seeded synthetic
inputs, none of the method's arithmetic).
"""
from .muon_ref import (  # noqa: F401
    QUINTIC,
    YOU_COEFFICIENTS,
    DEFAULT_EPS,
    coefficient_table,
    momentum_update,
    orient,
    frobenius_normalize,
    ns_iterate_left,
    ns_iterate_right,
    direct_newton_schulz,
    gram_windows,
    gram_newton_schulz_factors,
    gram_newton_schulz,
    gram_newton_schulz_distributed_local,
    muon_step,
    update_param,
    round_to_bf16,
)
from .optim_ref import (  # noqa: F401
    CLIP_EPS,
    ADAMW_DEFAULTS,
    total_norm,
    clip_grad_norm,
    adamw_step,
)
