"""Plain fp64 CPU oracle of the two element-wise companions of the Muon step:
gradient-norm clipping of the Muon gradients, and the AdamW update of the
parameters Muon does not own.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use it.  It shares no code with the HIP library.

1. Clipping (DMuon "API Reference", ``Muon.clip_grad_norm_`` and the free
   function ``clip_grad_norm_``: clip only the Muon gradients, norm_type 2.0
   by default, returning the pre-clip total norm, the coefficient, whether it
   clipped and whether the norm was non-finite; ``clip_grad_norm_buckets_``:
   every bucket keeps its own norm and coefficient).
   READING: the pages print no formula; the one PyTorch's
   ``clip_grad_norm_`` uses (which the same section tells users to keep for
   ordinary parameters) is taken: total = (sum |g|^p)^(1/p) over the
   bucket (p = inf: max |g|), coef = max_norm / (total + 1e-6), every
   gradient multiplied by min(coef, 1); ``max_norm`` None only measures.
   A NaN anywhere makes the total NaN (also for p = inf).
2. AdamW (DMuon "API Reference", ``Muon``: ``step`` runs AdamW on the
   parameters that are not Muon's; the signature's adamw_lr=1e-3,
   adamw_betas=(0.9, 0.999), adamw_weight_decay=0.01, adamw_eps=1e-8).
   READING: the pages name AdamW without its formula; the decoupled form of
   ``torch.optim.AdamW`` is taken: p <- p (1 - lr wd); m <- b1 m + (1-b1) g;
   v <- b2 v + (1-b2) g^2; p <- p - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps),
   with t the 1-based step count.
"""
from __future__ import annotations

import math

import numpy as np

CLIP_EPS = 1e-6  # added to the total norm before dividing (PyTorch convention)
ADAMW_DEFAULTS = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.01}


def total_norm(grads, norm_type: float = 2.0) -> float:
    """The p-norm of all entries of ``grads`` taken together (one bucket)."""
    flat = [np.abs(np.asarray(g, dtype=np.float64)).ravel() for g in grads]
    if not flat:
        return 0.0
    a = np.concatenate(flat)
    if a.size == 0:
        return 0.0
    if np.isnan(a).any():
        return float("nan")
    if math.isinf(norm_type):
        return float(a.max())
    return float(np.sum(a ** norm_type) ** (1.0 / norm_type))


def clip_grad_norm(grads, max_norm, norm_type: float = 2.0, buckets=None):
    """Clip a list of gradients in place of the caller: returns the scaled
    gradients (float64) and one stats dict per bucket.

    ``buckets`` gives each gradient's bucket index (None: one bucket).  A
    bucket's stats: total_norm, clip_coef (max_norm / (total + 1e-6), or 1.0
    when max_norm is None), clipped (coef < 1), found_inf (total not finite)
    and param_count (number of elements).
    """
    grads = [np.asarray(g, dtype=np.float64) for g in grads]
    if buckets is None:
        buckets = [0] * len(grads)
    nb = (max(buckets) + 1) if buckets else 0
    stats = []
    out = [g.copy() for g in grads]
    for b in range(nb):
        members = [i for i, k in enumerate(buckets) if k == b]
        tot = total_norm([grads[i] for i in members], norm_type)
        if max_norm is None:
            coef = 1.0
        else:
            coef = max_norm / (tot + CLIP_EPS)
            scale = min(coef, 1.0) if not math.isnan(coef) else coef
            for i in members:
                out[i] = grads[i] * scale
        stats.append({"total_norm": tot, "clip_coef": coef, "clipped": bool(coef < 1.0),
                      "found_inf": not math.isfinite(tot),
                      "param_count": int(sum(grads[i].size for i in members))})
    return out, stats


def adamw_step(param, grad, exp_avg, exp_avg_sq, step: int, lr: float = 1e-3,
               beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
               weight_decay: float = 0.01):
    """One AdamW update of one tensor (``step`` is the 1-based count after
    this update).  Returns (param, exp_avg, exp_avg_sq) in float64."""
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(param, dtype=np.float64) * (1.0 - lr * weight_decay)
    g = np.asarray(grad, dtype=np.float64)
    m = beta1 * np.asarray(exp_avg, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(exp_avg_sq, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
