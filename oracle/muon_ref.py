"""Plain, slow, fp64 CPU oracle of the per-owner Muon step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use it.  It shares no code with the HIP library.

What it computes, for each owned 2D matrix (sources are the DMuon
documentation pages; readings of unstated points are marked READING):

1. momentum (DMuon "API Reference", ``Muon``: the ``momentum`` argument and
   the ``nesterov`` argument, whose lookahead input is the gradient plus
   momentum times the buffer).
   READING: the buffer recursion is ``buf <- mu*buf + g`` with no dampening,
   and the Nesterov lookahead uses the buffer *after* this update.
2. orientation (DMuon "API Reference", ``gram_newton_schulz_factors``: NS
   may operate on the transpose of the normalized G).
   READING: transpose iff rows > cols; square matrices are not transposed.
3. normalization (same section: the normalizer is the Frobenius norm of G
   plus eps; ``direct_newton_schulz`` default eps = 1e-7).
4. direct Newton-Schulz (DMuon "API Reference", ``direct_newton_schulz``:
   X_{k+1} = a_k X + b_k (X X^T) X + c_k (X X^T)^2 X, one (a, b, c) per
   step, the list length is the number of steps).
   READING: the pages name but do not print the direct form's default
   coefficients; the standard quintic (3.4445, -4.7750, 2.0315) is used at
   every step.  YOU_COEFFICIENTS are printed on the same page and are the
   second table used here.
5. Gram-space NS (DMuon "API Reference", ``gram_newton_schulz`` and
   ``gram_newton_schulz_factors``: iterate on the Gram matrix instead of the
   full matrix, with per-step coefficients and restarts (default ``[2]``);
   the result is the normalized, oriented G left-multiplied by one Gram
   factor per restart window).
   READING: the pages give no formulas.  The iteration of step 4,
   X_{k+1} = P_k X_k with P_k = a I + b A_k + c A_k^2 and A_k = X_k X_k^T, is
   carried in Gram space: within a window starting at X_s, A_s = X_s X_s^T,
   Q accumulates P_k Q and A_{k+1} = P_k A_k P_k (P_k is symmetric); at the
   window's end X <- Q X_s.  A restart at step r starts a new window there
   (restart indices outside 1..steps-1 have no effect).  Exactly equal to
   step 4 in exact arithmetic.
6. Gram-space NS on a local shard (DMuon "API Reference",
   ``gram_newton_schulz_distributed_local`` and its ``_batched`` variant:
   orientation comes from the full logical matrix through the
   ``transposed`` argument; the oriented local block is a column block of
   the full oriented matrix; only the small Gram matrix is rebuilt by an
   all-reduce over the shard group; each rank gets its block of the full
   output and momentum / scaling / weight decay stay with the caller).
   READING: the Frobenius norm is needed before the first Gram factor and
   is also a sum over the shards, so it is reduced too; every reduction is
   a plain sum over the group, and each restart window reduces the Gram
   matrix of the current X once.  The oracle stands for the whole group at
   once: it takes every rank's block and writes each all-reduce as a sum
   over the list.
7. update (DMuon "HSDP Training (Multi-Node)", "What Happens Under the Hood":
   the owner runs NS + momentum + weight decay + update; "API Reference",
   ``Muon`` signature: lr=0.02, momentum=0.95, weight_decay=0.0).
   READING: decoupled weight decay ``p <- p - lr*wd*p - lr*O`` on the
   pre-update p, with no shape-dependent lr factor (none is printed).

Every function works on numpy float64; inputs in float32 / bfloat16 are
upcast exactly.  No blocking, fusion or reordering beyond the definitions.
"""
from __future__ import annotations

import numpy as np

# Standard quintic used when the pages leave the direct form's coefficients
# unstated (READING above).
QUINTIC = (3.4445, -4.7750, 2.0315)

# DMuon "API Reference", YOU_COEFFICIENTS (5 per-step (a, b, c) triples).
YOU_COEFFICIENTS = (
    (4.0848, -6.8946, 2.927),
    (3.9505, -6.3029, 2.6377),
    (3.7418, -5.5913, 2.3037),
    (2.8769, -3.1427, 1.2046),
    (2.8366, -3.0525, 1.2012),
)

# DMuon "API Reference", direct_newton_schulz signature: eps=1e-07.
DEFAULT_EPS = 1e-7


def coefficient_table(coefficients=None, ns_steps: int = 5):
    """Per-step (a, b, c) list.

    DMuon "API Reference", ``direct_newton_schulz``: ``steps`` is used only
    when no coefficient list is given; otherwise the list length is the step
    count.  With no list, the quintic is repeated ``ns_steps`` times.
    """
    if coefficients is None:
        return [tuple(float(v) for v in QUINTIC)] * int(ns_steps)
    table = [tuple(float(v) for v in row) for row in coefficients]
    for row in table:
        if len(row) != 3:
            raise ValueError("each coefficient row must be (a, b, c)")
    return table


def momentum_update(buf, grad, momentum: float, nesterov: bool):
    """Momentum buffer update and NS input.

    DMuon "API Reference", ``Muon`` › ``nesterov``: the NS input is
    ``grad + mu * buf`` when Nesterov is on.  READING: ``buf`` is first
    updated to ``mu*buf + grad``; without Nesterov the NS input is the
    updated buffer itself.

    Returns ``(new_buf, ns_input)`` in float64.
    """
    b = np.asarray(buf, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64)
    new_buf = momentum * b + g
    if nesterov:
        u = g + momentum * new_buf
    else:
        u = new_buf.copy()
    return new_buf, u


def orient(M):
    """Return ``(X, transposed)``: X is M, or M^T when M has more rows than
    columns (DMuon "API Reference", ``gram_newton_schulz_factors``: NS may
    act on the transposed matrix; READING: transpose iff rows > cols)."""
    M = np.asarray(M, dtype=np.float64)
    if M.ndim != 2:
        raise ValueError("Newton-Schulz needs a 2D matrix")
    transposed = M.shape[0] > M.shape[1]
    return (M.T if transposed else M), transposed


def frobenius_normalize(X, eps: float = DEFAULT_EPS):
    """X / (||X||_F + eps) (DMuon "API Reference",
    ``gram_newton_schulz_factors`` › Returns: the normalizer is the norm of
    G plus eps)."""
    X = np.asarray(X, dtype=np.float64)
    return X / (np.linalg.norm(X) + eps)


def ns_iterate_left(X, coefficients):
    """Direct NS on the oriented, normalized X (rows <= cols).

    DMuon "API Reference", ``direct_newton_schulz``:
    X <- a X + b (X X^T) X + c (X X^T)^2 X, written with A = X X^T and
    B = b A + c A A as X <- a X + B X.
    """
    X = np.asarray(X, dtype=np.float64)
    for a, b, c in coefficients:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def ns_iterate_right(X, coefficients):
    """The same polynomial applied from the right:
    X <- a X + X (b X^T X + c (X^T X)^2).

    Equal to :func:`ns_iterate_left` in exact arithmetic (both are
    a X + b X X^T X + c X X^T X X^T X); kept only so tests can check the
    left form against an independent evaluation order.
    """
    X = np.asarray(X, dtype=np.float64)
    for a, b, c in coefficients:
        S = X.T @ X
        X = a * X + X @ (b * S + c * (S @ S))
    return X


def direct_newton_schulz(G, steps: int = 5, eps: float = DEFAULT_EPS,
                         coefficients=None):
    """Orthogonalize G: orient, normalize, iterate, undo the orientation.

    DMuon "API Reference", ``direct_newton_schulz``: same shape as G.  The
    result here is float64; callers round to their storage dtype.
    """
    table = coefficient_table(coefficients, steps)
    X, transposed = orient(G)
    X = frobenius_normalize(X, eps)
    X = ns_iterate_left(X, table)
    return X.T if transposed else X


def gram_windows(n_steps: int, restart_iterations=None):
    """[start, end) step ranges between restarts (default restart at 2)."""
    restarts = [2] if restart_iterations is None else [int(r) for r in restart_iterations]
    if any(r < 0 for r in restarts):
        raise ValueError("restart indices are >= 0")
    cuts = sorted({0, n_steps} | {r for r in restarts if 0 < r < n_steps})
    return list(zip(cuts[:-1], cuts[1:]))


def gram_newton_schulz_factors(G, steps: int = 5, eps: float = DEFAULT_EPS, coefficients=None,
                               restart_iterations=None):
    """Gram-space NS factors of G: ``(segments, transposed, normalizer)``.

    DMuon "API Reference", ``gram_newton_schulz_factors``: one Gram factor
    per restart window, applied in order from the left to the normalized,
    oriented G; the normalizer is ||G||_F + eps (READING in the header).
    """
    table = coefficient_table(coefficients, steps)
    X, transposed = orient(G)
    normalizer = float(np.linalg.norm(X)) + eps
    X = X / normalizer
    p = X.shape[0]
    segments = []
    for s, e in gram_windows(len(table), restart_iterations):
        A = X @ X.T
        Q = np.eye(p)
        for k in range(s, e):
            a, b, c = table[k]
            P = a * np.eye(p) + b * A + c * (A @ A)
            Q = P @ Q
            A = P @ A @ P
        segments.append(Q)
        X = Q @ X
    return tuple(segments), transposed, normalizer


def gram_newton_schulz(G, steps: int = 5, eps: float = DEFAULT_EPS, coefficients=None,
                       restart_iterations=None):
    """Gram-space NS of G (DMuon "API Reference", ``gram_newton_schulz``):
    the factors of :func:`gram_newton_schulz_factors` applied to the
    normalized, oriented G; same shape as G, float64."""
    segments, transposed, normalizer = gram_newton_schulz_factors(
        G, steps, eps, coefficients, restart_iterations)
    X, _ = orient(G)
    X = X / normalizer
    for Q in segments:
        X = Q @ X
    return X.T if transposed else X


def gram_newton_schulz_distributed_local(shards, transposed: bool, steps: int = 5,
                                         eps: float = DEFAULT_EPS, coefficients=None,
                                         restart_iterations=None):
    """Gram-space NS of a matrix held as column shards of its oriented view
    (DMuon "API Reference", ``gram_newton_schulz_distributed_local``;
    READING 6 in the header).

    ``shards`` lists every rank's local block in the stored layout; with
    ``transposed`` its transpose is the rank's column block X_r (p x q_r) of
    the oriented matrix, else the block itself is.  Every rank's result is
    returned, each in its block's layout, float64.
    """
    table = coefficient_table(coefficients, steps)
    blocks = [np.asarray(g, dtype=np.float64) for g in shards]
    Xs = [B.T if transposed else B for B in blocks]
    p = Xs[0].shape[0]
    if any(X.shape[0] != p for X in Xs):
        raise ValueError("every oriented shard has the full matrix's p rows")
    # all-reduce of the squared norm, then every rank scales its block
    normalizer = np.sqrt(sum(float(np.sum(X * X)) for X in Xs)) + eps
    Xs = [X / normalizer for X in Xs]
    for s, e in gram_windows(len(table), restart_iterations):
        A = sum(X @ X.T for X in Xs)  # all-reduce of the local Gram matrices
        Q = np.eye(p)
        for k in range(s, e):
            a, b, c = table[k]
            P = a * np.eye(p) + b * A + c * (A @ A)
            Q = P @ Q
            A = P @ A @ P
        Xs = [Q @ X for X in Xs]
    return [X.T if transposed else X for X in Xs]


def muon_step(param, grad, buf, *, lr: float = 0.02, momentum: float = 0.95,
              weight_decay: float = 0.0, nesterov: bool = True,
              ns_steps: int = 5, coefficients=None, eps: float = DEFAULT_EPS):
    """One Muon step on one owned matrix.

    Momentum (see :func:`momentum_update`), NS of the momentum output
    (:func:`direct_newton_schulz`), then the update
    ``p <- p - lr*wd*p - lr*O`` (READING: decoupled weight decay on the
    pre-update p, no shape factor).  Defaults follow the ``Muon`` signature
    in DMuon "API Reference".

    Returns ``(new_param, new_buf, O)``, all float64.
    """
    new_buf, u = momentum_update(buf, grad, momentum, nesterov)
    O = direct_newton_schulz(u, steps=ns_steps, eps=eps,
                             coefficients=coefficients)
    return update_param(param, O, lr, weight_decay), new_buf, O


def update_param(param, O, lr: float, weight_decay: float = 0.0):
    """The weight update of a Muon step: ``p - lr*wd*p - lr*O`` in float64
    (READING: decoupled weight decay on the pre-update p, no shape-dependent
    factor on the lr; DMuon "HSDP Training (Multi-Node)", What Happens Under
    the Hood: the owner applies weight decay and the update)."""
    p = np.asarray(param, dtype=np.float64)
    return p - lr * weight_decay * p - lr * O


_BF16_DROP = 45  # fp64 keeps 52 explicit mantissa bits, bf16 keeps 7


def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Works on the float64 bit pattern (no detour through float32, so there is
    no double rounding).  Valid for finite values inside bfloat16's normal
    range; anything else raises, since no test here needs it.
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    mag = np.abs(x)
    if not finite.all():
        raise ValueError("round_to_bf16: non-finite input")
    nz = mag[mag != 0]
    if nz.size and (nz.min() < 2.0 ** -126 or nz.max() >= 3.3e38):
        raise ValueError("round_to_bf16: value outside bfloat16 normal range")
    bits = x.view(np.uint64)
    keep = (bits >> np.uint64(_BF16_DROP)) & np.uint64(1)
    half = np.uint64((1 << (_BF16_DROP - 1)) - 1)
    rounded = (bits + half + keep) & ~np.uint64((1 << _BF16_DROP) - 1)
    return rounded.view(np.float64)
