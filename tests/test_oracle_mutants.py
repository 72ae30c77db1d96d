"""Plants plausible mistakes in copies of the oracle's steps (on the CPU) and
checks that the closed-form pins reject every one of them, while accepting
the oracle as written."""
import math

import numpy as np
import pytest

from oracle import muon_ref as ref

QT = ref.coefficient_table(None, 5)
YT = ref.coefficient_table(ref.YOU_COEFFICIENTS)


def _phi(x, table):
    for a, b, c in table:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _svd_ns(G, table, eps=1e-7):
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    return (U * _phi(s / (math.sqrt(float(s @ s)) + eps), table)) @ Vt


def _battery(ns, mom, step):
    """Return the names of the pins that fail for the given implementation."""
    bad = []
    rng = np.random.default_rng(7)
    for shape in [(9, 5), (7, 7), (5, 9)]:
        G = rng.standard_normal(shape) * 2.0
        for name, t in (("quintic", QT), ("you", YT)):
            try:
                got = ns(G, t)
                ok = got.shape == G.shape and np.max(np.abs(got - _svd_ns(G, t))) < 1e-10
            except Exception:
                ok = False
            if not ok:
                bad.append(f"svd{shape}{name}")
    b, u = mom(np.array([1.0]), np.array([2.0]), 0.5, True)
    if not (b[0] == 2.5 and u[0] == 3.25):
        bad.append("momentum-nesterov")
    b, u = mom(np.array([1.0]), np.array([2.0]), 0.5, False)
    if not (b[0] == 2.5 and u[0] == 2.5):
        bad.append("momentum-plain")
    p = rng.standard_normal((4, 6)); g = rng.standard_normal((4, 6))
    buf = rng.standard_normal((4, 6))
    newp, _, O = step(p, g, buf)
    _, uu = ref.momentum_update(buf, g, 0.95, True)
    if np.max(np.abs(newp - (p * (1 - 0.02 * 0.1) - 0.02 * _svd_ns(uu, QT)))) > 1e-12:
        bad.append("update")
    return bad


def _ns_with(iterate=ref.ns_iterate_left, normalize=ref.frobenius_normalize,
             untranspose=True):
    def ns(G, table):
        X, t = ref.orient(G)
        X = iterate(normalize(X), table)
        return X.T if (t and untranspose) else X
    return ns


def _step_with(ns=None, sign=-1.0):
    ns = ns or _ns_with()

    def step(p, g, buf):
        nb, u = ref.momentum_update(buf, g, 0.95, True)
        O = ns(u, QT)
        return p - 0.02 * 0.1 * p + sign * 0.02 * O, nb, O
    return step


def _iter_drop_c(X, table):
    for a, b, c in table:
        A = X @ X.T
        X = a * X + (b * A) @ X
    return X


def _iter_sign_c(X, table):
    for a, b, c in table:
        A = X @ X.T
        X = a * X + (b * A - c * (A @ A)) @ X
    return X


def _iter_right_mult(X, table):
    for a, b, c in table:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + X @ B   # raises for non-square X
    return X


def _iter_reversed(X, table):
    return ref.ns_iterate_left(X, list(reversed(table)))


def _iter_one_short(X, table):
    return ref.ns_iterate_left(X, table[:-1])


def _norm_squared(X, eps=1e-7):
    return X / (np.sum(X * X) + eps)


def _norm_max(X, eps=1e-7):
    return X / (np.abs(X).max() + eps)


def _mom_old_buf(buf, g, mu, nesterov):
    nb = mu * buf + g
    return nb, (g + mu * buf if nesterov else nb)


def _mom_sign(buf, g, mu, nesterov):
    nb = mu * buf + g
    return nb, (g - mu * nb if nesterov else nb)


def _mom_dampened(buf, g, mu, nesterov):
    nb = mu * buf + (1 - mu) * g
    return nb, (g + mu * nb if nesterov else nb)


def _oracle_ns(G, t):
    return ref.direct_newton_schulz(G, coefficients=t)


def _oracle_step(p, g, buf):
    return ref.muon_step(p, g, buf, weight_decay=0.1, nesterov=True)


def test_oracle_as_written_passes_battery():
    assert _battery(_oracle_ns, ref.momentum_update, _oracle_step) == []


MUTANTS = {
    "dropped c term": dict(ns=_ns_with(iterate=_iter_drop_c)),
    "wrong sign on c": dict(ns=_ns_with(iterate=_iter_sign_c)),
    "B applied on the right (square)": dict(ns=_ns_with(iterate=_iter_right_mult)),
    "coefficients reversed": dict(ns=_ns_with(iterate=_iter_reversed)),
    "one step short": dict(ns=_ns_with(iterate=_iter_one_short)),
    "eps on squared norm": dict(ns=_ns_with(normalize=_norm_squared)),
    "max-abs normalizer": dict(ns=_ns_with(normalize=_norm_max)),
    "tall result not transposed back": dict(ns=_ns_with(untranspose=False)),
    "lookahead on old buffer": dict(mom=_mom_old_buf),
    "lookahead sign": dict(mom=_mom_sign),
    "dampened momentum": dict(mom=_mom_dampened),
    "update sign": dict(step=_step_with(sign=+1.0)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_battery_rejects_mutant(name):
    m = MUTANTS[name]
    bad = _battery(m.get("ns", _oracle_ns), m.get("mom", ref.momentum_update),
                   m.get("step", _oracle_step))
    assert bad, f"mutant '{name}' slipped through every pin"
