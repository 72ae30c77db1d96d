"""Pins for the fp64 oracle of Gram-space Newton-Schulz, against facts that do
not come from the oracle: the SVD closed form of the NS polynomial (every
restart placement must give it), the structure of the returned factors, and
hand cases.  Plausible slips planted in copies of the Gram iteration must
fail at least one pin.
"""
import math

import numpy as np
import pytest

import oracle
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


RESTARTS = [None, [], [1], [2], [1, 3], [4], [0, 9], [1, 2, 3, 4]]


@pytest.mark.parametrize("shape", [(9, 23), (23, 9), (16, 16), (1, 5), (6, 1)])
@pytest.mark.parametrize("coef", ["quintic", "you"])
def test_gram_matches_svd_closed_form_for_any_restarts(shape, coef):
    table = QT if coef == "quintic" else YT
    G = np.random.default_rng(sum(shape)).standard_normal(shape) * 3.0
    want = _svd_ns(G, table)
    for r in RESTARTS:
        got = oracle.gram_newton_schulz(G, coefficients=table, restart_iterations=r)
        assert got.shape == G.shape
        assert np.max(np.abs(got - want)) <= 1e-12, (shape, coef, r)


def test_windows():
    assert oracle.gram_windows(5) == [(0, 2), (2, 5)]
    assert oracle.gram_windows(5, []) == [(0, 5)]
    assert oracle.gram_windows(5, [0, 5, 7]) == [(0, 5)]
    assert oracle.gram_windows(5, [3, 1]) == [(0, 1), (1, 3), (3, 5)]
    with pytest.raises(ValueError):
        oracle.gram_windows(5, [-1])


def test_factors_structure():
    G = np.random.default_rng(3).standard_normal((30, 12)) + 0.5
    segs, transposed, nrm = oracle.gram_newton_schulz_factors(G, restart_iterations=[2])
    assert transposed and len(segs) == 2
    assert nrm == pytest.approx(np.linalg.norm(G) + 1e-7, rel=1e-15)
    X = G.T / (np.linalg.norm(G) + 1e-7)
    A0 = X @ X.T
    for Q in segs:
        assert Q.shape == (12, 12)
        assert np.max(np.abs(Q - Q.T)) <= 1e-12 * np.max(np.abs(Q))
    # the first factor is a polynomial in A0, so it commutes with it
    assert np.max(np.abs(segs[0] @ A0 - A0 @ segs[0])) <= 1e-12 * np.max(np.abs(segs[0]))
    for Q in segs:
        X = Q @ X
    assert np.allclose(X.T, oracle.gram_newton_schulz(G), rtol=0, atol=1e-14)


def test_zero_matrix_gives_zero():
    assert np.array_equal(oracle.gram_newton_schulz(np.zeros((4, 7))), np.zeros((4, 7)))


def _gram_variant(a_update="PAP", square=True, accumulate=True, untranspose=True):
    def ns(G, table, restarts):
        X, t = ref.orient(G)
        X = X / (np.linalg.norm(X) + 1e-7)
        p = X.shape[0]
        for s, e in ref.gram_windows(len(table), restarts):
            A = X @ X.T
            Q = np.eye(p)
            for k in range(s, e):
                a, b, c = table[k]
                P = a * np.eye(p) + b * A + c * (A @ A if square else A)
                Q = P @ Q if accumulate else P
                A = P @ A @ P if a_update == "PAP" else P @ A
            X = Q @ X
        return X.T if (t and untranspose) else X
    return ns


MUTANTS = {
    "A <- P A": _gram_variant(a_update="PA"),
    "no square": _gram_variant(square=False),
    "Q not accumulated": _gram_variant(accumulate=False),
    "no transpose back": _gram_variant(untranspose=False),
}


def _battery(ns):
    bad = []
    for shape in [(9, 23), (23, 9)]:
        G = np.random.default_rng(5).standard_normal(shape)
        for r in ([2], [], [1, 3]):
            try:
                got = ns(G, QT, r)
                ok = got.shape == G.shape and np.max(np.abs(got - _svd_ns(G, QT))) <= 1e-12
            except Exception:
                ok = False
            if not ok:
                bad.append(f"{shape}{r}")
    return bad


def test_oracle_passes_battery():
    assert _battery(lambda G, t, r: oracle.gram_newton_schulz(G, coefficients=t,
                                                              restart_iterations=r)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_battery_rejects_mutant(name):
    assert _battery(MUTANTS[name]) != []
