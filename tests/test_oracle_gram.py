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


# --- Gram-space NS on column shards of the oriented matrix -----------------

def _split(G, transposed, widths):
    """Blocks of G along the oriented matrix's columns: row blocks of the
    stored G when transposed, column blocks otherwise."""
    cuts = np.cumsum([0] + list(widths))
    if transposed:
        return [G[a:b, :] for a, b in zip(cuts[:-1], cuts[1:])]
    return [G[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]


def _join(blocks, transposed):
    return np.concatenate(blocks, axis=0 if transposed else 1)


LOCAL_CASES = [
    # (stored shape, transposed, oriented column widths of the shards)
    ((9, 23), False, [23]),
    ((9, 23), False, [8, 8, 7]),
    ((9, 23), False, [1, 20, 2]),
    ((23, 9), True, [23]),
    ((23, 9), True, [5, 5, 5, 8]),
    ((16, 16), False, [4, 12]),
    ((16, 16), True, [10, 6]),
    ((23, 9), False, [3, 6]),    # forced orientation: the tall side is p
    ((9, 23), True, [4, 5]),     # forced orientation: the wide side is p
    ((1, 5), False, [2, 3]),
    ((6, 1), True, [6]),
]


@pytest.mark.parametrize("shape,transposed,widths", LOCAL_CASES)
@pytest.mark.parametrize("coef", ["quintic", "you"])
def test_local_shards_join_to_svd_closed_form(shape, transposed, widths, coef):
    table = QT if coef == "quintic" else YT
    G = np.random.default_rng(sum(shape) + len(widths)).standard_normal(shape) * 2.0
    want = _svd_ns(G, table)
    for r in (None, [], [1, 3], [1, 2, 3, 4]):
        outs = oracle.gram_newton_schulz_distributed_local(
            _split(G, transposed, widths), transposed, coefficients=table, restart_iterations=r)
        assert [o.shape for o in outs] == [b.shape for b in _split(G, transposed, widths)]
        assert np.max(np.abs(_join(outs, transposed) - want)) <= 1e-12, (shape, widths, r)


def test_local_single_shard_equals_gram_ns():
    G = np.random.default_rng(8).standard_normal((12, 30))
    (got,) = oracle.gram_newton_schulz_distributed_local([G], False, restart_iterations=[1, 3])
    assert np.array_equal(got.shape, G.shape)
    assert np.max(np.abs(got - oracle.gram_newton_schulz(G, restart_iterations=[1, 3]))) <= 1e-13


def test_local_rejects_mismatched_p():
    with pytest.raises(ValueError):
        oracle.gram_newton_schulz_distributed_local([np.ones((3, 4)), np.ones((4, 4))], False)


def _local_variant(reduce_norm=True, reduce_gram=True, rereduce=True, orient_shards=True):
    def ns(shards, transposed, table, restarts):
        Xs = [np.asarray(g, float).T if (transposed and orient_shards) else np.asarray(g, float)
              for g in shards]
        if reduce_norm:
            nrm = np.sqrt(sum(np.sum(X * X) for X in Xs)) + 1e-7
            Xs = [X / nrm for X in Xs]
        else:
            Xs = [X / (np.linalg.norm(X) + 1e-7) for X in Xs]
        p = Xs[0].shape[0]
        for w, (s, e) in enumerate(ref.gram_windows(len(table), restarts)):
            if reduce_gram and (rereduce or w == 0):
                A = sum(X @ X.T for X in Xs)
                As = [A] * len(Xs)
            else:
                As = [X @ X.T for X in Xs]
            new = []
            for X, A in zip(Xs, As):
                Q = np.eye(p)
                for k in range(s, e):
                    a, b, c = table[k]
                    P = a * np.eye(p) + b * A + c * (A @ A)
                    Q = P @ Q
                    A = P @ A @ P
                new.append(Q @ X)
            Xs = new
        return [X.T if (transposed and orient_shards) else X for X in Xs]
    return ns


LOCAL_MUTANTS = {
    "norm not reduced": _local_variant(reduce_norm=False),
    "Gram not reduced": _local_variant(reduce_gram=False),
    "Gram reduced on the first window only": _local_variant(rereduce=False),
    "shards not oriented": _local_variant(orient_shards=False),
}


def _local_battery(ns):
    bad = []
    for shape, transposed, widths in [((9, 23), False, [8, 8, 7]), ((23, 9), True, [5, 18])]:
        G = np.random.default_rng(6).standard_normal(shape)
        for r in ([2], [1, 3]):
            try:
                outs = ns(_split(G, transposed, widths), transposed, QT, r)
                got = _join(outs, transposed)
                ok = got.shape == G.shape and np.max(np.abs(got - _svd_ns(G, QT))) <= 1e-12
            except Exception:
                ok = False
            if not ok:
                bad.append(f"{shape}{r}")
    return bad


def test_local_oracle_passes_battery():
    assert _local_battery(lambda sh, t, tab, r: oracle.gram_newton_schulz_distributed_local(
        sh, t, coefficients=tab, restart_iterations=r)) == []


@pytest.mark.parametrize("name", sorted(LOCAL_MUTANTS))
def test_local_battery_rejects_mutant(name):
    assert _local_battery(LOCAL_MUTANTS[name]) != []
