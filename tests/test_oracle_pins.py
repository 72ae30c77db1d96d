"""Pins for the fp64 oracle, checked against facts that do not come from the
oracle itself: SVD closed forms, scalar-polynomial closed forms, matrix
invariances, printed constants, and a library bf16 conversion.

A plausible slip in the oracle (dropped c-term, wrong sign, momentum order,
wrong orientation, eps in the wrong place) fails at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import (QUINTIC, YOU_COEFFICIENTS, coefficient_table,
                    direct_newton_schulz, momentum_update, muon_step,
                    ns_iterate_left, ns_iterate_right, frobenius_normalize,
                    orient, round_to_bf16)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _phi(x, table):
    """Scalar odd polynomial x -> a x + b x^3 + c x^5, composed per step.
    The NS matrix polynomial acts on each singular value this way."""
    x = np.asarray(x, dtype=np.float64)
    for a, b, c in table:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _svd_reference(G, table, eps=1e-7):
    U, s, Vt = np.linalg.svd(np.asarray(G, np.float64), full_matrices=False)
    sn = s / (math.sqrt(float(np.sum(s * s))) + eps)
    return (U * _phi(sn, table)) @ Vt


def _haar(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


TABLES = {"quintic": coefficient_table(None, 5),
          "you": coefficient_table(YOU_COEFFICIENTS)}


# ------------------------------------------------------------- constants --

def test_printed_constants_match_pages():
    with open(os.path.join(GOLDEN, "dmuon_api_constants.json")) as f:
        g = json.load(f)
    assert [list(r) for r in YOU_COEFFICIENTS] == g["you_coefficients"]["value"]
    assert oracle.DEFAULT_EPS == g["direct_newton_schulz_defaults"]["eps"]
    import inspect
    sig = inspect.signature(muon_step).parameters
    d = g["muon_defaults"]
    assert sig["lr"].default == d["lr"]
    assert sig["momentum"].default == d["momentum"]
    assert sig["weight_decay"].default == d["weight_decay"]
    assert sig["ns_steps"].default == d["ns_steps"]
    assert sig["nesterov"].default == d["nesterov"]
    sig = inspect.signature(direct_newton_schulz).parameters
    assert sig["steps"].default == g["direct_newton_schulz_defaults"]["steps"]


def test_coefficient_table_semantics():
    # no list -> the quintic repeated `steps` times
    assert coefficient_table(None, 3) == [QUINTIC] * 3
    # a list -> its length is the step count, `steps` ignored
    G = np.random.default_rng(0).standard_normal((6, 10))
    a = direct_newton_schulz(G, steps=2, coefficients=YOU_COEFFICIENTS)
    b = direct_newton_schulz(G, steps=7, coefficients=YOU_COEFFICIENTS)
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        coefficient_table([(1.0, 2.0)])


# ------------------------------------------------------- NS closed forms --

@pytest.mark.parametrize("table", ["quintic", "you"])
@pytest.mark.parametrize("shape", [(5, 9), (9, 5), (7, 7), (16, 48), (48, 16),
                                   (64, 128), (128, 64), (1, 6), (6, 1)])
def test_ns_matches_svd_closed_form(shape, table):
    rng = np.random.default_rng([shape[0], shape[1], len(table)])
    G = rng.standard_normal(shape) * 3.0
    got = direct_newton_schulz(G, coefficients=TABLES[table])
    want = _svd_reference(G, TABLES[table])
    assert got.shape == G.shape
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.abs(want).max())


@pytest.mark.parametrize("table", ["quintic", "you"])
def test_ns_svd_closed_form_spread_spectrum(table):
    # prescribed singular values spread over [1e-2, 1] after normalization
    rng = np.random.default_rng(11)
    m, n = 24, 40
    U = _haar(rng, m)
    V = _haar(rng, n)[:, :m]
    s = np.exp(np.linspace(np.log(1.0), np.log(1e-2), m)) * 7.0
    G = (U * s) @ V.T
    got = direct_newton_schulz(G, coefficients=TABLES[table])
    want = (U * _phi(s / (np.linalg.norm(s) + 1e-7), TABLES[table])) @ V.T
    assert np.max(np.abs(got - want)) <= 1e-12


@pytest.mark.parametrize("table,band", [("quintic", (0.6818, 1.1344)),
                                        ("you", (0.9777, 1.0318))])
def test_output_singular_values_in_band(table, band):
    # Normalized input singular values in [0.01, 1] land in the scalar map's
    # band, which the scalar polynomial gives independently here; the band
    # itself sits inside the "roughly 0.7 to 1.2" range quoted for the quintic.
    x = np.exp(np.linspace(np.log(1e-2), 0.0, 200001))
    y = _phi(x, TABLES[table])
    assert band[0] - 1e-4 <= y.min() and y.max() <= band[1] + 1e-4
    assert 0.65 <= y.min() and y.max() <= 1.25
    rng = np.random.default_rng(5)
    for shape in [(32, 96), (96, 32), (40, 40)]:
        G = rng.standard_normal(shape)
        sn = np.linalg.svd(G, compute_uv=False)
        sn = sn / np.linalg.norm(sn)
        if sn.min() < 1e-2:
            continue
        so = np.linalg.svd(direct_newton_schulz(G, coefficients=TABLES[table]),
                           compute_uv=False)
        assert y.min() - 1e-9 <= so.min() and so.max() <= y.max() + 1e-9


def test_rank_one_closed_form():
    rng = np.random.default_rng(3)
    u = rng.standard_normal(20); u /= np.linalg.norm(u)
    v = rng.standard_normal(50); v /= np.linalg.norm(v)
    for sigma in (1e-3, 1.0, 250.0):
        G = sigma * np.outer(u, v)
        for t in TABLES.values():
            want = _phi(sigma / (sigma + 1e-7), t) * np.outer(u, v)
            assert np.max(np.abs(direct_newton_schulz(G, coefficients=t) - want)) < 1e-12
            want_T = want.T
            assert np.max(np.abs(direct_newton_schulz(G.T, coefficients=t) - want_T)) < 1e-12
    # the scalar value itself, for use as a pin of GPU runs at full size
    assert abs(_phi(1.0, TABLES["quintic"]) - 0.6964364095) < 1e-9
    assert abs(_phi(1.0, TABLES["you"]) - 0.9783455603) < 1e-9


@pytest.mark.parametrize("p,q", [(4, 4), (8, 24), (24, 8), (16, 64)])
def test_orthonormal_rows_closed_form(p, q):
    # G with orthonormal rows (or columns when tall): all singular values 1,
    # normalized to 1/sqrt(min side) -> output = phi(1/sqrt(k)) * G
    rng = np.random.default_rng(p * 1000 + q)
    k = min(p, q)
    Q = _haar(rng, max(p, q))[:, :k]
    G = Q.T if p < q else Q
    if p == q:
        G = Q
    for t in TABLES.values():
        want = _phi(1.0 / (math.sqrt(k) + 1e-7), t) * G
        assert np.max(np.abs(direct_newton_schulz(G, coefficients=t) - want)) < 1e-12


def test_zero_input_gives_zero():
    # eps on the norm: 0 / (0 + eps) = 0, so NS(0) = 0
    assert np.array_equal(direct_newton_schulz(np.zeros((4, 9))), np.zeros((4, 9)))


def test_eps_is_added_to_the_norm_not_its_square():
    # A scalar-like 1x1 input: X0 = g / (|g| + eps); result = phi(X0)
    for g in (1e-6, 3e-7, 2.0):
        got = direct_newton_schulz(np.array([[g]]))[0, 0]
        want = _phi(g / (g + 1e-7), TABLES["quintic"])
        assert abs(got - want) < 1e-12


# ----------------------------------------------------------- invariances --

def test_transpose_equivariance_square():
    rng = np.random.default_rng(21)
    for n in (6, 17, 33):
        G = rng.standard_normal((n, n))
        a = direct_newton_schulz(G.T)
        b = direct_newton_schulz(G).T
        assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("shape", [(9, 30), (30, 9), (12, 12)])
def test_left_form_equals_right_form(shape):
    rng = np.random.default_rng(31)
    G = rng.standard_normal(shape)
    t = TABLES["quintic"]
    X = frobenius_normalize(G)
    right = ns_iterate_right(X, t)            # on G's own layout
    left = direct_newton_schulz(G)            # oriented left form
    assert np.max(np.abs(left - right)) < 1e-12
    Xo, tr = orient(G)
    assert tr == (shape[0] > shape[1])
    left2 = ns_iterate_left(frobenius_normalize(Xo), t)
    assert np.max(np.abs((left2.T if tr else left2) - right)) < 1e-12


@pytest.mark.parametrize("alpha", [1e-3, 1e3])
def test_positive_scale_invariance(alpha):
    rng = np.random.default_rng(41)
    G = rng.standard_normal((10, 26))
    a = direct_newton_schulz(alpha * G)
    b = direct_newton_schulz(G)
    # the two normalizations differ by a relative eps/(alpha*|G|) - eps/|G|
    delta = 1e-7 * abs(1.0 / alpha - 1.0) / np.linalg.norm(G)
    assert np.max(np.abs(a - b)) <= 50 * delta + 1e-12


@pytest.mark.parametrize("shape", [(8, 20), (20, 8), (11, 11)])
def test_orthogonal_invariance(shape):
    rng = np.random.default_rng(51)
    G = rng.standard_normal(shape)
    Q = _haar(rng, shape[0])
    R = _haar(rng, shape[1])
    O = direct_newton_schulz(G)
    assert np.max(np.abs(direct_newton_schulz(Q @ G) - Q @ O)) < 1e-12
    assert np.max(np.abs(direct_newton_schulz(G @ R) - O @ R)) < 1e-12


# -------------------------------------------------------------- momentum --

def test_momentum_scalar_values():
    # buf=1, g=2, mu=0.5: buffer first -> 2.5; lookahead g + mu*buf -> 3.25
    b, u = momentum_update(np.array([1.0]), np.array([2.0]), 0.5, True)
    assert b[0] == 2.5 and u[0] == 3.25
    b, u = momentum_update(np.array([1.0]), np.array([2.0]), 0.5, False)
    assert b[0] == 2.5 and u[0] == 2.5


@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_closed_form_constant_gradient(nesterov):
    mu = 0.95
    g = np.random.default_rng(61).standard_normal((3, 4))
    buf = np.zeros_like(g)
    for t in range(1, 21):
        buf, u = momentum_update(buf, g, mu, nesterov)
        want_buf = g * (1 - mu ** t) / (1 - mu)
        assert np.max(np.abs(buf - want_buf)) < 1e-12
        want_u = g + mu * want_buf if nesterov else want_buf
        assert np.max(np.abs(u - want_u)) < 1e-12


# ---------------------------------------------------------------- update --

def test_update_closed_forms():
    rng = np.random.default_rng(71)
    p = rng.standard_normal((6, 14))
    g = rng.standard_normal((6, 14))
    buf = rng.standard_normal((6, 14))
    lr, mu, wd = 0.02, 0.95, 0.1
    new_p, new_buf, O = muon_step(p, g, buf, lr=lr, momentum=mu,
                                  weight_decay=wd, nesterov=True)
    _, u = momentum_update(buf, g, mu, True)
    assert np.max(np.abs(O - _svd_reference(u, TABLES["quintic"]))) < 1e-12
    assert np.max(np.abs(new_p - (p * (1 - lr * wd) - lr * O))) < 1e-14
    # wd = 0: p_new = p - lr * O
    new_p0, _, O0 = muon_step(p, g, buf, lr=lr, momentum=mu, weight_decay=0.0)
    assert np.max(np.abs(new_p0 - (p - lr * O0))) < 1e-15
    # zero gradient and zero buffer: O = 0, only decay remains
    z = np.zeros_like(p)
    new_pz, new_bz, Oz = muon_step(p, z, z, lr=lr, momentum=mu, weight_decay=wd)
    assert np.array_equal(Oz, z) and np.array_equal(new_bz, z)
    assert np.max(np.abs(new_pz - (1 - lr * wd) * p)) < 1e-15


# ------------------------------------------------------------------ bf16 --

def test_round_to_bf16_known_values():
    e = 2.0 ** -8   # half an ulp of bf16 at 1.0 (ulp = 2^-7)
    cases = {1.0: 1.0, 1.0 + e: 1.0, 1.0 + 3 * e: 1.0 + 4 * e,
             1.0 + e * 1.0000001: 1.0 + 2 * e, -1.0 - 3 * e: -1.0 - 4 * e,
             3.0: 3.0, 0.0: 0.0}
    for x, want in cases.items():
        assert round_to_bf16(np.array([x]))[0] == want, x


def test_round_to_bf16_matches_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(81)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-3).astype(np.float32)])
    # force exact ties too: float32 values whose low 16 bits are 0x8000
    ties = (x[:500].view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
