"""GPU parity of dmuon_ns_orthogonalize against the fp64 oracle.

Single-term coefficient tables isolate the kernels: (1, 0, 0) returns the
normalized, oriented input (input pass + norm + output pass); (0, 1, 0)
gives X X^T X (SYRK + update-X); (0, 0, 1) gives (X X^T)^2 X (adds the
symmetric polynomial product).  Full tables are then checked at the
tolerances of the method: fp32 NS relative Frobenius <= 1e-4; bf16 NS
relative Frobenius and max singular-value deviation <= 2e-2.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import exact64, rel_frobenius, sigma_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import newton_schulz_06_amd as dm  # noqa: E402

# Shapes spanning several 64/128 tiles, ragged tails, both orientations.
SHAPES = [(64, 64), (100, 300), (300, 100), (33, 33), (1, 7), (7, 1), (257, 700),
          (700, 257), (520, 1100), (129, 129)]


def _gen(shape, seed, kind="gauss"):
    return workloads.grad_np(kind, shape[0], shape[1], 90, seed, 0)


def _run_ns(gs_np, dtype, prec, coefficients=None, ns_steps=5):
    gs = [to_dev(g, dtype) for g in gs_np]
    outs = dm.ns_orthogonalize(gs, coefficients=coefficients, ns_steps=ns_steps, prec=prec)
    torch.cuda.synchronize()
    return [exact64(g) for g in gs], [exact64(o) for o in outs]


UNIT_TABLES = {"identity": [(1.0, 0.0, 0.0)], "syrk": [(0.0, 1.0, 0.0)],
               "poly": [(0.0, 0.0, 1.0)], "mixed2": [(1.5, -0.5, 0.25), (0.5, 1.0, -0.5)]}


@pytest.mark.parametrize("prec,dtype,tol", [("f32", "f32", 2e-6), ("bf16", "f32", 1.5e-2),
                                            ("bf16", "bf16", 1.5e-2),
                                            ("bf16_split", "bf16", 1.5e-2)])
@pytest.mark.parametrize("table", sorted(UNIT_TABLES))
def test_single_term_tables(table, prec, dtype, tol):
    coeffs = UNIT_TABLES[table]
    gs_np = [_gen(s, i) for i, s in enumerate(SHAPES)]
    gin, outs = _run_ns(gs_np, dtype, prec, coefficients=coeffs)
    for s, g, o in zip(SHAPES, gin, outs):
        want = oracle.direct_newton_schulz(g, coefficients=coeffs)
        err = rel_frobenius(o, want)
        # The identity table only rounds the normalized input: fp32 mode
        # keeps X in fp32; the bf16 modes keep X as bf16 X plus the bf16
        # rounding of the remainder: with bf16's unit roundoff 2^-8 the
        # remainder is at most 2^-8 |x| and its rounding at most 2^-16 |x|.
        if table == "identity" and dtype == "f32":
            lim = 2e-6 if prec == "f32" else 2.0 ** -16
        else:
            lim = 1e-2 if table == "identity" else tol
        assert err <= lim, (table, prec, dtype, s, err)


@pytest.mark.parametrize("coef", ["quintic", "you"])
def test_ns_f32_matches_oracle(coef):
    table = None if coef == "quintic" else oracle.YOU_COEFFICIENTS
    gs_np = [_gen(s, 10 + i) for i, s in enumerate(SHAPES)]
    gin, outs = _run_ns(gs_np, "f32", "f32", coefficients=table)
    for s, g, o in zip(SHAPES, gin, outs):
        want = oracle.direct_newton_schulz(g, coefficients=table)
        assert rel_frobenius(o, want) <= 1e-4, (s, rel_frobenius(o, want))


@pytest.mark.parametrize("steps", [1, 2, 3, 4, 16])
def test_ns_iteration_counts(steps):
    """Odd and even iteration counts, 1 to the maximum of 16 (the quintic at
    every step): the X operand buffers alternate between iterations and the
    last iteration writes the output, so a wrong parity would show as an
    O(1) error.  fp32 operands on 64- and 128-wide tiles; 16-bit operands
    (automatic mode: fp16 after a bf16 first iteration on 64- and 128-wide
    tiles, plain bf16 on 256-wide ones) for up to 4 steps.  Tolerances: 1e-4 (fp32; 1e-3 at
    16 steps, where small singular values are amplified by up to 3.44 per
    step before they converge) and 2e-2 (16-bit)."""
    f32_shapes = [(300, 200), (200, 300), (800, 1000), (1000, 800), (129, 129)]
    gs_np = [_gen(s, 100 + i) for i, s in enumerate(f32_shapes)]
    gin, outs = _run_ns(gs_np, "f32", "f32", ns_steps=steps)
    for s, g, o in zip(f32_shapes, gin, outs):
        want = oracle.direct_newton_schulz(g, steps=steps)
        e = rel_frobenius(o, want)
        assert e <= (1e-3 if steps > 5 else 1e-4), (s, steps, e)
    if steps > 4:
        return
    bf_shapes = [(300, 200), (800, 1000), (1024, 1300), (1300, 1024)]
    gs_np = [_gen(s, 110 + i) for i, s in enumerate(bf_shapes)]
    gin, outs = _run_ns(gs_np, "bf16", "auto", ns_steps=steps)
    for s, g, o in zip(bf_shapes, gin, outs):
        want = oracle.direct_newton_schulz(g, steps=steps)
        e = rel_frobenius(o, want)
        assert e <= 2e-2, (s, steps, e)


@pytest.mark.parametrize("prec", ["bf16_split", "f16", "auto"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ns_bf16_matches_oracle(prec, dtype):
    """iid Gaussian inputs (the hardest spectra for bf16 operands) with hi/lo
    split bf16 operands, and in the fp16 mode (which auto resolves to)."""
    gs_np = [_gen(s, 20 + i) for i, s in enumerate(SHAPES)]
    gin, outs = _run_ns(gs_np, dtype, prec)
    for s, g, o in zip(SHAPES, gin, outs):
        want = oracle.direct_newton_schulz(g)
        e = rel_frobenius(o, want)
        d = sigma_dev(o, want)
        assert e <= 2e-2 and d <= 2e-2, (s, prec, dtype, e, d)


@pytest.mark.parametrize("prec", ["bf16_split_a", "f16"])
def test_ns_split_a_mid_gaussian(prec):
    """hi/lo A with plain bf16 B, and the fp16 mode, on iid Gaussians with
    min sides 257 to 1024, the hardest spectra for bf16 operands."""
    shapes = [(257, 700), (700, 257), (520, 1100), (2048, 512), (512, 512), (160, 640)]
    gs_np = [_gen(s, 70 + i) for i, s in enumerate(shapes)]
    gin, outs = _run_ns(gs_np, "bf16", prec)
    for s, g, o in zip(shapes, gin, outs):
        want = oracle.direct_newton_schulz(g)
        e = rel_frobenius(o, want)
        d = sigma_dev(o, want)
        assert e <= 2e-2 and d <= 2e-2, (s, prec, e, d)


@pytest.mark.parametrize("prec", ["bf16", "f16"])
def test_ns_plain_bf16_large_gaussian(prec):
    """Plain bf16 operands, and the fp16 mode, on 128-wide tiles (1100 pads
    too much for 256): an iid Gaussian 1100 x 4400 and its transpose."""
    gs_np = [_gen((1100, 4400), 60), _gen((4400, 1100), 61)]
    gin, outs = _run_ns(gs_np, "bf16", prec)
    for g, o in zip(gin, outs):
        want = oracle.direct_newton_schulz(g)
        e = rel_frobenius(o, want)
        d = sigma_dev(o, want)
        assert e <= 2e-2 and d <= 2e-2, (g.shape, prec, e, d)


def test_ns_c4_packed_batch():
    """512 small matrices (sides log-uniform in [32, 1024], multiples of 32)
    in one call, per-matrix tolerance, automatic precision."""
    cfg = workloads.BY_NAME["packed_small_512"]
    gs_np = [workloads.grad_np(cfg.grad_kind, m, n, 4, 0, i) for i, (m, n) in enumerate(cfg.shapes)]
    gin, outs = _run_ns(gs_np, "bf16", "auto")
    worst_e = worst_d = 0.0
    for i, (g, o) in enumerate(zip(gin, outs)):
        want = oracle.direct_newton_schulz(g)
        e = rel_frobenius(o, want)
        worst_e = max(worst_e, e)
        if min(g.shape) <= 256 or i % 8 == 0:
            worst_d = max(worst_d, sigma_dev(o, want))
        assert e <= 2e-2, (i, g.shape, e)
    assert worst_d <= 2e-2, worst_d
    print(f"c4: worst relF {worst_e:.3e}, worst sigma dev {worst_d:.3e}")


@pytest.mark.parametrize("kind,shape", [("lowrank", (1024, 3584)), ("lowrank", (3584, 1024)),
                                        ("powerlaw_t3", (3584, 1024)),
                                        ("powerlaw_t3", (1024, 3584))])
def test_ns_structured_gradients_bf16(kind, shape):
    """Scaled-down stand-ins of the Llama-8B (low rank + noise) and 70B MLP
    (power law + Student-t) gradients, bf16 storage, bf16 NS."""
    g = workloads.grad_np(kind, shape[0], shape[1], 91, 0, 0)
    gin, outs = _run_ns([g], "bf16", "bf16")
    want = oracle.direct_newton_schulz(gin[0])
    e = rel_frobenius(outs[0], want)
    d = sigma_dev(outs[0], want)
    assert e <= 2e-2 and d <= 2e-2, (kind, shape, e, d)


def test_ns_deterministic_and_in_place():
    gs_np = [_gen(s, 40 + i) for i, s in enumerate(SHAPES)]
    gs = [to_dev(g, "bf16") for g in gs_np]
    a = dm.ns_orthogonalize(gs, prec="bf16")
    b = dm.ns_orthogonalize(gs, prec="bf16")
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    inp = [g.clone() for g in gs]
    dm.ns_orthogonalize(inp, outs=inp, prec="bf16")
    torch.cuda.synchronize()
    for x, y in zip(a, inp):
        assert torch.equal(x, y)


def test_ns_zero_and_nan():
    z = torch.zeros(40, 70, device="cuda")
    n = torch.randn(40, 70, device="cuda")
    n[3, 5] = float("nan")
    out = dm.ns_orthogonalize([z, n], prec="f32")
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0]).item() == 0
    assert torch.isnan(out[1]).any().item()


def test_ns_tiny_shapes():
    for shape in [(1, 1), (1, 2), (2, 1), (3, 3)]:
        g = _gen(shape, 50)
        gin, outs = _run_ns([g], "f32", "f32")
        want = oracle.direct_newton_schulz(gin[0])
        assert rel_frobenius(outs[0], want) <= 1e-5, shape


@pytest.mark.parametrize("prec", ["bf16", "bf16_split", "f16"])
def test_bf16_output_is_rne_of_fp32_output(prec):
    """The same values (exactly representable in bf16) given once as fp32
    and once as bf16 go through identical arithmetic; only the final
    rounding differs, so the bf16 output must equal round-to-nearest-even
    of the fp32 output bit for bit (pins the kernels' conversion)."""
    shapes = [(96, 200), (200, 96), (64, 64), (130, 70)]
    g16 = [to_dev(_gen(s, 60 + i), "bf16") for i, s in enumerate(shapes)]
    g32 = [g.float() for g in g16]
    o16 = dm.ns_orthogonalize(g16, prec=prec)
    o32 = dm.ns_orthogonalize(g32, prec=prec)
    torch.cuda.synchronize()
    for s, a, b in zip(shapes, o16, o32):
        want = oracle.round_to_bf16(exact64(b))
        got = exact64(a)
        assert np.array_equal(got, want), (s, int(np.sum(got != want)))


# Batches whose 64-wide products take 128-deep main-loop stages (every K of
# the launch a multiple of 128 and >= 1536).  DEEP_SYRK: the SYRK, with
# several K values, both orientations and a ragged row count.  DEEP_BOTH:
# the SYRK and the split-A polynomial (K = 3P = 1536, 1920).
DEEP_SYRK = [(512, 2048), (2048, 448), (320, 1536), (1664, 200)]
DEEP_BOTH = [(512, 2048), (640, 1536), (2048, 512)]


@pytest.mark.parametrize("shapes", ["syrk", "both"])
@pytest.mark.parametrize("table", ["syrk", "poly"])
def test_deep_stage_products(table, shapes):
    sh = DEEP_SYRK if shapes == "syrk" else DEEP_BOTH
    coeffs = UNIT_TABLES[table]
    gs_np = [_gen(s, 40 + i) for i, s in enumerate(sh)]
    gin, outs = _run_ns(gs_np, "f32", "bf16_split_a", coefficients=coeffs)
    for s, g, o in zip(sh, gin, outs):
        want = oracle.direct_newton_schulz(g, coefficients=coeffs)
        assert rel_frobenius(o, want) <= 1.5e-2, (s, table)


def test_deep_stage_full_table():
    sh = DEEP_SYRK + DEEP_BOTH
    gs_np = [_gen(s, 50 + i) for i, s in enumerate(sh)]
    gin, outs = _run_ns(gs_np, "f32", "auto")
    for s, g, o in zip(sh, gin, outs):
        want = oracle.direct_newton_schulz(g)
        assert rel_frobenius(o, want) <= 2e-2, s
        assert sigma_dev(o, want) <= 2e-2, s


@pytest.mark.parametrize("shapes,prec,dtype,tol", [
    # fp32 TinyMLP d=256: 408 SYRK and polynomial tiles of 16 x 16 per launch
    ([(1024, 256), (1024, 256), (256, 1024)], "f32", "f32", 1e-4),
    # one TinyMLP d=512 matrix, automatic precision
    ([(2048, 512)], "auto", "bf16", 2e-2),
    # two ragged 64-tile matrices in one launch, both orientations,
    # automatic precision
    ([(500, 2000), (2000, 480)], "auto", "bf16", 2e-2),
])
def test_few_tile_launches(shapes, prec, dtype, tol):
    """Launches of fewer tiles than CUs, with long K (up to 2048): the
    result matches the oracle and repeats bit for bit, also through the
    single-term tables that isolate the SYRK and the polynomial."""
    gs_np = [_gen(s, 60 + i) for i, s in enumerate(shapes)]
    gin, outs = _run_ns(gs_np, dtype, prec)
    _, again = _run_ns(gs_np, dtype, prec)
    for i, (g, o) in enumerate(zip(gin, outs)):
        assert np.array_equal(o, again[i]), ("repeat", i)
        want = oracle.direct_newton_schulz(g)
        e = rel_frobenius(o, want)
        assert e <= tol, (shapes[i], prec, e)
        if prec != "f32":
            assert sigma_dev(o, want) <= 2e-2
    for name in ("syrk", "poly"):
        gin, outs = _run_ns(gs_np, dtype, prec, coefficients=UNIT_TABLES[name], ns_steps=1)
        for i, (g, o) in enumerate(zip(gin, outs)):
            want = oracle.direct_newton_schulz(g, steps=1, coefficients=UNIT_TABLES[name])
            e = rel_frobenius(o, want)
            # as test_single_term_tables: 2e-6 with fp32 operands, 1.5e-2 bf16
            assert e <= (2e-6 if prec == "f32" else 1.5e-2), (name, shapes[i], e)


@pytest.mark.parametrize("shape", [(2048, 512), (500, 2000), (96, 96), (32, 480), (1100, 4400),
                                   (4400, 1200)])
def test_f16_mode_beats_bf16(shape):
    """fp16 operands after a bf16 first iteration, nothing split: on iid
    Gaussians (64-, 128- and 256-wide tiles, both orientations) the error falls to
    a fraction of plain bf16's (a numpy emulation gives 3.0e-3 against
    2.4e-2 at 2048 x 512): within 8e-3 relative Frobenius and singular-value
    deviation, and at most half the bf16 error."""
    g = _gen(shape, 120)
    gin, o16 = _run_ns([g], "bf16", "f16")
    _, obf = _run_ns([g], "bf16", "bf16")
    want = oracle.direct_newton_schulz(gin[0])
    e16, ebf = rel_frobenius(o16[0], want), rel_frobenius(obf[0], want)
    print(f"f16 mode {shape}: relF {e16:.3e} (plain bf16 {ebf:.3e})")
    assert e16 <= 8e-3 and sigma_dev(o16[0], want) <= 8e-3, (shape, e16)
    assert e16 <= 0.5 * ebf, (shape, e16, ebf)


@pytest.mark.parametrize("table", ["syrk", "poly", "mixed2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_f16_mode_second_iteration_products(table, dtype):
    """Two-row tables whose first row is the identity (a X update that only
    normalizes, in bf16) isolate one fp16 iteration: SYRK, polynomial and a
    full step on fp16 operands of the normalized X.  fp16's unit roundoff is
    2^-11, so 4e-3 relative error (bf16 single terms: 1.5e-2)."""
    coeffs = [(1.0, 0.0, 0.0)] + UNIT_TABLES[table][:1]
    gs_np = [_gen(s, 130 + i) for i, s in enumerate(SHAPES)]
    gin, outs = _run_ns(gs_np, dtype, "f16", coefficients=coeffs, ns_steps=2)
    for s, g, o in zip(SHAPES, gin, outs):
        want = oracle.direct_newton_schulz(g, steps=2, coefficients=coeffs)
        err = rel_frobenius(o, want)
        assert err <= 4e-3, (table, dtype, s, err)


def test_auto_resolution():
    """The automatic mode is the fp16 mode on 64- and 128-wide tiles and plain
    bf16 on 256-wide ones: bit for bit the same outputs (one batch mixing
    both classes)."""
    shapes = [(300, 700), (800, 1200), (1200, 4400)]  # tiles 64, 128, 256
    gs = [to_dev(_gen(s, 140 + i), "bf16") for i, s in enumerate(shapes)]
    auto = dm.ns_orthogonalize(gs, prec="auto")
    f16 = dm.ns_orthogonalize(gs[:2], prec="f16")
    bf16 = dm.ns_orthogonalize(gs[2:], prec="bf16")
    torch.cuda.synchronize()
    assert torch.equal(auto[0], f16[0]) and torch.equal(auto[1], f16[1])
    assert torch.equal(auto[2], bf16[0])


def test_f16_mode_you_table_and_special_inputs():
    """The fp16 mode with the printed YOU coefficient table (larger early
    coefficients than the quintic: the scaled A and B operands must stay in
    fp16's range) against the oracle, and a zero and a NaN-holding input
    (zero stays zero, NaN propagates)."""
    table = oracle.YOU_COEFFICIENTS
    shapes = [(300, 700), (2048, 512), (96, 96)]
    gs_np = [_gen(s, 150 + i) for i, s in enumerate(shapes)]
    gin, outs = _run_ns(gs_np, "bf16", "f16", coefficients=table, ns_steps=len(table))
    for s, g, o in zip(shapes, gin, outs):
        want = oracle.direct_newton_schulz(g, steps=len(table), coefficients=table)
        assert np.all(np.isfinite(o)), s
        assert rel_frobenius(o, want) <= 2e-2, (s, rel_frobenius(o, want))
    z = torch.zeros(64, 200, device="cuda", dtype=torch.bfloat16)
    n = torch.randn(200, 64, device="cuda").to(torch.bfloat16)
    n[3, 5] = float("nan")
    out = dm.ns_orthogonalize([z, n], prec="f16")
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0]).item() == 0
    assert torch.isnan(out[1].float()).any().item()
