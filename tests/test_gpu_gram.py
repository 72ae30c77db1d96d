"""GPU parity of Gram-space Newton-Schulz (backend "gram", fp32 operands)
against the fp64 oracle's Gram iteration, through the C ABI.

Tolerance: fp32 NS, <= 1e-4 relative Frobenius (the bound the direct fp32
path is held to); the single-term tables isolate the products.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import exact64, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import newton_schulz_06_amd as dm  # noqa: E402

SHAPES = [(64, 64), (100, 300), (300, 100), (33, 33), (1, 7), (7, 1), (257, 700),
          (700, 257), (520, 1100), (129, 129)]


def _gen(shape, seed, kind="gauss"):
    return workloads.grad_np(kind, shape[0], shape[1], 91, seed, 0)


def _gram_gpu(gs_np, dtype="f32", **kw):
    gs = [to_dev(g, dtype) for g in gs_np]
    outs = dm.ns_orthogonalize(gs, prec=kw.pop("prec", "f32"), backend="gram", **kw)
    torch.cuda.synchronize()
    return [exact64(g) for g in gs], [exact64(o) for o in outs]


@pytest.mark.parametrize("table", [[(1.0, 0.0, 0.0)], [(0.0, 1.0, 0.0)], [(0.0, 0.0, 1.0)],
                                   [(1.5, -0.5, 0.25), (0.5, 1.0, -0.5)]])
def test_gram_single_terms(table):
    gs_np = [_gen(s, i) for i, s in enumerate(SHAPES)]
    gin, outs = _gram_gpu(gs_np, coefficients=table)
    for s, g, o in zip(SHAPES, gin, outs):
        want = oracle.gram_newton_schulz(g, coefficients=table)
        assert rel_frobenius(o, want) <= 1e-5, (s, table)


@pytest.mark.parametrize("restarts", [None, [], [1, 3], [4], [1, 2, 3, 4]])
@pytest.mark.parametrize("coef", ["quintic", "you"])
def test_gram_matches_oracle(restarts, coef):
    table = None if coef == "quintic" else oracle.YOU_COEFFICIENTS
    gs_np = [_gen(s, 10 + i) for i, s in enumerate(SHAPES)]
    gin, outs = _gram_gpu(gs_np, coefficients=table, restart_iterations=restarts)
    for s, g, o in zip(SHAPES, gin, outs):
        want = oracle.gram_newton_schulz(g, coefficients=table, restart_iterations=restarts)
        e = rel_frobenius(o, want)
        assert e <= 1e-4, (s, restarts, coef, e)


def test_gram_structured_and_auto_precision():
    shapes = [(1024, 256), (200, 640)]
    gs_np = [_gen(s, 30 + i, kind) for i, (s, kind) in
             enumerate(zip(shapes, ["lowrank", "powerlaw_t3"]))]
    gin, outs = _gram_gpu(gs_np, "bf16", prec="auto")
    for s, g, o in zip(shapes, gin, outs):
        want = oracle.gram_newton_schulz(g)
        # bf16 output: the final rounding, then the fp32 NS bound
        assert rel_frobenius(o, want) <= 1e-2, s


def test_gram_muon_step_matches_oracle():
    cfg = workloads.BY_NAME["tinymlp_d256_ff1024_fp32"]
    shapes = cfg.shapes
    params = [to_dev(workloads.param_np(m, n, 1, i), "f32") for i, (m, n) in enumerate(shapes)]
    bufs = [torch.zeros(m, n, device="cuda") for m, n in shapes]
    ref_bufs = [np.zeros(s) for s in shapes]
    for step in range(2):
        grads = [to_dev(workloads.grad_np("gauss", m, n, 1, step, i), "f32")
                 for i, (m, n) in enumerate(shapes)]
        before = [exact64(p) for p in params]
        dm.muon_step(params, grads, bufs, lr=0.02, momentum=0.95, nesterov=True, prec="f32",
                     backend="gram")
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            ref_bufs[i], u = oracle.momentum_update(ref_bufs[i], exact64(grads[i]), 0.95, True)
            assert rel_frobenius(exact64(bufs[i]), ref_bufs[i]) <= 1e-6
            O = oracle.gram_newton_schulz(u)
            got = (before[i] - exact64(params[i])) / 0.02
            assert rel_frobenius(got, O) <= 1e-4, (step, i)


def test_gram_tinymlp_batch_and_llama_matrix_full_size():
    """The 12-matrix TinyMLP batch (512 x 2048 oriented) and one Llama-8B
    gate matrix (14336 x 4096), NS only, against the oracle."""
    shapes = list(workloads.BY_NAME["tinymlp_d512_ff2048_x4"].shapes) + [(14336, 4096)]
    gs_np = [workloads.grad_np("gauss", m, n, 92, 0, i) for i, (m, n) in enumerate(shapes)]
    gin, outs = _gram_gpu(gs_np)
    for i in (0, 2, len(shapes) - 1):
        g = gin[i]
        # column-major copy: the oracle's transposed view is then row-major for BLAS
        u = np.asfortranarray(g) if g.shape[0] > g.shape[1] else g
        want = oracle.gram_newton_schulz(u)
        assert rel_frobenius(outs[i], want) <= 1e-4, shapes[i]
