"""GPU parity of Gram-space Newton-Schulz with fp16 operands (backend
"gram", prec "f16") against the fp64 oracle's Gram iteration, through the
C ABI.

The products take fp16 operands (X normalized before the first window; A
and P A stored times 2^12, P and Q times 2^10) with fp32 accumulation, and
keep the fp32 A for the polynomial's linear term.  The bounds come from a
numpy emulation of exactly that arithmetic (fp16 rounding of every operand,
fp32 products, mirrored symmetric outputs) on the same inputs:
- single-term tables (one product each): emulated at most 2.2e-3; held to
  5e-3;
- the quintic on well-conditioned rectangular Gaussian matrices: at most
  3.2e-3 with the default restart, 4.4e-3 with restarts [1, 3] or [1, 2, 3,
  4]; held to 1e-2;
- square Gaussian matrices (condition number ~300) with the default restart
  (a window of three steps): 1.6e-2 to 2.0e-2; held to 3e-2.  Shorter
  windows bring them to 2e-3 to 4e-3 (held to 1e-2);
- the workload stand-ins, bf16 inputs (Gaussian 2048 x 512, low-rank
  1024 x 3584, power-law 3584 x 1024, lognormal-scaled 96 x 96 and
  32 x 480): relative Frobenius 3.3e-3, 1.9e-2, 1.3e-2, 1.6e-2, 5.4e-3,
  singular-value deviation at most 1.2e-2.  Held to 8e-3, 2.5e-2, 2e-2,
  2e-2, 1e-2 and 2e-2: the low-rank input sits at the 2e-2 line the bf16
  modes are held to (measured 2.03e-2), the cost of fp16 operands in the
  Gram form, whose window polynomial Q amplifies the small singular
  directions (up to 41x with the quintic) together with their rounding
  errors.  Restarts at [2, 4] bring it to 1.2e-2 (emulated).
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

# 64-wide tiles up to p = 520, 128-wide at p = 800, 256-wide at p = 1000
# (padded to 1024)
RECT = [(100, 300), (300, 100), (1, 7), (7, 1), (257, 700), (700, 257), (520, 1100),
        (800, 1200), (3000, 1000)]
SQUARE = [(64, 64), (33, 33), (129, 129)]


def _say(msg):
    print(f"[gram f16] {msg}", flush=True)


def _gen(shape, seed, kind="gauss"):
    return workloads.grad_np(kind, shape[0], shape[1], 91, seed, 0)


def _gram16(gs_np, dtype="f32", **kw):
    gs = [to_dev(g, dtype) for g in gs_np]
    outs = dm.ns_orthogonalize(gs, prec="f16", backend="gram", **kw)
    torch.cuda.synchronize()
    return [exact64(g) for g in gs], [exact64(o) for o in outs]


@pytest.mark.parametrize("table", [[(1.0, 0.0, 0.0)], [(0.0, 1.0, 0.0)], [(0.0, 0.0, 1.0)],
                                   [(1.5, -0.5, 0.25), (0.5, 1.0, -0.5)]])
def test_gram_f16_single_terms(table):
    shapes = RECT + SQUARE
    gs_np = [_gen(s, i) for i, s in enumerate(shapes)]
    gin, outs = _gram16(gs_np, coefficients=table)
    worst = 0.0
    for s, g, o in zip(shapes, gin, outs):
        e = rel_frobenius(o, oracle.gram_newton_schulz(g, coefficients=table))
        worst = max(worst, e)
        assert e <= 5e-3, (s, table, e)
    _say(f"table {table}: worst relF {worst:.2e}")


@pytest.mark.parametrize("restarts", [None, [1, 3], [1, 2, 3, 4]])
@pytest.mark.parametrize("coef", ["quintic", "you"])
def test_gram_f16_matches_oracle(restarts, coef):
    """Both coefficient tables (the YOU table's window bounds: 16.1 and 30.5
    under the default restart).  Emulated with the YOU table: rectangular
    shapes at most 1.9e-3, square ones up to 2.3e-2 with the default
    restart and 2.8e-3 with [1, 3]."""
    table = None if coef == "quintic" else oracle.YOU_COEFFICIENTS
    shapes = RECT + SQUARE
    gs_np = [_gen(s, 10 + i) for i, s in enumerate(shapes)]
    gin, outs = _gram16(gs_np, coefficients=table, restart_iterations=restarts)
    for s, g, o in zip(shapes, gin, outs):
        want = oracle.gram_newton_schulz(g, coefficients=table, restart_iterations=restarts)
        e = rel_frobenius(o, want)
        bound = 3e-2 if (s in SQUARE and restarts is None) else 1e-2
        _say(f"{coef} restarts {restarts} {s}: relF {e:.2e} (bound {bound})")
        assert e <= bound, (s, restarts, coef, e)


def test_gram_f16_edge_cases():
    """A zero matrix (O = 0), one NS step (a single window with no factor
    products), 16 steps (six windows under restarts every third step), and
    an empty batch."""
    g = torch.zeros(64, 200, device="cuda")
    (o,) = dm.ns_orthogonalize([g], prec="f16", backend="gram")
    torch.cuda.synchronize()
    assert torch.count_nonzero(o).item() == 0
    gs_np = [_gen(s, 60 + i) for i, s in enumerate([(100, 300), (520, 1100)])]
    for steps, restarts in [(1, None), (16, [3, 6, 9, 12, 15])]:
        gin, outs = _gram16(gs_np, ns_steps=steps, restart_iterations=restarts)
        for g64, o64 in zip(gin, outs):
            want = oracle.gram_newton_schulz(g64, steps=steps, restart_iterations=restarts)
            e = rel_frobenius(o64, want)
            _say(f"{steps} steps, restarts {restarts} {g64.shape}: relF {e:.2e}")
            assert e <= 1e-2, (steps, e)
    assert dm.ns_orthogonalize([], prec="f16", backend="gram") == []


STAND_INS = [("gauss", (2048, 512), 8e-3), ("lowrank", (1024, 3584), 2.5e-2),
             ("powerlaw_t3", (3584, 1024), 2e-2), ("gauss_lognormal", (96, 96), 2e-2),
             ("gauss_lognormal", (32, 480), 1e-2)]


def test_gram_f16_workload_stand_ins():
    """The emulation's five stand-ins (64-, 128- and 256-wide tiles), bf16
    inputs as the optimizer hands them over."""
    gs_np = [workloads.grad_np(kind, m, n, 93, 0, i)
             for i, (kind, (m, n), _) in enumerate(STAND_INS)]
    gin, outs = _gram16(gs_np, "bf16")
    bad = []
    for (kind, s, bound), g, o in zip(STAND_INS, gin, outs):
        want = oracle.gram_newton_schulz(g)
        e, sd = rel_frobenius(o, want), sigma_dev(o, want)
        _say(f"{kind} {s}: relF {e:.2e} (bound {bound}) sigma-dev {sd:.2e}")
        if not (e <= bound and sd <= 2e-2):
            bad.append((kind, s, e, sd))
    assert not bad, bad


def test_gram_f16_muon_step_matches_oracle():
    """Two Nesterov steps of the fp32 TinyMLP d=256 batch: the momentum
    buffer exactly as the oracle's, the update direction within the fp16
    Gram bound."""
    cfg = workloads.BY_NAME["tinymlp_d256_ff1024_fp32"]
    shapes = cfg.shapes
    params = [to_dev(workloads.param_np(m, n, 1, i), "f32") for i, (m, n) in enumerate(shapes)]
    bufs = [torch.zeros(m, n, device="cuda") for m, n in shapes]
    ref_bufs = [np.zeros(s) for s in shapes]
    for step in range(2):
        grads = [to_dev(workloads.grad_np("gauss", m, n, 1, step, i), "f32")
                 for i, (m, n) in enumerate(shapes)]
        before = [exact64(p) for p in params]
        dm.muon_step(params, grads, bufs, lr=0.02, momentum=0.95, nesterov=True, prec="f16",
                     backend="gram")
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            ref_bufs[i], u = oracle.momentum_update(ref_bufs[i], exact64(grads[i]), 0.95, True)
            assert rel_frobenius(exact64(bufs[i]), ref_bufs[i]) <= 1e-6
            O = oracle.gram_newton_schulz(u)
            got = (before[i] - exact64(params[i])) / 0.02
            e = rel_frobenius(got, O)
            _say(f"step {step} matrix {i} {shapes[i]}: relF {e:.2e}")
            assert e <= 1e-2, (step, i, e)


def test_gram_f16_graph_replays_bitwise():
    """A recorded fp16 Gram call replays bit for bit what the direct call
    computes, with new contents in the recorded input buffers."""
    shapes = [(300, 120), (120, 500), (1024, 2048)]
    gs = [to_dev(_gen(s, 40 + i), "f32") for i, s in enumerate(shapes)]
    o_direct = [torch.empty_like(t) for t in gs]
    o_graph = [torch.empty_like(t) for t in gs]
    graph = dm.ns_orthogonalize_graph(gs, o_graph, prec="f16", backend="gram")
    for rep in range(2):
        if rep:
            for i, t in enumerate(gs):
                t.copy_(to_dev(_gen(shapes[i], 50 + i), "f32"))
            torch.cuda.synchronize()
        graph()
        dm.ns_orthogonalize(gs, o_direct, prec="f16", backend="gram")
        torch.cuda.synchronize()
        for i in range(len(gs)):
            assert torch.equal(o_graph[i], o_direct[i]), ("replay", rep, i)
        _say(f"replay {rep}: graph == direct")
    graph.close()


def test_gram_f16_full_size_llama8b_matrices():
    """Full Llama-8B projection shapes on 256-wide tiles: a gate matrix
    (14336 x 4096) with the configuration's low-rank recipe and a k
    projection (1024 x 4096, Gaussian), NS only, bf16 inputs.  Emulated on
    the same recipe at this size: 1.9e-2 (low-rank)."""
    cases = [("lowrank", (14336, 4096), 2.5e-2), ("gauss", (1024, 4096), 8e-3)]
    gs_np = [workloads.grad_np(kind, m, n, 94, 0, i) for i, (kind, (m, n), _) in enumerate(cases)]
    gin, outs = _gram16(gs_np, "bf16")
    for (kind, s, bound), g, o in zip(cases, gin, outs):
        # column-major copy: the oracle's transposed view is then row-major for BLAS
        u = np.asfortranarray(g) if g.shape[0] > g.shape[1] else g
        e = rel_frobenius(o, oracle.gram_newton_schulz(u))
        _say(f"full size {kind} {s}: relF {e:.2e} (bound {bound})")
        assert e <= bound, (kind, s, e)


def test_gram_f16_full_size_70b_matrix():
    """One 70B MLP gate matrix (28672 x 8192, power-law spectrum with
    Student-t noise, bf16), NS only: fp16 Gram-space NS within the 2e-2
    bound (measured 1.64e-2; the direct path in its automatic precision
    measures 1.7e-3 on the same matrix)."""
    cfg = workloads.CONFIGS[5]
    m, n = cfg.shapes[0]
    gin, outs = _gram16([workloads.grad_np(cfg.grad_kind, m, n, 5, 0, 0)], "bf16")
    u = np.asfortranarray(gin[0])  # tall: the oracle's transposed view is row-major
    e = rel_frobenius(outs[0], oracle.gram_newton_schulz(u))
    _say(f"full size 70B {m}x{n}: relF {e:.2e}")
    assert e <= 2e-2, e
