"""GPU parity of dmuon_muon_step against the fp64 oracle.

Momentum runs free against the oracle's own recursion (<= 1e-6 relative
Frobenius every step).  The orthogonalized update O is read back as
(p_before - p_after) / lr for fp32 params and compared with the oracle's O
computed from the oracle's momentum output (fp32 NS <= 1e-4; bf16 NS
<= 2e-2 relative Frobenius and singular-value deviation).  bf16 params are
compared with p - lr*O_oracle: beyond half an ulp of the stored bf16
value (the final rounding) the difference must stay within the NS
tolerance relative to lr*O.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (bf16_frac_cap, bf16_param_check, bf16_param_excess, exact64,
                            rel_frobenius, sigma_dev, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import newton_schulz_06_amd as dm  # noqa: E402


def _state(cfg, shapes=None, cfg_id=None):
    shapes = shapes or cfg.shapes
    cid = cfg.cfg_id if cfg_id is None else cfg_id
    params = [to_dev(workloads.param_np(m, n, cid, i), cfg.param_dtype)
              for i, (m, n) in enumerate(shapes)]
    bufs = [torch.zeros(m, n, dtype=torch.float32, device="cuda") for m, n in shapes]
    return params, bufs


def _grads(cfg, step, shapes=None, cfg_id=None):
    shapes = shapes or cfg.shapes
    cid = cfg.cfg_id if cfg_id is None else cfg_id
    return [to_dev(workloads.grad_np(cfg.grad_kind, m, n, cid, step, i), cfg.grad_dtype)
            for i, (m, n) in enumerate(shapes)]


def _run(cfg, steps, check_ns_steps, shapes=None, cfg_id=None, nesterov=None):
    shapes = shapes or cfg.shapes
    nesterov = cfg.nesterov if nesterov is None else nesterov
    params, bufs = _state(cfg, shapes, cfg_id)
    ws = dm.alloc_workspace(shapes, cfg.ns_prec)
    ref_bufs = [np.zeros(s) for s in shapes]
    ns_tol = 1e-4 if cfg.ns_prec == "f32" else 2e-2
    report = []
    for step in range(steps):
        grads = _grads(cfg, step, shapes, cfg_id)
        p_before = [exact64(p) for p in params]
        dm.muon_step(params, grads, bufs, lr=cfg.lr, momentum=cfg.momentum,
                     weight_decay=cfg.weight_decay, nesterov=nesterov, ns_steps=cfg.ns_steps,
                     prec=cfg.ns_prec, workspace=ws)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            g64 = exact64(grads[i])
            ref_bufs[i], u = oracle.momentum_update(ref_bufs[i], g64, cfg.momentum, nesterov)
            e_buf = rel_frobenius(exact64(bufs[i]), ref_bufs[i])
            assert e_buf <= 1e-6, ("momentum", step, i, e_buf)
            if step not in check_ns_steps:
                continue
            O = oracle.direct_newton_schulz(u, steps=cfg.ns_steps)
            p_after = exact64(params[i])
            if cfg.param_dtype == "f32":
                O_gpu = (p_before[i] - p_after) / cfg.lr
                e = rel_frobenius(O_gpu, O)
                assert e <= ns_tol, ("NS", step, i, shapes[i], e)
                if cfg.ns_prec != "f32" and min(shapes[i]) <= 1024:
                    d = sigma_dev(O_gpu, O)
                    assert d <= 2e-2, ("sigma", step, i, d)
                report.append(e)
            else:
                # Only the final rounding to bf16 (half an ulp of the stored
                # value) may separate p_after from p_before - lr*O_oracle;
                # whatever exceeds it is NS error and must stay within the
                # NS tolerance, relative to lr*O.
                e, _ = bf16_param_excess(p_before[i], p_after, O, cfg.lr)
                assert e <= ns_tol, ("param excess", step, i, shapes[i], e)
                # Against the exact update rounded once: every element within
                # one bf16 spacing, and at most 5% of them different at all --
                # or, where lr*O spans several spacings (these reduced sizes),
                # the share an NS error at the tolerance would move.
                # Truncating instead of rounding would move about half.
                dist, frac = bf16_param_check(p_before[i], p_after, O, cfg.lr)
                cap = bf16_frac_cap(p_before[i], O, cfg.lr, ns_tol)
                assert dist <= 1.0 + 1e-9, ("param distance", step, i, dist)
                assert frac <= cap, ("param frac", step, i, frac, cap)
                report.append(frac)
    return report


def test_c1_tinymlp_fp32():
    """3 fp32 matrices (1024x256, 1024x256, 256x1024), one step, fp32 NS."""
    cfg = workloads.BY_NAME["tinymlp_d256_ff1024_fp32"]
    _run(cfg, 1, {0})


@pytest.mark.parametrize("nesterov", [False, True])
def test_c1_both_nesterov(nesterov):
    cfg = workloads.BY_NAME["tinymlp_d256_ff1024_fp32"]
    _run(cfg, 3, {0, 2}, nesterov=nesterov)


def test_c2_tinymlp_20_steps():
    """12 matrices of the 4-layer TinyMLP (d=512, ff=2048), 20 steps, fp32
    momentum, bf16 NS; NS checked on the first, second and last steps."""
    cfg = workloads.BY_NAME["tinymlp_d512_ff2048_x4"]
    _run(cfg, 20, {0, 1, 19})


def test_c2_nesterov_on():
    cfg = workloads.BY_NAME["tinymlp_d512_ff2048_x4"]
    _run(cfg, 2, {1}, nesterov=True)


def test_c3_like_bf16_params():
    """Llama-8B projection recipe (low rank + noise, bf16 storage) at a
    quarter of the sizes: 1024x1024, 256x1024, 3584x1024, 1024x3584."""
    cfg = workloads.BY_NAME["llama8b_proj_x4"]
    shapes = [(1024, 1024), (256, 1024), (3584, 1024), (1024, 3584)]
    _run(cfg, 2, {0, 1}, shapes=shapes, cfg_id=93)


def test_c5_like_nesterov_bf16_params():
    """70B-MLP recipe (power law + Student-t, Nesterov) at an eighth of the
    sizes: 3584x1024 (x2) and 1024x3584, three steps."""
    cfg = workloads.BY_NAME["llama70b_mlp"]
    shapes = [(3584, 1024), (3584, 1024), (1024, 3584)]
    _run(cfg, 3, {0, 2}, shapes=shapes, cfg_id=95)


def test_zero_gradient_only_decays():
    shapes = [(64, 200), (200, 64)]
    params = [torch.randn(m, n, device="cuda") for m, n in shapes]
    before = [p.clone() for p in params]
    grads = [torch.zeros(m, n, device="cuda") for m, n in shapes]
    bufs = [torch.zeros(m, n, device="cuda") for m, n in shapes]
    dm.muon_step(params, grads, bufs, lr=0.1, weight_decay=0.5, prec="f32")
    torch.cuda.synchronize()
    for p, b in zip(params, before):
        assert torch.allclose(p, b * (1 - 0.05), rtol=1e-6, atol=0)


def test_step_is_deterministic_and_resumable():
    """Two runs from the same state agree bit for bit; a run that is stopped,
    copied to the host and restored continues bit-identically."""
    cfg = workloads.BY_NAME["tinymlp_d512_ff2048_x4"]
    shapes = cfg.shapes[:3]

    def run(steps, state=None):
        params, bufs = _state(cfg, shapes) if state is None else state
        for s in range(steps):
            dm.muon_step(params, _grads(cfg, s if state is None else s + 2, shapes), bufs,
                         prec="bf16", nesterov=False)
        torch.cuda.synchronize()
        return params, bufs

    a = run(4)
    b = run(4)
    for x, y in zip(a[0] + a[1], b[0] + b[1]):
        assert torch.equal(x, y)
    half = run(2)
    saved = ([p.cpu() for p in half[0]], [q.cpu() for q in half[1]])
    restored = ([p.cuda() for p in saved[0]], [q.cuda() for q in saved[1]])
    c = run(2, restored)
    for x, y in zip(a[0] + a[1], c[0] + c[1]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("nesterov,grad_dtype,ns_steps",
                         [(True, "bf16", 5), (False, "bf16", 5), (True, "f32", 1),
                          (False, "f32", 5), (True, "bf16", 1)])
def test_ragged_256_tiles_nesterov_and_iteration_counts(nesterov, grad_dtype, ns_steps):
    """256-wide tiles with bf16 operands (fp32 master X) on a ragged shape
    in both orientations (p = 1200: a 176-row last tile row and column),
    Nesterov on and off, fp32 and bf16 gradients, one and five NS
    iterations (with one, the first X update is also the one that writes
    the param).  Checked against the oracle on the second step, where the
    momentum buffer is not a multiple of the gradient."""
    shapes = [(1200, 1500), (1500, 1200)]  # p = 1200: 256-wide tiles, 176-row tail
    mu, lr = 0.95, 0.02
    params = [to_dev(workloads.param_np(m, n, 96, i), "f32") for i, (m, n) in enumerate(shapes)]
    bufs = [torch.zeros(m, n, dtype=torch.float32, device="cuda") for m, n in shapes]
    ref = [np.zeros(s) for s in shapes]
    for step in range(2):
        gs = [to_dev(workloads.grad_np("gauss", m, n, 96, step, i), grad_dtype)
              for i, (m, n) in enumerate(shapes)]
        p_before = [exact64(p) for p in params]
        dm.muon_step(params, gs, bufs, lr=lr, momentum=mu, nesterov=nesterov,
                     ns_steps=ns_steps, prec="bf16")
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            ref[i], u = oracle.momentum_update(ref[i], exact64(gs[i]), mu, nesterov)
            assert rel_frobenius(exact64(bufs[i]), ref[i]) <= 1e-6
            if step == 0:
                continue
            O = oracle.direct_newton_schulz(u, steps=ns_steps)
            O_gpu = (p_before[i] - exact64(params[i])) / lr
            e = rel_frobenius(O_gpu, O)
            d = sigma_dev(O_gpu, O)
            assert e <= 2e-2 and d <= 2e-2, (shapes[i], e, d)


@pytest.mark.parametrize("ns_steps", [1, 5])
def test_in_place_ns_256_tiles(ns_steps):
    """NS only on 256-wide tiles, in place (out is g) and out of place give
    the same bits; one iteration (the first X update writes the output) and
    five."""
    shapes = [(1200, 1500), (1500, 1200)]
    gs = [to_dev(workloads.grad_np("gauss", m, n, 97, 0, i), "bf16") for i, (m, n) in enumerate(shapes)]
    out = dm.ns_orthogonalize(gs, prec="bf16", ns_steps=ns_steps)
    inp = [g.clone() for g in gs]
    dm.ns_orthogonalize(inp, outs=inp, prec="bf16", ns_steps=ns_steps)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(out[i], inp[i]), i
        want = oracle.direct_newton_schulz(exact64(gs[i]), steps=ns_steps)
        assert rel_frobenius(exact64(out[i]), want) <= 2e-2
