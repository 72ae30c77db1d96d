"""GPU parity at the benchmark's full sizes, in the launch configuration it
times.

The Llama-8B projection batch (4 layers, 28 matrices up to 14336 x 4096)
and the 70B MLP batch (6 matrices of 28672 x 8192 / 8192 x 28672, Nesterov)
run two Muon steps through ``PreparedMuonStep`` on inputs from bench.py's
own generator, so the shapes, precision mode and tile plan are the ones it
measures.

Checked on every matrix of both steps: the momentum buffer (bit-exact on
step 0 from a zero buffer, <= 1e-6 relative after).

Checked on step 1, where the buffer is no longer zero (so the Nesterov
lookahead g + mu*buf is not a multiple of g, and Newton-Schulz's scale
invariance cannot hide a wrong flag), on one matrix of each distinct
oriented shape (q 4096 x 4096, k 1024 x 4096, a tall gate 14336 x 4096, a
wide down 4096 x 14336; a tall and a wide 70B matrix):

* the NS output itself: the step's NS input u = g + mu*buf (Nesterov) or
  buf is formed on the GPU in fp32 and orthogonalized by
  dmuon_ns_orthogonalize with the same precision mode and tile class (so O
  comes back unrounded, in fp32), then compared with the fp64 oracle's O:
  relative Frobenius error <= 2e-2 and max singular-value deviation
  <= 2e-2 (the bf16-operand tolerances);
* the step's bf16 parameter update against RNE(p - lr*O_oracle), the exact
  update rounded once: every element within one bf16 spacing of it (the
  spacing at the larger of the element's magnitude and the rms of p), and
  at most 5% of the elements different from it.
"""
import time

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import bf16_param_check, exact64, rel_frobenius, sigma_dev_gram

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bench  # noqa: E402
import newton_schulz_06_amd as dm  # noqa: E402

NS_TOL = 2e-2        # bf16-operand NS: relative Frobenius and sigma deviation
PARAM_FRAC = 0.05    # share of bf16 params allowed to differ from RNE(exact)


def _say(msg):
    print(f"[fullsize] {msg}", flush=True)


def _oracle_ns(u, steps, label):
    """oracle.direct_newton_schulz, its steps called one by one (the same
    operations in the same order) so that each iteration reports."""
    X, transposed = oracle.orient(u)
    X = oracle.frobenius_normalize(X)
    for k, row in enumerate(oracle.coefficient_table(None, steps)):
        t0 = time.perf_counter()
        X = oracle.ns_iterate_left(X, [row])
        _say(f"{label}: oracle NS iteration {k + 1}/{steps} took {time.perf_counter() - t0:.1f} s")
    return X.T if transposed else X


def _full_run(name, ns_check):
    cfg = workloads.BY_NAME[name]
    dev = torch.device("cuda", 0)
    steps = 2
    params, bufs, sets = bench.make_inputs(cfg, steps, dev)
    call = dm.PreparedMuonStep(params, bufs, sets, lr=cfg.lr, momentum=cfg.momentum,
                               weight_decay=cfg.weight_decay, nesterov=cfg.nesterov,
                               ns_steps=cfg.ns_steps, prec=cfg.ns_prec)
    mu = cfg.momentum
    ref_bufs = {}
    for step in range(steps):
        last = step == steps - 1
        p_before = {i: exact64(params[i]) for i in ns_check} if last else {}
        # The step's NS input, formed on the GPU in fp32 from the buffers
        # before the step (buf <- mu*buf + g; u = g + mu*buf or buf).
        u_gpu = {}
        if last:
            for i in ns_check:
                g32 = sets[step][i].float()
                b32 = bufs[i] * mu + g32
                u_gpu[i] = (g32 + mu * b32) if cfg.nesterov else b32
                del g32, b32
        call(step)
        torch.cuda.synchronize()
        _say(f"{name} step {step} done on the GPU")
        us = {}
        for i, (m, n) in enumerate(cfg.shapes):
            g = exact64(sets[step][i])
            if step == 0:
                # buf = 0*mu + g: exact in any arithmetic
                assert torch.equal(bufs[i], sets[0][i].float()), ("buf", step, i)
                ref_bufs[i] = g
                continue
            ref_bufs[i], u = oracle.momentum_update(ref_bufs[i], g, mu, cfg.nesterov)
            e = rel_frobenius(exact64(bufs[i]), ref_bufs[i])
            assert e <= 1e-6, ("momentum", step, i, e)
            if i in ns_check:
                us[i] = u
        if not last:
            continue
        # NS of the same inputs through dmuon_ns_orthogonalize (fp32 out)
        o_gpu = {}
        for i in ns_check:
            out = dm.ns_orthogonalize([u_gpu[i]], prec=cfg.ns_prec, ns_steps=cfg.ns_steps)[0]
            torch.cuda.synchronize()
            o_gpu[i] = exact64(out)
            del out, u_gpu[i]
        torch.cuda.empty_cache()
        for i in ns_check:
            m, n = cfg.shapes[i]
            # A tall u is handed over column-major so that the oracle's
            # transposed view is row-major for BLAS (same values, faster).
            u = np.asfortranarray(us[i]) if m > n else us[i]
            O = _oracle_ns(u, cfg.ns_steps, f"matrix {i} ({m}x{n})")
            rel = rel_frobenius(o_gpu[i], O)
            sdev = sigma_dev_gram(o_gpu[i], O)
            dist, frac = bf16_param_check(p_before[i], exact64(params[i]), O, cfg.lr)
            _say(f"matrix {i} ({m}x{n}): NS relF {rel:.3e}, sigma dev {sdev:.3e}; "
                 f"bf16 params: max {dist:.2f} spacings from RNE(exact), {frac:.3%} differ")
            assert rel <= NS_TOL, ("NS relF", i, (m, n), rel)
            assert sdev <= NS_TOL, ("NS sigma dev", i, (m, n), sdev)
            assert dist <= 1.0 + 1e-9, ("param distance", i, (m, n), dist)
            assert frac <= PARAM_FRAC, ("param frac", i, (m, n), frac)
            del O, o_gpu[i]


def test_llama8b_projections_full_size():
    """28 matrices, two steps; on step 1 NS of q (4096x4096), k (1024x4096),
    gate (14336x4096, tall) and the last down (4096x14336, wide) vs the
    oracle."""
    _full_run("llama8b_proj_x4", ns_check=(0, 1, 4, 27))


def test_llama70b_mlp_full_size():
    """6 matrices with Nesterov, two steps; on step 1 NS of one tall
    (28672x8192) and one wide (8192x28672) matrix vs the oracle."""
    _full_run("llama70b_mlp", ns_check=(0, 5))
