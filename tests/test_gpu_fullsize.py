"""GPU parity at the benchmark's full sizes, in the launch configuration it
times.

The Llama-8B projection batch (4 layers, 28 matrices up to 14336 x 4096)
and the 70B MLP batch (6 matrices of 28672 x 8192 / 8192 x 28672) run
through ``PreparedMuonStep`` on inputs from bench.py's own generator, so the
shapes, precision mode and tile plan are the ones it measures.  Momentum is
checked on every matrix of every step (bit-exact on step 1 from a zero
buffer, <= 1e-6 relative after); the Newton-Schulz update is checked
against the fp64 oracle on the matrices the host can afford: one of each
distinct oriented shape of the projection batch (4096 x 4096, 1024 x 4096,
a tall and a wide 4096 x 14336), and one tall and one wide 70B matrix.
The TinyMLP and the 512-matrix batch are checked whole elsewhere.
"""
import time

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import bf16_param_excess, exact64, rel_frobenius

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bench  # noqa: E402
import newton_schulz_06_amd as dm  # noqa: E402


def _say(msg):
    print(f"[fullsize] {msg}", flush=True)


def _full_run(name, steps, ns_check):
    cfg = workloads.BY_NAME[name]
    dev = torch.device("cuda", 0)
    params, bufs, sets = bench.make_inputs(cfg, steps, dev)
    call = dm.PreparedMuonStep(params, bufs, sets, lr=cfg.lr, momentum=cfg.momentum,
                               weight_decay=cfg.weight_decay, nesterov=cfg.nesterov,
                               ns_steps=cfg.ns_steps, prec=cfg.ns_prec)
    ref_bufs = {}
    for step in range(steps):
        p_before = {i: exact64(params[i]) for i in ns_check} if step == 0 else {}
        call(step)
        torch.cuda.synchronize()
        _say(f"{name} step {step} done on the GPU")
        us = {}
        for i, (m, n) in enumerate(cfg.shapes):
            if step == 0:
                # buf = 0*mu + g: exact in any arithmetic
                assert torch.equal(bufs[i], sets[0][i].float()), ("buf", step, i)
                if i in ns_check:
                    g = exact64(sets[0][i])
                    ref_bufs[i], us[i] = oracle.momentum_update(np.zeros((m, n)), g,
                                                                cfg.momentum, cfg.nesterov)
            else:
                prev = ref_bufs.get(i)
                if prev is None:
                    prev = exact64(sets[0][i])
                g = exact64(sets[step][i])
                ref_bufs[i], _ = oracle.momentum_update(prev, g, cfg.momentum, cfg.nesterov)
                e = rel_frobenius(exact64(bufs[i]), ref_bufs[i])
                assert e <= 1e-6, ("momentum", step, i, e)
        if step != 0:
            continue
        for i in ns_check:
            m, n = cfg.shapes[i]
            t0 = time.perf_counter()
            # A tall u is handed over column-major so that the oracle's
            # transposed view is row-major for BLAS (same values, faster).
            u = np.asfortranarray(us[i]) if m > n else us[i]
            O = oracle.direct_newton_schulz(u, steps=cfg.ns_steps)
            _say(f"oracle NS of matrix {i} ({m}x{n}) took {time.perf_counter() - t0:.1f} s")
            e, frac = bf16_param_excess(p_before[i], exact64(params[i]), O, cfg.lr)
            _say(f"matrix {i} ({m}x{n}): param excess {e:.3e}, differing {frac:.3%}")
            assert e <= 2e-2, ("param excess", i, (m, n), e)
            assert frac <= 0.25, ("param frac", i, frac)
            del O


def test_llama8b_projections_full_size():
    """28 matrices, two steps; NS of q (4096x4096), k (1024x4096), gate
    (14336x4096, tall) and the last down (4096x14336, wide) vs the oracle."""
    _full_run("llama8b_proj_x4", 2, ns_check=(0, 1, 4, 27))


def test_llama70b_mlp_full_size():
    """6 matrices with Nesterov, two steps; NS of one tall (28672x8192) and
    one wide (8192x28672) matrix vs the oracle."""
    _full_run("llama70b_mlp", 2, ns_check=(0, 5))
