"""The steady state of the hot path allocates nothing.

Launch tables are keyed by the shapes and options of a call, never by its
pointers: 40 distinct sets of gradient, output, parameter and momentum
buffers cycled through one workspace must build one table per entry point
and still match the fp64 oracle on every call.  Also: a workspace that the
binding allocates for a call on a side stream stays valid for that stream's
kernels.
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

# several tiles and ragged tails, both orientations, fp32 operands
SHAPES = [(200, 72), (72, 330), (64, 64)]
SETS = 40


def _grad(s, i, m, n):
    return workloads.grad_np("gauss", m, n, 71, s, i)


def test_ns_pointer_sets_reuse_one_table():
    ws = dm.alloc_workspace(SHAPES, "f32")
    # all sets stay alive, so every call has distinct pointers
    gs = [[to_dev(_grad(s, i, m, n), "f32") for i, (m, n) in enumerate(SHAPES)]
          for s in range(SETS)]
    outs = [[torch.empty_like(g) for g in row] for row in gs]
    ptrs = {(g.data_ptr(), o.data_ptr()) for rg, ro in zip(gs, outs) for g, o in zip(rg, ro)}
    assert len(ptrs) == SETS * len(SHAPES)
    dm.ns_orthogonalize(gs[0], outs[0], prec="f32", workspace=ws)  # builds the table
    built = dm.plan_builds()
    for s in range(1, SETS):
        dm.ns_orthogonalize(gs[s], outs[s], prec="f32", workspace=ws)
    torch.cuda.synchronize()
    assert dm.plan_builds() == built, "a pointer change built a new table"
    for s in range(SETS):
        for i, (m, n) in enumerate(SHAPES):
            want = oracle.direct_newton_schulz(_grad(s, i, m, n).astype(np.float64))
            e = rel_frobenius(exact64(outs[s][i]), want)
            assert e <= 1e-4, (s, i, e)


def test_step_pointer_sets_reuse_one_table():
    """Momentum buffers and params move too (each set its own), with one
    workspace; every step checked against the oracle."""
    sets = 12
    ws = dm.alloc_workspace(SHAPES, "f32")
    ps0 = [[workloads.param_np(m, n, 72, i + 10 * s) for i, (m, n) in enumerate(SHAPES)]
           for s in range(sets)]
    params = [[to_dev(p, "f32") for p in row] for row in ps0]
    bufs = [[torch.zeros(m, n, device="cuda") for m, n in SHAPES] for _ in range(sets)]
    grads = [[to_dev(_grad(s, i, m, n), "f32") for i, (m, n) in enumerate(SHAPES)]
             for s in range(sets)]
    dm.muon_step(params[0], grads[0], bufs[0], prec="f32", nesterov=True, workspace=ws)
    built = dm.plan_builds()
    for s in range(1, sets):
        dm.muon_step(params[s], grads[s], bufs[s], prec="f32", nesterov=True, workspace=ws)
    torch.cuda.synchronize()
    assert dm.plan_builds() == built
    for s in range(sets):
        for i, (m, n) in enumerate(SHAPES):
            g = _grad(s, i, m, n).astype(np.float64)
            want_p, want_b, _ = oracle.muon_step(ps0[s][i].astype(np.float64), g,
                                                 np.zeros((m, n)), nesterov=True)
            assert rel_frobenius(exact64(bufs[s][i]), want_b) <= 1e-6
            O_gpu = (ps0[s][i].astype(np.float64) - exact64(params[s][i])) / 0.02
            O = (ps0[s][i].astype(np.float64) - want_p) / 0.02
            assert rel_frobenius(O_gpu, O) <= 1e-4, (s, i)


def test_side_stream_call_with_binding_workspace():
    """workspace=None on a side stream: the temporary workspace belongs to
    that stream, so later allocations on the default stream cannot take it
    while the call's kernels still run.  Same bits as a default-stream call."""
    gs = [to_dev(_grad(0, i, m, n), "f32").to(torch.bfloat16) for i, (m, n) in enumerate(SHAPES)]
    ref = dm.ns_orthogonalize(gs, prec="auto")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = [torch.empty_like(g) for g in gs]
    dm.ns_orthogonalize(gs, outs, prec="auto", stream=side)
    # churn the default stream's allocator while the side stream works
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    del junk
    side.synchronize()
    torch.cuda.synchronize()
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)
