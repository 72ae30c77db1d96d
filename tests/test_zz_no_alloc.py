"""dmuon_muon_step_noalloc (the library's static device scratch instead of a
workspace) against dmuon_muon_step on the same state, through the C ABI:
two calls in a row, the second on a smaller batch, each compared bit for bit
with the workspace entry point and against the fp64 oracle (momentum
<= 1e-6, NS <= 1e-4 fp32 / 2e-2 bf16).  Also: an oversized batch is refused
before anything is enqueued."""
import ctypes

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

# one TinyMLP d=512 layer (bf16 NS, fp32 params), then the fp32 TinyMLP d=256
CALLS = [
    ("auto", [(2048, 512), (2048, 512), (512, 2048)], 81),
    ("f32", [(1024, 256), (1024, 256), (256, 1024)], 82),
]


def _state(shapes, seed):
    ps = [workloads.param_np(m, n, seed, i) for i, (m, n) in enumerate(shapes)]
    gs = [workloads.grad_np("gauss", m, n, seed, 0, i) for i, (m, n) in enumerate(shapes)]
    return ps, gs


def test_noalloc_matches_workspace_step_twice():
    for prec, shapes, seed in CALLS:
        print(f"[noalloc] prec {prec}, shapes {shapes}", flush=True)
        ps, gs = _state(shapes, seed)
        # the same state twice: one for each entry point
        pa = [to_dev(p, "f32") for p in ps]
        pb = [to_dev(p, "f32") for p in ps]
        ba = [torch.zeros(m, n, device="cuda") for m, n in shapes]
        bb = [torch.zeros(m, n, device="cuda") for m, n in shapes]
        grads = [to_dev(g, "f32") for g in gs]
        for b in ba:  # a nonzero buffer, so the Nesterov lookahead matters
            b.fill_(0.25)
        for b in bb:
            b.fill_(0.25)
        dm.muon_step_noalloc(pa, grads, ba, prec=prec, nesterov=True)
        dm.muon_step(pb, grads, bb, prec=prec, nesterov=True)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(pa[i], pb[i]), ("params differ", prec, i)
            assert torch.equal(ba[i], bb[i]), ("bufs differ", prec, i)
            want_p, want_b, O = oracle.muon_step(ps[i].astype(np.float64), gs[i].astype(np.float64),
                                                 np.full(shapes[i], 0.25), nesterov=True)
            assert rel_frobenius(exact64(ba[i]), want_b) <= 1e-6
            O_gpu = (ps[i].astype(np.float64) - exact64(pa[i])) / 0.02
            tol = 1e-4 if prec == "f32" else 2e-2
            e = rel_frobenius(O_gpu, O)
            print(f"[noalloc] matrix {i} {shapes[i]}: NS rel err {e:.2e}", flush=True)
            assert e <= tol, (prec, i, e)


def test_noalloc_rejects_oversized_batch():
    shapes = [(8192, 8192)]
    b, keep = dm.shape_batch(shapes, dm.DMUON_F32)
    for i in range(1):
        b.mats[i].ptr = 0x10000000 + 0x10000000 * i
    bg, k2 = dm.shape_batch(shapes, dm.DMUON_F32)
    bg.mats[0].ptr = 0x50000000
    bb, k3 = dm.shape_batch(shapes, dm.DMUON_F32)
    bb.mats[0].ptr = 0x90000000
    cfg, kc = dm.make_cfg(prec="f32")
    st = dm.lib().dmuon_muon_step_noalloc(ctypes.byref(b), ctypes.byref(bg), ctypes.byref(bb),
                                          ctypes.byref(cfg), 0.95, 0.02, 0.0, 1, None)
    assert st == dm.DMUON_E_UNSUPPORTED
    assert "scratch" in dm.lib().dmuon_last_error().decode()
