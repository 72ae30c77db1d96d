"""Recorded calls (dmuon_muon_step_graph, dmuon_ns_orthogonalize_graph,
dmuon_graph_launch) replay exactly what the direct calls enqueue.

Each replay is compared bitwise with the direct call on a second copy of
the same buffers (same kernels, same tables: the results must be identical),
with the program's own eager work and synchronizations between replays, on
the TinyMLP step shapes (fp32 d=256 x1, fp32 d=512 x4) and the packed batch
of 512 small bf16 matrices.  The NS replays are also held to the oracle.
Also: a graph outlives the eviction of its launch tables from the cache,
and replays on a stream other than the current one.
"""
import pytest

import oracle
import workloads
from tests.gpu_util import exact64, rel_frobenius, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import newton_schulz_06_amd as dm  # noqa: E402


def _say(msg):
    print(f"[graph] {msg}", flush=True)


def _eager_noise():
    """Unrelated eager work between replays (a product and a reduction)."""
    a = torch.randn(512, 512, device="cuda")
    return float((a @ a).sum().item())


def _step_case(cid, sets=3):
    cfg = workloads.CONFIGS[cid]
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    ps = [workloads.param_torch(m, n, cid, i, "cuda", dt[cfg.param_dtype])
          for i, (m, n) in enumerate(cfg.shapes)]
    grads = [[to_dev(workloads.grad_np(cfg.grad_kind, m, n, cid, s, i), cfg.grad_dtype)
              for i, (m, n) in enumerate(cfg.shapes)] for s in range(sets)]
    return cfg, ps, grads


@pytest.mark.parametrize("cid", [1, 2])
def test_step_graph_replays_bitwise(cid):
    cfg, ps, grads = _step_case(cid)
    kw = dict(lr=cfg.lr, momentum=cfg.momentum, weight_decay=cfg.weight_decay,
              nesterov=cfg.nesterov, ns_steps=cfg.ns_steps, prec=cfg.ns_prec)
    pa = [p.clone() for p in ps]
    pb = [p.clone() for p in ps]
    ba = [torch.zeros(p.shape, dtype=torch.float32, device="cuda") for p in ps]
    bb = [torch.zeros_like(b) for b in ba]
    direct = dm.PreparedMuonStep(pa, ba, grads, **kw)
    graphed = dm.PreparedMuonStep(pb, bb, grads, graph=True, **kw)
    for step in range(6):
        s = step % len(grads)
        direct(s)
        graphed(s)
        torch.cuda.synchronize()
        _eager_noise()
        for i in range(len(ps)):
            assert torch.equal(pa[i], pb[i]), ("param", cid, step, i)
            assert torch.equal(ba[i], bb[i]), ("buf", cid, step, i)
        _say(f"config {cid} step {step}: graph replay == direct call")
    assert sum(g is not None for g in graphed.graphs) == len(grads)
    # the parameters moved: the replays did run
    assert not torch.equal(pb[0], ps[0])


def test_ns_graph_packed_batch_bitwise_and_oracle():
    cfg = workloads.CONFIGS[4]
    gs_np = [workloads.grad_np(cfg.grad_kind, m, n, 4, 0, i) for i, (m, n) in enumerate(cfg.shapes)]
    g = [to_dev(a, "bf16") for a in gs_np]
    o_direct = [torch.empty_like(t) for t in g]
    o_graph = [torch.empty_like(t) for t in g]
    direct = dm.PreparedNs(g, o_direct, ns_steps=cfg.ns_steps, prec=cfg.ns_prec)
    graphed = dm.PreparedNs(g, o_graph, ns_steps=cfg.ns_steps, prec=cfg.ns_prec, graph=True)
    side = torch.cuda.Stream()
    for rep in range(3):
        if rep:
            # new contents in the recorded input buffers: the replay reads them
            for i, t in enumerate(g):
                t.copy_(to_dev(workloads.grad_np(cfg.grad_kind, *cfg.shapes[i], 4, rep, i),
                               "bf16"))
            torch.cuda.synchronize()
        direct()
        if rep == 2:
            # a replay on another stream, ordered after the direct call
            side.wait_stream(torch.cuda.current_stream())
            dm.lib().dmuon_graph_launch(graphed.graph.handle, dm._stream_handle(side))
            torch.cuda.current_stream().wait_stream(side)
        else:
            graphed()
        torch.cuda.synchronize()
        _eager_noise()
        for i in range(len(g)):
            assert torch.equal(o_direct[i], o_graph[i]), ("out", rep, i)
        _say(f"packed batch replay {rep}: graph == direct")
    # the last replay's inputs against the oracle (bf16 operands: 2e-2)
    worst = 0.0
    for i, (m, n) in enumerate(cfg.shapes[:64]):
        x = exact64(g[i])
        want = oracle.direct_newton_schulz(x, steps=cfg.ns_steps)
        worst = max(worst, rel_frobenius(exact64(o_graph[i]), want))
    _say(f"packed batch vs oracle: worst relF {worst:.3e} over 64 matrices")
    assert worst <= 2e-2


def test_graph_outlives_table_eviction():
    """Past the cache's 256 layouts the graph's tables are evicted from the
    cache; the graph keeps them, and its replays stay exact."""
    shapes = [(96, 160), (160, 96)]
    gs = [to_dev(workloads.grad_np("gauss", m, n, 73, 0, i), "f32") for i, (m, n) in enumerate(shapes)]
    o_graph = [torch.empty_like(t) for t in gs]
    o_direct = [torch.empty_like(t) for t in gs]
    graph = dm.ns_orthogonalize_graph(gs, o_graph, prec="f32")
    graph()
    torch.cuda.synchronize()
    first = [t.clone() for t in o_graph]
    # 260 other layouts, more than the cache's 256: ours is evicted
    for k in range(260):
        x = torch.randn(32 + (k % 13), 40 + k, device="cuda")
        dm.ns_orthogonalize([x], prec="f32")
    torch.cuda.synchronize()
    for t in o_graph:
        t.zero_()
    graph()
    dm.ns_orthogonalize(gs, o_direct, prec="f32")
    torch.cuda.synchronize()
    for i in range(len(gs)):
        assert torch.equal(o_graph[i], first[i]), ("after eviction", i)
        assert torch.equal(o_graph[i], o_direct[i]), ("graph vs direct", i)
    graph.close()
    graph.close()  # idempotent
    dm.ns_orthogonalize(gs, o_direct, prec="f32")
    torch.cuda.synchronize()
    for i, (m, n) in enumerate(shapes):
        want = oracle.direct_newton_schulz(exact64(gs[i]))
        assert rel_frobenius(exact64(o_direct[i]), want) <= 1e-4


def test_gram_backend_graph_replays_bitwise():
    """A recorded Gram-space NS call (fp32 operands, restart windows) and a
    recorded fp32 step on 16-wide tiles replay bit for bit what the direct
    calls compute."""
    shapes = [(300, 120), (120, 500)]
    gs = [to_dev(workloads.grad_np("gauss", m, n, 74, 0, i), "f32") for i, (m, n) in enumerate(shapes)]
    o_direct = [torch.empty_like(t) for t in gs]
    o_graph = [torch.empty_like(t) for t in gs]
    graph = dm.ns_orthogonalize_graph(gs, o_graph, prec="f32", backend="gram",
                                      restart_iterations=[2])
    for rep in range(2):
        graph()
        dm.ns_orthogonalize(gs, o_direct, prec="f32", backend="gram", restart_iterations=[2])
        torch.cuda.synchronize()
        _eager_noise()
        for i in range(len(gs)):
            assert torch.equal(o_graph[i], o_direct[i]), ("gram", rep, i)
    for i in range(len(gs)):
        want = oracle.direct_newton_schulz(exact64(gs[i]))
        assert rel_frobenius(exact64(o_graph[i]), want) <= 1e-4
    graph.close()
