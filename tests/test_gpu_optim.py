"""GPU parity of dmuon_clip_grad_norm and dmuon_adamw_step against the fp64
oracle, through the C ABI.

Tolerances follow the kernels' arithmetic:
- **Clipping.** Norms are fp32 partial sums of 4096 elements, combined in
  fp64 per bucket: relative error 1e-5. An fp32 gradient after scaling is
  within 1e-5 relative of the oracle. For a bf16 one, the part beyond half
  an ulp (the final rounding) is within 1e-5 of |g|.
- **AdamW.** The update is computed in fp32, within 1e-5 relative of the
  oracle (moments) and 1e-5 of the update size (params), plus half an ulp
  for bf16 params.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import bf16_ulp, exact64, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import newton_schulz_06_amd as dm  # noqa: E402

# ragged sizes, one past a 4096-element chunk, a vector, a tall and a wide matrix
SHAPES = [(3, 5), (4097,), (64, 65), (1, 1), (300, 100), (257, 33), (8, 4096)]


def _grads(shapes, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(s) * scale * (i + 1) for i, s in enumerate(shapes)]


def _dev(arrs, dtype):
    return [to_dev(np.atleast_1d(a), dtype) for a in arrs]


def _check_clip(got, want, dtype):
    for g, w in zip(got, want):
        g = exact64(g)
        if dtype == "f32":
            assert np.allclose(g, w, rtol=1e-5, atol=0), np.max(np.abs(g - w) / np.abs(w))
        else:
            excess = np.abs(g - w) - 0.5 * bf16_ulp(g) * 1.0001
            assert np.all(excess <= 1e-5 * np.abs(w) + 1e-30), np.max(excess)


def _check_stats(st, want):
    assert len(st) == len(want)
    for s, w in zip(st, want):
        assert s["param_count"] == w["param_count"]
        assert s["clipped"] == w["clipped"] and s["found_inf"] == w["found_inf"]
        for k in ("total_norm", "clip_coef"):
            if math.isfinite(w[k]):
                assert abs(s[k] - w[k]) <= 1e-5 * abs(w[k]), (k, s[k], w[k])
            else:
                assert (math.isnan(w[k]) and math.isnan(s[k])) or s[k] == w[k], (k, s[k], w[k])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [2.0, 1.0, 3.0, math.inf])
def test_clip_one_bucket(dtype, p):
    arrs = _grads(SHAPES, 1)
    gs = _dev(arrs, dtype)
    ins = [exact64(g) for g in gs]
    max_norm = 0.25 * oracle.total_norm(ins, p)  # clipping applies
    st = dm.clip_grad_norm(gs, max_norm, norm_type=p)
    want_g, want_st = oracle.clip_grad_norm(ins, max_norm, norm_type=p)
    _check_stats(st, want_st)
    _check_clip(gs, want_g, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_clip_buckets_are_segment_local(dtype):
    arrs = _grads(SHAPES, 2)
    buckets = [2, 0, 1, 0, 2, 1, 0]
    gs = _dev(arrs, dtype)
    ins = [exact64(g) for g in gs]
    st = dm.clip_grad_norm(gs, 5.0, buckets=buckets)
    want_g, want_st = oracle.clip_grad_norm(ins, 5.0, buckets=buckets)
    _check_stats(st, want_st)
    _check_clip(gs, want_g, dtype)


def test_clip_misaligned_views_take_the_scalar_path():
    base = [torch.randn(n + 1, device="cuda") for n in (4097, 30, 7)]
    gs = [b[1:] for b in base]  # contiguous, 4 bytes off a 16-byte boundary
    ins = [exact64(g) for g in gs]
    st = dm.clip_grad_norm(gs, 1.0)
    want_g, want_st = oracle.clip_grad_norm(ins, 1.0)
    _check_stats(st, want_st)
    _check_clip(gs, want_g, "f32")


def test_clip_below_limit_and_stats_only_leave_grads_untouched():
    gs = _dev(_grads(SHAPES, 3), "bf16")
    before = [g.clone() for g in gs]
    ins = [exact64(g) for g in gs]
    st = dm.clip_grad_norm(gs, 1e9)
    _check_stats(st, oracle.clip_grad_norm(ins, 1e9)[1])
    st = dm.clip_grad_norm(gs, None)
    _check_stats(st, oracle.clip_grad_norm(ins, None)[1])
    for a, b in zip(gs, before):
        assert torch.equal(a, b)


def test_clip_nonfinite():
    g = [torch.tensor([1.0, 2.0, float("inf"), 3.0, 4.0], device="cuda"),
         torch.ones(10, device="cuda")]
    ins = [exact64(t) for t in g]
    st = dm.clip_grad_norm(g, 1.0)
    want_g, want_st = oracle.clip_grad_norm(ins, 1.0)
    _check_stats(st, want_st)
    for a, w in zip(g, want_g):  # coefficient 0: inf * 0 = NaN, the rest 0
        assert np.array_equal(exact64(a), w, equal_nan=True)
    g = [torch.tensor([1.0, float("nan"), 3.0], device="cuda")]
    st = dm.clip_grad_norm(g, 1.0, norm_type=math.inf)
    assert st[0]["found_inf"] and math.isnan(st[0]["total_norm"])
    assert torch.isnan(g[0]).all()


def test_clip_llama8b_projection_grads_full_size():
    """The 28 bf16 projection gradients of the Llama-8B batch (872M
    elements), one bucket per layer: every bucket's stats against the
    oracle's clip_grad_norm on the same gradients, and a sample of scaled
    rows against its scaled gradients (within the final bf16 rounding)."""
    import workloads
    cfg = workloads.BY_NAME["llama8b_proj_x4"]
    gs = [workloads.grad_torch("gauss", m, n, 3, 0, i, "cuda", torch.bfloat16)
          for i, (m, n) in enumerate(cfg.shapes)]
    buckets = [i // 7 for i in range(len(gs))]
    rows = [0, 1, 1023, -1]
    want_g, want_st = oracle.clip_grad_norm([exact64(g) for g in gs], 100.0, buckets=buckets)
    want_rows = [w[rows] for w in want_g]
    del want_g
    st = dm.clip_grad_norm(gs, 100.0, buckets=buckets)
    _check_stats(st, want_st)
    assert all(s["clipped"] for s in st)
    for g, want in zip(gs, want_rows):
        got = exact64(g[rows])
        excess = np.abs(got - want) - 0.5 * bf16_ulp(got) * 1.0001
        assert np.all(excess <= 1e-5 * np.abs(want) + 1e-30)


# ------------------------------------------------------------------- AdamW --

def _adam_state(shapes, seed, pdt, gdt):
    rng = np.random.default_rng(seed)
    ps = [to_dev(np.atleast_1d(0.02 * rng.standard_normal(s)), pdt) for s in shapes]
    ms = [torch.zeros_like(p, dtype=torch.float32) for p in ps]
    vs = [torch.zeros_like(p, dtype=torch.float32) for p in ps]
    return ps, ms, vs


def _check_adamw(p, m, v, wp, wm, wv, p0, m0, g, t, lr, wd, pdt, b1=0.9, b2=0.999, eps=1e-8):
    """Errors bounded relative to the magnitudes of the terms (the moment
    update can cancel): m within 1e-5 of b1|m0| + (1-b1)|g|, v within 1e-5
    relative, p within 1e-5 of the step formed from those magnitudes, plus
    the final rounding of p."""
    mag_m = b1 * np.abs(m0) + (1 - b1) * np.abs(g)
    assert np.all(np.abs(m - wm) <= 1e-5 * mag_m + 1e-30)
    assert np.allclose(v, wv, rtol=1e-5, atol=1e-30)
    den = np.sqrt(wv / (1 - b2 ** t)) + eps
    mag_step = lr * (mag_m / (1 - b1 ** t)) / den + lr * wd * np.abs(p0)
    slack = 0.5 * bf16_ulp(p) * 1.0001 if pdt == "bf16" else 2.0 ** -23 * np.abs(wp)
    assert np.all(np.abs(p - wp) <= 1e-5 * mag_step + slack)


@pytest.mark.parametrize("pdt,gdt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_adamw_steps(pdt, gdt):
    hp = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    ps, ms, vs = _adam_state(SHAPES, 11, pdt, gdt)
    for t in range(1, 5):
        gs = _dev(_grads(SHAPES, 20 + t, 0.1), gdt)
        p0 = [exact64(p) for p in ps]
        m0 = [exact64(m) for m in ms]
        v0 = [exact64(v) for v in vs]
        dm.adamw_step(ps, gs, ms, vs, t, **hp)
        torch.cuda.synchronize()
        for i in range(len(ps)):
            g64 = exact64(gs[i])
            wp, wm, wv = oracle.adamw_step(p0[i], g64, m0[i], v0[i], t, lr=hp["lr"],
                                           beta1=0.9, beta2=0.999, eps=1e-8,
                                           weight_decay=0.01)
            _check_adamw(exact64(ps[i]), exact64(ms[i]), exact64(vs[i]), wp, wm, wv, p0[i],
                         m0[i], g64, t, hp["lr"], 0.01, pdt)


def test_adamw_misaligned_views():
    base_p = torch.randn(4098, device="cuda") * 0.02
    base_g = torch.randn(4099, device="cuda")
    p, g = base_p[1:], base_g[2:]
    m = torch.zeros(4097, device="cuda")
    v = torch.zeros(4097, device="cuda")
    p0 = exact64(p)
    dm.adamw_step([p], [g], [m], [v], 1, lr=0.01, weight_decay=0.1)
    torch.cuda.synchronize()
    g64 = exact64(g)
    wp, wm, wv = oracle.adamw_step(p0, g64, np.zeros(4097), np.zeros(4097), 1, lr=0.01,
                                   weight_decay=0.1)
    _check_adamw(exact64(p), exact64(m), exact64(v), wp, wm, wv, p0, np.zeros(4097), g64, 1,
                 0.01, 0.1, "f32")


def test_adamw_llama8b_embeddings_full_size():
    """Embedding and LM head of Llama-8B (2 x 128256 x 4096 bf16 params, fp32
    moments), three steps; sampled rows against the oracle."""
    shape = (128256, 4096)
    gen = torch.Generator(device="cuda").manual_seed(5)
    ps = [(0.02 * torch.randn(shape, device="cuda", generator=gen)).to(torch.bfloat16)
          for _ in range(2)]
    ms = [torch.zeros(shape, device="cuda") for _ in range(2)]
    vs = [torch.zeros(shape, device="cuda") for _ in range(2)]
    rows = [0, 7, 65535, 128255]
    p_ref = [exact64(p[rows]) for p in ps]
    m_ref = [np.zeros((4, 4096)) for _ in range(2)]
    v_ref = [np.zeros((4, 4096)) for _ in range(2)]
    for t in range(1, 4):
        gs = [(torch.randn(shape, device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
              for _ in range(2)]
        dm.adamw_step(ps, gs, ms, vs, t)
        torch.cuda.synchronize()
        for i in range(2):
            # teacher-forced: the oracle starts each step from the GPU's state
            g64 = exact64(gs[i][rows])
            wp, wm, wv = oracle.adamw_step(p_ref[i], g64, m_ref[i], v_ref[i], t)
            got_m, got_v = exact64(ms[i][rows]), exact64(vs[i][rows])
            _check_adamw(exact64(ps[i][rows]), got_m, got_v, wp, wm, wv, p_ref[i], m_ref[i],
                         g64, t, 1e-3, 0.01, "bf16")
            p_ref[i], m_ref[i], v_ref[i] = exact64(ps[i][rows]), got_m, got_v
        del gs
