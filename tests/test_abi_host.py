"""C-ABI checks that need no GPU: the library loads, exports every function
include/dmuon.h declares, sizes workspaces, and rejects bad arguments
synchronously (validation runs before any HIP call, so fake device
addresses are never dereferenced)."""
import ctypes
import os
import re

import pytest

import newton_schulz_06_amd as dm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dmuon_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    L = dm.lib()
    declared = _declared()
    assert {"dmuon_muon_step", "dmuon_ns_orthogonalize"} <= declared
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert declared == set(dm.EXPORTS)


def test_status_strings_and_info():
    L = dm.lib()
    assert L.dmuon_status_str(0) == b"ok"
    assert L.dmuon_status_str(3) == b"workspace"
    assert b"gfx950" in L.dmuon_backend_info()


def _mats(specs, dtype=dm.DMUON_F32):
    arr = (dm.Mat * max(1, len(specs)))()
    for i, (m, n, ptr) in enumerate(specs):
        arr[i] = dm.Mat(m, n, ptr)
    return dm.Batch(arr, len(specs), dtype), arr


def _pad(x, t):
    return (x + t - 1) // t * t


def _ld(n, esz):
    """Row stride: an odd multiple of 256 bytes."""
    u = -(-n * esz // 256)
    if u % 2 == 0:
        u += 1
    return u * 256 // esz


def _tile(p, prec, gram=False):
    if prec == "f32":
        return 16 if p <= 256 and not gram else 64 if p <= 512 else 128

    def fits(t):
        return _pad(p, t) * 8 <= p * 9

    if p >= 1024 and fits(256):
        return 256
    if p >= 768 and fits(128):
        return 128
    return 64


def _expected_ws(shapes, prec):
    """Workspace rule: partials, scales, a 16-byte sink and the call's
    pointer slots (three per matrix), then per matrix
    the master X (fp32 X, plus bf16 X for bf16 operands; or, below 256-tiles,
    bf16 X plus its bf16 remainder), two X^T
    buffers, fp32 A (unless A is split), the operand forms of A ([hi|lo|hi|hi]
    rows when split) and B ([hi|lo] when split); each region rounded to 256
    bytes, rows padded to odd multiples of 256 bytes."""
    a = lambda x: _pad(x, 256)  # noqa: E731
    tiles = 0
    per = []
    for m, n in shapes:
        p, q = min(m, n), max(m, n)
        t = _tile(p, prec)
        P, Q = _pad(p, max(t, 64)), _pad(q, max(t, 64))  # 64 x 64 element-wise tiles
        tiles += (P // 64) * (Q // 64)
        split_b = prec == "bf16_split"
        split_a = prec in ("bf16_split", "bf16_split_a")  # auto (= f16) splits nothing
        if prec == "f32":
            per.append(a(4 * P * _ld(Q, 4)) + 2 * a(4 * Q * _ld(P, 4)) + a(4 * P * _ld(P, 4))
                       + a(4 * P * _ld(P, 4)))
        else:
            hilo = t < 256  # master X: bf16 + bf16 remainder below 256-tiles, else fp32
            base = a(2 * P * _ld(Q, 2)) + 2 * a(2 * Q * _ld(P, 2))
            base += a(2 * P * _ld(Q, 2)) if hilo else a(4 * P * _ld(Q, 4))
            if not split_a:
                base += a(4 * P * _ld(P, 4))
            base += a(2 * P * _ld(4 * P if split_a else P, 2))
            base += a(2 * P * _ld(2 * P if split_b else P, 2))
            per.append(base)
    return a(4 * tiles) + a(16 * len(shapes)) + a(16) + a(24 * len(shapes)) + sum(per)


def test_workspace_size_gram_fp16():
    """Gram-space layout with fp16 operands: the direct fp16 layout's head
    and per-matrix X buffers (master X: bf16 hi + remainder below 256-wide
    tiles, else fp32 beside the 16-bit copy; two 16-bit X^T; fp32 A), then
    five 16-bit P x P buffers (A's operand form, P, P A and the Q pair)."""
    a = lambda x: _pad(x, 256)  # noqa: E731
    shapes = [(1024, 256), (256, 1024), (100, 37), (700, 900), (4096, 1024)]
    tiles, per = 0, 0
    for m, n in shapes:
        p, q = min(m, n), max(m, n)
        t = _tile(p, "f16")
        P, Q = _pad(p, max(t, 64)), _pad(q, max(t, 64))
        tiles += (P // 64) * (Q // 64)
        master = 2 * a(2 * P * _ld(Q, 2)) if t < 256 else a(2 * P * _ld(Q, 2)) + a(4 * P * _ld(Q, 4))
        per += master + 2 * a(2 * Q * _ld(P, 2)) + a(4 * P * _ld(P, 4)) + 5 * a(2 * P * _ld(P, 2))
    want = a(4 * tiles) + a(16 * len(shapes)) + a(16) + a(24 * len(shapes)) + per
    assert dm.workspace_size(shapes, "f16", backend="gram") == want
    assert dm.workspace_size(shapes, "f16", backend="gram") != dm.workspace_size(shapes, "f32",
                                                                                  backend="gram")


def test_workspace_size_gram():
    """Gram-space layout (fp32 operands): partials, scales, sink, pointer
    slots, then per
    matrix fp32 X, two fp32 X^T, and five fp32 P x P buffers (A, P, P A and
    the Q pair)."""
    a = lambda x: _pad(x, 256)  # noqa: E731
    shapes = [(1024, 256), (256, 1024), (100, 37), (700, 900)]
    tiles, per = 0, 0
    for m, n in shapes:
        p, q = min(m, n), max(m, n)
        t = _tile(p, "f32", gram=True)
        P, Q = _pad(p, t), _pad(q, t)
        tiles += (P // 64) * (Q // 64)
        per += a(4 * P * _ld(Q, 4)) + 2 * a(4 * Q * _ld(P, 4)) + 5 * a(4 * P * _ld(P, 4))
    want = a(4 * tiles) + a(16 * len(shapes)) + a(16) + a(24 * len(shapes)) + per
    for prec in ("f32", "auto"):
        assert dm.workspace_size(shapes, prec, backend="gram") == want


@pytest.mark.parametrize("prec", ["f32", "bf16", "bf16_split", "auto", "bf16_split_a", "f16"])
def test_workspace_size(prec):
    shapes = [(1024, 256), (256, 1024), (100, 37), (4096, 14336), (32, 480), (544, 800),
              (900, 960), (8192, 28672)]
    assert dm.workspace_size(shapes, prec) == _expected_ws(shapes, prec)
    assert dm.workspace_size([], prec) == 0


FAKE_G, FAKE_O, FAKE_B, FAKE_WS = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _call_ns(g, o, cfg, ws=FAKE_WS, ws_bytes=None):
    L = dm.lib()
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return L.dmuon_ns_orthogonalize(ctypes.byref(g) if g is not None else None,
                                    ctypes.byref(o) if o is not None else None,
                                    ctypes.byref(cfg) if cfg is not None else None,
                                    ctypes.c_void_p(ws), ws_bytes, None)


def _call_step(p, g, b, cfg, mu=0.95, lr=0.02, wd=0.0, ws=FAKE_WS, ws_bytes=1 << 40):
    L = dm.lib()
    return L.dmuon_muon_step(ctypes.byref(p), ctypes.byref(g), ctypes.byref(b),
                             ctypes.byref(cfg), mu, lr, wd, 1, ctypes.c_void_p(ws), ws_bytes,
                             None)


def _err():
    return dm.lib().dmuon_last_error().decode()


_KEEP = []


def _keep_cfg(**kw):
    cfg, keep = dm.make_cfg(**kw)
    _KEEP.append(keep)
    return cfg


def _cfg_with(**fields):
    cfg = _keep_cfg(prec="f32", backend="gram")
    for k, v in fields.items():
        setattr(cfg, k, v)
    return cfg


def test_gram_needs_fp32_or_fp16_operands():
    g, k1 = _mats([(64, 96, FAKE_G)])
    o, k2 = _mats([(64, 96, FAKE_O)])
    for prec in ("bf16", "bf16_split", "bf16_split_a"):
        cfg = _keep_cfg(prec=prec, backend="gram")
        assert _call_ns(g, o, cfg) == dm.DMUON_E_UNSUPPORTED, _err()
        assert "fp32" in _err() and "fp16" in _err()
    # fp16 operands pass validation: the first HIP call is reached
    cfg = _keep_cfg(prec="f16", backend="gram")
    assert _call_ns(g, o, cfg) == dm.DMUON_E_HIP, _err()


def test_gram_fp16_coefficient_bound():
    """fp16 Gram NS stores P and Q times 2^10: coefficient tables whose
    per-window bound on |Q| over eigenvalues in [0, 1.25] exceeds 48 are
    rejected before any device work; the quintic (3.4445 per step, 40.9
    over a three-step window) passes."""
    g, k1 = _mats([(64, 96, FAKE_G)])
    o, k2 = _mats([(64, 96, FAKE_O)])
    quintic = [(3.4445, -4.7750, 2.0315)] * 5
    cfg = _keep_cfg(prec="f16", backend="gram", coefficients=quintic)
    assert _call_ns(g, o, cfg) == dm.DMUON_E_HIP, _err()
    # four steps in one window: 3.4445^4 = 140.8 > 48
    cfg = _keep_cfg(prec="f16", backend="gram", coefficients=quintic[:4], restart_iterations=[])
    assert _call_ns(g, o, cfg) == dm.DMUON_E_UNSUPPORTED, _err()
    assert "window 0" in _err()
    # the same table split into windows of two: 11.9 each
    cfg = _keep_cfg(prec="f16", backend="gram", coefficients=quintic[:4],
                    restart_iterations=[2])
    assert _call_ns(g, o, cfg) == dm.DMUON_E_HIP, _err()
    # two quintic steps (11.9), then three steps of the constant 4 (64 > 48):
    # only the second window trips
    late = quintic[:2] + [(4.0, 0.0, 0.0)] * 3
    cfg = _keep_cfg(prec="f16", backend="gram", coefficients=late)
    assert _call_ns(g, o, cfg) == dm.DMUON_E_UNSUPPORTED, _err()
    assert "window 1" in _err()
    # 1 + 40 l (1 - l), 11 at l = 1/2 and -11.5 at l = 1.25: 11.5^2 = 132 > 48
    # in window 0
    bump = [(1.0, 40.0, -40.0)] * 5
    cfg = _keep_cfg(prec="f16", backend="gram", coefficients=bump)
    assert _call_ns(g, o, cfg) == dm.DMUON_E_UNSUPPORTED, _err()
    assert "window 0" in _err()
    # fp32 Gram NS takes any finite table
    cfg = _keep_cfg(prec="f32", backend="gram", coefficients=bump)
    assert _call_ns(g, o, cfg) == dm.DMUON_E_HIP, _err()


def test_valid_call_reaches_the_device():
    # With arguments that pass validation, the first HIP call is reached:
    # on a host without a GPU that is the only failure.
    g, k1 = _mats([(64, 96, FAKE_G)])
    o, k2 = _mats([(64, 96, FAKE_O)])
    cfg, kc = dm.make_cfg(prec="f32")
    st = _call_ns(g, o, cfg)
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if not has_gpu:
        assert st == dm.DMUON_E_HIP, _err()


def test_empty_batch_is_a_noop():
    g, k1 = _mats([])
    o, k2 = _mats([])
    cfg, kc = dm.make_cfg()
    assert _call_ns(g, o, cfg, ws=0, ws_bytes=0) == dm.DMUON_OK
    p, k3 = _mats([])
    b, k4 = _mats([])
    assert _call_step(p, g, b, cfg, ws=0, ws_bytes=0) == dm.DMUON_OK


NS_BAD = {
    "null batch": lambda: (None, _mats([(4, 4, FAKE_O)])[0], dm.make_cfg()[0], {}),
    "null cfg": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_O)])[0], None, {}),
    "count differs": lambda: (_mats([(4, 4, FAKE_G)])[0],
                              _mats([(4, 4, FAKE_O), (4, 4, FAKE_O + 4096)])[0],
                              dm.make_cfg()[0], {}),
    "shape differs": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 5, FAKE_O)])[0],
                              dm.make_cfg()[0], {}),
    "dtype differs": lambda: (_mats([(4, 4, FAKE_G)])[0],
                              _mats([(4, 4, FAKE_O)], dm.DMUON_BF16)[0], dm.make_cfg()[0], {}),
    "unknown dtype": lambda: (_mats([(4, 4, FAKE_G)], 7)[0], _mats([(4, 4, FAKE_O)], 7)[0],
                              dm.make_cfg()[0], {}),
    "zero rows": lambda: (_mats([(0, 4, FAKE_G)])[0], _mats([(0, 4, FAKE_O)])[0],
                          dm.make_cfg()[0], {}),
    "negative cols": lambda: (_mats([(4, -1, FAKE_G)])[0], _mats([(4, -1, FAKE_O)])[0],
                              dm.make_cfg()[0], {}),
    "null pointer": lambda: (_mats([(4, 4, 0)])[0], _mats([(4, 4, FAKE_O)])[0],
                             dm.make_cfg()[0], {}),
    "misaligned f32": lambda: (_mats([(4, 4, FAKE_G + 2)])[0], _mats([(4, 4, FAKE_O)])[0],
                               dm.make_cfg()[0], {}),
    "ns_steps 0": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_O)])[0],
                           dm.make_cfg(ns_steps=0)[0], {}),
    "ns_steps 17": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_O)])[0],
                            dm.make_cfg(ns_steps=17)[0], {}),
    "negative eps": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_O)])[0],
                             dm.make_cfg(eps=-1.0)[0], {}),
    "bad precision": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_O)])[0],
                              dm.make_cfg(prec=9)[0], {}),
    "partial overlap": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_G + 16)])[0],
                                dm.make_cfg()[0], {}),
    "unknown backend": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_O)])[0],
                                dm.make_cfg(backend=7)[0], {}),
    "negative restart": lambda: (_mats([(4, 4, FAKE_G)])[0], _mats([(4, 4, FAKE_O)])[0],
                                 _keep_cfg(prec="f32", backend="gram",
                                           restart_iterations=[2, -1]), {}),
    "restarts count without list": lambda: (_mats([(4, 4, FAKE_G)])[0],
                                            _mats([(4, 4, FAKE_O)])[0],
                                            _cfg_with(nrestarts=2), {}),
    "two inputs overlap": lambda: (_mats([(4, 4, FAKE_G), (4, 4, FAKE_G + 32)])[0],
                                   _mats([(4, 4, FAKE_O), (4, 4, FAKE_O + 4096)])[0],
                                   dm.make_cfg()[0], {}),
    "workspace overlaps": lambda: (_mats([(4, 4, FAKE_WS + 1024)])[0],
                                   _mats([(4, 4, FAKE_O)])[0], dm.make_cfg()[0], {}),
}


@pytest.mark.parametrize("case", sorted(NS_BAD))
def test_ns_rejects(case):
    keep = []
    g, o, cfg, kw = NS_BAD[case]()
    st = _call_ns(g, o, cfg, **kw)
    assert st == dm.DMUON_E_INVALID, (case, st, _err())
    assert _err()


def test_nonfinite_coefficient_rejected():
    cfg, keep = dm.make_cfg(coefficients=[(1.0, float("nan"), 0.0)])
    g, k1 = _mats([(4, 4, FAKE_G)])
    o, k2 = _mats([(4, 4, FAKE_O)])
    assert _call_ns(g, o, cfg) == dm.DMUON_E_INVALID


def test_in_place_alias_allowed_by_validation():
    g, k1 = _mats([(8, 8, FAKE_G)])
    cfg, kc = dm.make_cfg()
    st = _call_ns(g, g, cfg)
    assert st != dm.DMUON_E_INVALID, _err()


def test_workspace_errors():
    g, k1 = _mats([(64, 64, FAKE_G)])
    o, k2 = _mats([(64, 64, FAKE_O)])
    cfg, kc = dm.make_cfg(prec="bf16")
    need = dm.workspace_size([(64, 64)], "bf16")
    assert _call_ns(g, o, cfg, ws=0) == dm.DMUON_E_WORKSPACE
    assert _call_ns(g, o, cfg, ws=FAKE_WS + 64) == dm.DMUON_E_WORKSPACE
    assert _call_ns(g, o, cfg, ws_bytes=need - 1) == dm.DMUON_E_WORKSPACE
    assert "needed" in _err()


def test_oversized_matrix_unsupported():
    g, k1 = _mats([(1 << 21, 4, FAKE_G)])
    o, k2 = _mats([(1 << 21, 4, FAKE_O)])
    cfg, kc = dm.make_cfg()
    assert _call_ns(g, o, cfg) == dm.DMUON_E_UNSUPPORTED
    g, k1 = _mats([(60000, 60000, FAKE_G)])
    o, k2 = _mats([(60000, 60000, FAKE_O)])
    assert _call_ns(g, o, cfg) == dm.DMUON_E_UNSUPPORTED


STEP_BAD = {
    "bufs bf16": dict(bdt=dm.DMUON_BF16),
    "param shape": dict(pshape=(8, 9)),
    "grad aliases buf": dict(gptr=FAKE_B),
    "param overlaps grad": dict(pptr=FAKE_G + 8),
    "nan lr": dict(lr=float("nan")),
    "inf momentum": dict(mu=float("inf")),
}


@pytest.mark.parametrize("case", sorted(STEP_BAD))
def test_step_rejects(case):
    c = STEP_BAD[case]
    p, k1 = _mats([(*c.get("pshape", (8, 8)), c.get("pptr", FAKE_O))])
    g, k2 = _mats([(8, 8, c.get("gptr", FAKE_G))])
    b, k3 = _mats([(8, 8, FAKE_B)], c.get("bdt", dm.DMUON_F32))
    cfg, kc = dm.make_cfg()
    st = _call_step(p, g, b, cfg, mu=c.get("mu", 0.95), lr=c.get("lr", 0.02))
    assert st == dm.DMUON_E_INVALID, (case, st, _err())


# ------------------------------------------------- recorded calls (graphs) --

def _step_graph(p, g, b, cfg, mu=0.95, lr=0.02, ws=FAKE_WS, ws_bytes=1 << 40, out=True):
    h = ctypes.c_void_p(0x1234)
    st = dm.lib().dmuon_muon_step_graph(ctypes.byref(p), ctypes.byref(g), ctypes.byref(b),
                                        ctypes.byref(cfg), mu, lr, 0.0, 1, ctypes.c_void_p(ws),
                                        ws_bytes, ctypes.byref(h) if out else None)
    return st, h


@pytest.mark.parametrize("case", sorted(STEP_BAD))
def test_step_graph_rejects_what_the_step_rejects(case):
    """The graph form validates as the direct call, before anything is
    recorded, and leaves no handle behind."""
    c = STEP_BAD[case]
    p, k1 = _mats([(*c.get("pshape", (8, 8)), c.get("pptr", FAKE_O))])
    g, k2 = _mats([(8, 8, c.get("gptr", FAKE_G))])
    b, k3 = _mats([(8, 8, FAKE_B)], c.get("bdt", dm.DMUON_F32))
    cfg, kc = dm.make_cfg()
    st, h = _step_graph(p, g, b, cfg, mu=c.get("mu", 0.95), lr=c.get("lr", 0.02))
    assert st == dm.DMUON_E_INVALID, (case, st, _err())
    assert not h.value


@pytest.mark.parametrize("case", ["null batch", "shape differs", "partial overlap",
                                  "workspace overlaps", "ns_steps 0"])
def test_ns_graph_rejects_what_ns_rejects(case):
    g, o, cfg, kw = NS_BAD[case]()
    h = ctypes.c_void_p(0x1234)
    st = dm.lib().dmuon_ns_orthogonalize_graph(ctypes.byref(g) if g is not None else None,
                                               ctypes.byref(o), ctypes.byref(cfg),
                                               ctypes.c_void_p(FAKE_WS), 1 << 40,
                                               ctypes.byref(h))
    assert st == dm.DMUON_E_INVALID, (case, st, _err())
    assert not h.value


def test_graph_arguments():
    p, k1 = _mats([(8, 8, FAKE_O)])
    g, k2 = _mats([(8, 8, FAKE_G)])
    b, k3 = _mats([(8, 8, FAKE_B)])
    cfg, kc = dm.make_cfg()
    st, _ = _step_graph(p, g, b, cfg, out=False)
    assert st == dm.DMUON_E_INVALID and "graph" in _err()
    st, _ = _step_graph(p, g, b, cfg, ws_bytes=16)
    assert st == dm.DMUON_E_WORKSPACE, _err()
    e1, e2, e3 = _mats([])[0], _mats([])[0], _mats([])[0]
    st, h = _step_graph(e1, e2, e3, cfg, ws=0, ws_bytes=0)
    assert st == dm.DMUON_E_INVALID and "empty" in _err()
    assert dm.lib().dmuon_graph_launch(None, None) == dm.DMUON_E_INVALID
    dm.lib().dmuon_graph_destroy(None)  # a no-op


def test_python_binding_maps_errors():
    with pytest.raises(ValueError):
        dm.workspace_size([(0, 3)])
    with pytest.raises(dm.DmuonError):
        dm.workspace_size([(1 << 21, 3)])


# ------------------------------------------- clipping and AdamW validation --

FAKE_P, FAKE_M, FAKE_V, FAKE_ST = 0x50000000, 0x60000000, 0x70000000, 0x80000000


def _call_clip(g, buckets=None, nb=1, max_norm=1.0, stats_only=0, p=2.0, stats=FAKE_ST,
               ws=FAKE_WS, ws_bytes=1 << 40):
    bk = None
    if buckets is not None:
        arr = (ctypes.c_int32 * len(buckets))(*buckets)
        bk = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return dm.lib().dmuon_clip_grad_norm(ctypes.byref(g), bk, nb, max_norm, stats_only, p,
                                         stats, ctypes.c_void_p(ws), ws_bytes, None)


def test_clip_workspace_size():
    # per-block fp32 partials (blocks of 16384 elements), then one fp32
    # factor per bucket, each rounded up to 256 bytes
    shapes = [(100, 300), (4096, 14336), (7, 1)]
    blocks = sum(-(-m * n // 16384) for m, n in shapes)
    assert dm.clip_workspace_size(shapes, 3) == _pad(4 * blocks, 256) + _pad(12, 256)
    assert dm.clip_workspace_size([], 1) == 0


CLIP_BAD = {
    "no buckets": dict(nb=0),
    "bucket map missing": dict(nb=2),
    "bucket out of range": dict(buckets=[0, 2], nb=2),
    "negative bucket": dict(buckets=[-1, 0], nb=2),
    "zero norm type": dict(p=0.0),
    "nan norm type": dict(p=float("nan")),
    "negative max_norm": dict(max_norm=-1.0),
    "nan max_norm": dict(max_norm=float("nan")),
    "null stats": dict(stats=0),
    "misaligned stats": dict(stats=FAKE_ST + 4),
    "workspace too small": dict(ws_bytes=16),
    "null workspace": dict(ws=0),
    "stats overlap grads": dict(stats=FAKE_G + 64),
}


@pytest.mark.parametrize("name", sorted(CLIP_BAD))
def test_clip_rejects(name):
    g, k = _mats([(64, 96, FAKE_G), (32, 8, FAKE_G + 64 * 96 * 4)])
    want = dm.DMUON_E_WORKSPACE if "workspace" in name else dm.DMUON_E_INVALID
    assert _call_clip(g, **CLIP_BAD[name]) == want, _err()


def test_clip_stats_only_ignores_max_norm():
    # max_norm is not checked when only measuring: validation passes and the
    # call reaches the device
    g, k = _mats([(64, 96, FAKE_G)])
    st = _call_clip(g, max_norm=float("nan"), stats_only=1)
    assert st in (dm.DMUON_OK, dm.DMUON_E_HIP), _err()
    assert st != dm.DMUON_E_INVALID


def _call_adamw(p, g, m, v, step=1, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.01):
    return dm.lib().dmuon_adamw_step(ctypes.byref(p), ctypes.byref(g), ctypes.byref(m),
                                     ctypes.byref(v), step, lr, b1, b2, eps, wd, None)


def _adam_mats(shape=(16, 8), pd=dm.DMUON_F32, gd=dm.DMUON_F32, md=dm.DMUON_F32,
               gptr=FAKE_G):
    return (_mats([(*shape, FAKE_P)], pd)[0], _mats([(*shape, gptr)], gd)[0],
            _mats([(*shape, FAKE_M)], md)[0], _mats([(*shape, FAKE_V)], dm.DMUON_F32)[0])


ADAMW_BAD = {
    "step 0": (dict(), dict(step=0)),
    "beta1 1": (dict(), dict(b1=1.0)),
    "beta2 negative": (dict(), dict(b2=-0.1)),
    "eps 0": (dict(), dict(eps=0.0)),
    "lr inf": (dict(), dict(lr=float("inf"))),
    "bf16 moments": (dict(md=dm.DMUON_BF16), dict()),
    "grads overlap params": (dict(gptr=FAKE_P + 8), dict()),
}


@pytest.mark.parametrize("name", sorted(ADAMW_BAD))
def test_adamw_rejects(name):
    mk, kw = ADAMW_BAD[name]
    p, g, m, v = _adam_mats(**mk)
    assert _call_adamw(p, g, m, v, **kw) == dm.DMUON_E_INVALID, _err()


def test_adamw_shape_mismatch_rejected():
    p, g, m, v = _adam_mats()
    g2 = _mats([(16, 9, FAKE_G)])[0]
    assert _call_adamw(p, g2, m, v) == dm.DMUON_E_INVALID, _err()


# --- Gram-space NS on shards (dmuon_gram_local_*) ---------------------------

def _expected_local(shapes, transposed):
    """Shard layout: partials, scales, sink, then the bucket (sums of squares
    padded to 256 bytes, every fp32 A back to back), then per matrix fp32 X,
    two fp32 X^T and the four other P x P buffers.  p comes from the flag."""
    a = lambda x: _pad(x, 256)  # noqa: E731
    tiles, per, bucket = 0, 0, a(4 * len(shapes))
    for m, n in shapes:
        p, q = (n, m) if transposed else (m, n)
        t = _tile(p, "f32", gram=True)
        P, Q = _pad(p, t), _pad(q, t)
        tiles += (P // 64) * (Q // 64)
        bucket += a(4 * P * _ld(P, 4))
        per += a(4 * P * _ld(Q, 4)) + 2 * a(4 * Q * _ld(P, 4)) + 4 * a(4 * P * _ld(P, 4))
    head = a(4 * tiles) + a(16 * len(shapes)) + a(16) + a(24 * len(shapes))
    return head + bucket + per, head, bucket


LOCAL_SHAPES = [(1792, 4096), (512, 1024), (100, 37), (37, 300)]


@pytest.mark.parametrize("transposed", [0, 1])
def test_gram_local_layout(transposed):
    total, head, bucket = _expected_local(LOCAL_SHAPES, transposed)
    for prec in ("f32", "auto"):
        assert dm.gram_local_workspace_size(LOCAL_SHAPES, transposed, prec) == total
    off, cnt, win = dm.gram_local_bucket(LOCAL_SHAPES, transposed)
    assert (off, 4 * cnt, win) == (head, bucket, 2)
    assert dm.gram_local_bucket(LOCAL_SHAPES, transposed, restart_iterations=[])[2] == 1
    assert dm.gram_local_bucket(LOCAL_SHAPES, transposed, restart_iterations=[3, 1, 9])[2] == 3
    assert dm.gram_local_bucket(LOCAL_SHAPES, transposed, ns_steps=2)[2] == 1
    assert dm.gram_local_workspace_size([], transposed) == 0
    assert dm.gram_local_bucket([], transposed)[:2] == (0, 0)


def test_gram_local_one_rank_matches_gram_sizes():
    # with the auto orientation, the shard layout is the Gram layout plus the
    # sums of squares
    shapes = [(1024, 256), (256, 1024)]
    got = dm.gram_local_workspace_size(shapes[:1], 1) + dm.gram_local_workspace_size(shapes[1:], 0)
    want = dm.workspace_size(shapes[:1], "f32", "gram") + dm.workspace_size(shapes[1:], "f32", "gram")
    assert got == want + 2 * 256


def _call_local(fn, g, o, transposed, cfg, window=0, ws=FAKE_WS, ws_bytes=1 << 40):
    L = dm.lib()
    args = [ctypes.byref(g), ctypes.byref(o), transposed, ctypes.byref(cfg)]
    if fn == "advance":
        return L.dmuon_gram_local_advance(*args, window, ctypes.c_void_p(ws), ws_bytes, None)
    return L.dmuon_gram_local_begin(*args, ctypes.c_void_p(ws), ws_bytes, None)


LOCAL_BAD = {
    "transposed 2": (dict(transposed=2), dm.DMUON_E_INVALID),
    "direct backend": (dict(cfg=dict(prec="f32")), dm.DMUON_E_INVALID),
    "bf16 operands": (dict(cfg=dict(prec="bf16", backend="gram")), dm.DMUON_E_UNSUPPORTED),
    "fp16 operands": (dict(cfg=dict(prec="f16", backend="gram")), dm.DMUON_E_UNSUPPORTED),
    "window -1": (dict(fn="advance", window=-1), dm.DMUON_E_INVALID),
    "window past the last": (dict(fn="advance", window=2), dm.DMUON_E_INVALID),
    "one window only": (dict(fn="advance", window=1,
                             cfg=dict(prec="f32", backend="gram", restart_iterations=[])),
                        dm.DMUON_E_INVALID),
    "small workspace": (dict(ws_bytes=4096), dm.DMUON_E_WORKSPACE),
    "shape differs": (dict(o=[(64, 97, FAKE_O)]), dm.DMUON_E_INVALID),
}


@pytest.mark.parametrize("name", sorted(LOCAL_BAD))
@pytest.mark.parametrize("fn", ["begin", "advance"])
def test_gram_local_rejects(name, fn):
    spec, want = LOCAL_BAD[name]
    fn = spec.get("fn", fn)
    g, k1 = _mats([(64, 96, FAKE_G)])
    o, k2 = _mats(spec.get("o", [(64, 96, FAKE_O)]))
    cfg = _keep_cfg(**spec.get("cfg", dict(prec="f32", backend="gram")))
    st = _call_local(fn, g, o, spec.get("transposed", 0), cfg, window=spec.get("window", 0),
                     ws_bytes=spec.get("ws_bytes", 1 << 40))
    assert st == want, (name, st, _err())
    assert _err()


def test_gram_local_valid_call_reaches_the_device():
    g, k1 = _mats([(64, 96, FAKE_G)])
    o, k2 = _mats([(64, 96, FAKE_O)])
    cfg = _keep_cfg(prec="f32", backend="gram")
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if not has_gpu:
        for fn in ("begin", "advance"):
            assert _call_local(fn, g, o, 1, cfg, window=1) == dm.DMUON_E_HIP, _err()
