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


def _tile(p, prec):
    if prec == "f32":
        return 64 if p <= 512 else 128

    def fits(t):
        return _pad(p, t) * 8 <= p * 9

    if p >= 1024 and fits(256):
        return 256
    if p >= 768 and fits(128):
        return 128
    return 64


def _expected_ws(shapes, prec):
    """Workspace rule: partials, scales and a 16-byte sink, then per matrix
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
        P, Q = _pad(p, t), _pad(q, t)
        tiles += (P // 64) * (Q // 64)
        split_b = prec == "bf16_split" or (prec == "auto" and p <= 128)
        split_a = prec in ("bf16_split", "bf16_split_a") or (prec == "auto" and p <= 1024)
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
    return a(4 * tiles) + a(16 * len(shapes)) + a(16) + sum(per)


@pytest.mark.parametrize("prec", ["f32", "bf16", "bf16_split", "auto", "bf16_split_a"])
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


def test_python_binding_maps_errors():
    with pytest.raises(ValueError):
        dm.workspace_size([(0, 3)])
    with pytest.raises(dm.DmuonError):
        dm.workspace_size([(1 << 21, 3)])
