"""Python binding of libdmuon, the MI355X (gfx950) per-owner Muon step.

Argument marshalling only: the names mirror the C ABI in include/dmuon.h
and every step of the computation runs in the library's HIP kernels.  There
is no CPU fallback; if libdmuon.so is missing, the first call fails loudly.
PyTorch is used for device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdmuon.so")

DMUON_OK, DMUON_E_INVALID, DMUON_E_UNSUPPORTED, DMUON_E_WORKSPACE, DMUON_E_HIP = range(5)
DMUON_F32, DMUON_BF16 = 0, 1
PREC = {"f32": 0, "bf16": 1, "bf16_split": 2, "auto": 3, "bf16_split_a": 4, "f16": 5}

# Quintic used when no coefficient list is given.
QUINTIC = (3.4445, -4.7750, 2.0315)


class DmuonError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"dmuon status {status}: {message}")
        self.status = status


class DmuonValueError(DmuonError, ValueError):
    pass


class Mat(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("ptr", ctypes.c_void_p)]


class Batch(ctypes.Structure):
    _fields_ = [("mats", ctypes.POINTER(Mat)), ("count", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class NsCfg(ctypes.Structure):
    _fields_ = [("coeffs", ctypes.POINTER(ctypes.c_float)), ("ns_steps", ctypes.c_int32),
                ("eps", ctypes.c_float), ("prec", ctypes.c_int32), ("backend", ctypes.c_int32),
                ("nrestarts", ctypes.c_int32), ("restarts", ctypes.POINTER(ctypes.c_int32))]


BACKEND = {"direct": 0, "gram": 1}


class ProfileRow(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("kind", ctypes.c_int32),
                ("launches", ctypes.c_int32),
                ("ms", ctypes.c_double), ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class ClipStats(ctypes.Structure):
    _fields_ = [("total_norm", ctypes.c_double), ("clip_coef", ctypes.c_double),
                ("clipped", ctypes.c_int32), ("found_inf", ctypes.c_int32),
                ("param_count", ctypes.c_int64)]


EXPORTS = ("dmuon_ns_workspace_size", "dmuon_ns_orthogonalize", "dmuon_muon_step",
           "dmuon_gram_local_workspace_size", "dmuon_gram_local_bucket",
           "dmuon_gram_local_begin", "dmuon_gram_local_advance",
           "dmuon_clip_workspace_size", "dmuon_clip_grad_norm", "dmuon_adamw_step",
           "dmuon_status_str", "dmuon_last_error", "dmuon_backend_info",
           "dmuon_profile_begin", "dmuon_profile_end", "dmuon_plan_builds",
           "dmuon_muon_step_noalloc", "dmuon_muon_step_graph",
           "dmuon_ns_orthogonalize_graph", "dmuon_graph_launch", "dmuon_graph_destroy")

_lib = None


def lib():
    """Loads libdmuon.so (built in-tree by newton_schulz_06_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m newton_schulz_06_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    L.dmuon_ns_workspace_size.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(NsCfg),
                                          ctypes.POINTER(ctypes.c_size_t)]
    L.dmuon_ns_workspace_size.restype = st
    L.dmuon_ns_orthogonalize.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Batch),
                                         ctypes.POINTER(NsCfg), ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
    L.dmuon_ns_orthogonalize.restype = st
    L.dmuon_muon_step.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Batch),
                                  ctypes.POINTER(Batch), ctypes.POINTER(NsCfg),
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
    L.dmuon_muon_step.restype = st
    L.dmuon_muon_step_noalloc.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Batch),
                                          ctypes.POINTER(Batch), ctypes.POINTER(NsCfg),
                                          ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_int32, ctypes.c_void_p]
    L.dmuon_muon_step_noalloc.restype = st
    gp = ctypes.POINTER(ctypes.c_void_p)
    L.dmuon_muon_step_graph.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Batch),
                                        ctypes.POINTER(Batch), ctypes.POINTER(NsCfg),
                                        ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, gp]
    L.dmuon_muon_step_graph.restype = st
    L.dmuon_ns_orthogonalize_graph.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Batch),
                                               ctypes.POINTER(NsCfg), ctypes.c_void_p,
                                               ctypes.c_size_t, gp]
    L.dmuon_ns_orthogonalize_graph.restype = st
    L.dmuon_graph_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.dmuon_graph_launch.restype = st
    L.dmuon_graph_destroy.argtypes = [ctypes.c_void_p]
    L.dmuon_graph_destroy.restype = None
    L.dmuon_gram_local_workspace_size.argtypes = [ctypes.POINTER(Batch), ctypes.c_int32,
                                                  ctypes.POINTER(NsCfg),
                                                  ctypes.POINTER(ctypes.c_size_t)]
    L.dmuon_gram_local_workspace_size.restype = st
    L.dmuon_gram_local_bucket.argtypes = [ctypes.POINTER(Batch), ctypes.c_int32,
                                          ctypes.POINTER(NsCfg), ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int32)]
    L.dmuon_gram_local_bucket.restype = st
    L.dmuon_gram_local_begin.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Batch),
                                         ctypes.c_int32, ctypes.POINTER(NsCfg), ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
    L.dmuon_gram_local_begin.restype = st
    L.dmuon_gram_local_advance.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Batch),
                                           ctypes.c_int32, ctypes.POINTER(NsCfg),
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]
    L.dmuon_gram_local_advance.restype = st
    L.dmuon_clip_workspace_size.argtypes = [ctypes.POINTER(Batch), ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_size_t)]
    L.dmuon_clip_workspace_size.restype = st
    L.dmuon_clip_grad_norm.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(ctypes.c_int32),
                                       ctypes.c_int32, ctypes.c_double, ctypes.c_int32,
                                       ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
    L.dmuon_clip_grad_norm.restype = st
    L.dmuon_adamw_step.argtypes = [ctypes.POINTER(Batch)] * 4 + [
        ctypes.c_int64, ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
        ctypes.c_double, ctypes.c_void_p]
    L.dmuon_adamw_step.restype = st
    L.dmuon_status_str.argtypes = [ctypes.c_int]
    L.dmuon_status_str.restype = ctypes.c_char_p
    L.dmuon_last_error.argtypes = []
    L.dmuon_last_error.restype = ctypes.c_char_p
    L.dmuon_backend_info.argtypes = []
    L.dmuon_backend_info.restype = ctypes.c_char_p
    L.dmuon_profile_begin.argtypes = [ctypes.c_uint32]
    L.dmuon_profile_begin.restype = ctypes.c_int32
    L.dmuon_profile_end.argtypes = [ctypes.POINTER(ProfileRow), ctypes.c_int32]
    L.dmuon_profile_end.restype = ctypes.c_int32
    L.dmuon_plan_builds.argtypes = []
    L.dmuon_plan_builds.restype = ctypes.c_int64
    _lib = L
    return L


def _check(status):
    if status == DMUON_OK:
        return
    msg = lib().dmuon_last_error().decode()
    if status == DMUON_E_INVALID:
        raise DmuonValueError(status, msg)
    raise DmuonError(status, msg)


# ------------------------------------------------------------ marshalling --

def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return DMUON_F32
    if t.dtype == torch.bfloat16:
        return DMUON_BF16
    raise DmuonValueError(DMUON_E_INVALID, f"unsupported dtype {t.dtype}")


def make_batch(tensors):
    """Batch descriptor over 2D contiguous device tensors of one dtype.
    Returns (Batch, keepalive)."""
    tensors = list(tensors)
    arr = (Mat * max(1, len(tensors)))()
    code = DMUON_F32
    for i, t in enumerate(tensors):
        if t.dim() != 2:
            raise DmuonValueError(DMUON_E_INVALID, "every matrix must be 2D")
        if not t.is_contiguous():
            raise DmuonValueError(DMUON_E_INVALID, "every matrix must be contiguous")
        c = _dtype_code(t)
        if i == 0:
            code = c
        elif c != code:
            raise DmuonValueError(DMUON_E_INVALID, "a batch holds one dtype")
        arr[i] = Mat(int(t.shape[0]), int(t.shape[1]), int(t.data_ptr()))
    return Batch(arr, len(tensors), code), arr


def make_flat_batch(tensors):
    """Batch descriptor for the element-wise entry points: any contiguous
    device tensor, described as (first dim) x (the rest), or 1 x n for a
    vector.  Returns (Batch, keepalive)."""
    tensors = list(tensors)
    arr = (Mat * max(1, len(tensors)))()
    code = DMUON_F32
    for i, t in enumerate(tensors):
        if not t.is_contiguous():
            raise DmuonValueError(DMUON_E_INVALID, "every tensor must be contiguous")
        c = _dtype_code(t)
        if i == 0:
            code = c
        elif c != code:
            raise DmuonValueError(DMUON_E_INVALID, "a batch holds one dtype")
        if t.dim() == 0 or t.numel() == 0:
            raise DmuonValueError(DMUON_E_INVALID, "empty tensors are not supported")
        m = int(t.shape[0]) if t.dim() > 1 else 1
        arr[i] = Mat(m, int(t.numel()) // m, int(t.data_ptr()))
    return Batch(arr, len(tensors), code), arr


def shape_batch(shapes, dtype=DMUON_BF16):
    arr = (Mat * max(1, len(shapes)))()
    for i, (m, n) in enumerate(shapes):
        arr[i] = Mat(int(m), int(n), None)
    return Batch(arr, len(shapes), dtype), arr


def make_cfg(coefficients=None, ns_steps=5, eps=1e-7, prec="bf16", backend="direct",
             restart_iterations=None):
    """NS configuration.  ``backend``: "direct" or "gram"; for "gram",
    ``restart_iterations`` None means DMuon's default [2]."""
    if isinstance(prec, str):
        prec = PREC[prec]
    if isinstance(backend, str):
        backend = BACKEND[backend]
    keep = []
    ptr = None
    if coefficients is not None:
        flat = [float(v) for row in coefficients for v in row]
        if len(flat) != 3 * len(coefficients):
            raise DmuonValueError(DMUON_E_INVALID, "coefficient rows must be (a, b, c)")
        ns_steps = len(coefficients)
        arr = (ctypes.c_float * len(flat))(*flat)
        keep.append(arr)
        ptr = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    rptr, nr = None, 0
    if restart_iterations is not None:
        r = [int(v) for v in restart_iterations]
        arr = (ctypes.c_int32 * max(1, len(r)))(*r)
        keep.append(arr)
        rptr, nr = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), len(r)
    return NsCfg(ptr, int(ns_steps), float(eps), int(prec), int(backend), nr, rptr), keep


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


# ------------------------------------------------------------------- API --

def backend_info() -> str:
    return lib().dmuon_backend_info().decode()


def workspace_size(shapes, prec="bf16", backend="direct") -> int:
    """dmuon_ns_workspace_size for a list of (m, n) shapes."""
    b, keep = shape_batch(shapes)
    cfg, ck = make_cfg(prec=prec, backend=backend)
    out = ctypes.c_size_t(0)
    _check(lib().dmuon_ns_workspace_size(ctypes.byref(b), ctypes.byref(cfg), ctypes.byref(out)))
    return int(out.value)


def alloc_workspace(shapes, prec="bf16", device="cuda", backend="direct"):
    """Device workspace (a torch uint8 tensor) big enough for these shapes."""
    import torch
    return torch.empty(max(1, workspace_size(shapes, prec, backend)), dtype=torch.uint8,
                       device=device)


def _ws(workspace, shapes, prec, device, backend="direct", stream=None):
    """The caller's workspace, or a new one for this call.  A new one is
    allocated with `stream` current, so torch's caching allocator keeps the
    block for work on that stream: the kernels still use it after the call
    returns, and a block freed from another stream could be handed out again
    while they run."""
    if workspace is None:
        import torch
        if stream is None:
            workspace = alloc_workspace(shapes, prec, device, backend)
        else:
            with torch.cuda.stream(stream):
                workspace = alloc_workspace(shapes, prec, device, backend)
    return workspace, ctypes.c_void_p(int(workspace.data_ptr())), int(workspace.numel())


def plan_builds() -> int:
    """dmuon_plan_builds: launch tables built so far in this process."""
    return int(lib().dmuon_plan_builds())


def ns_orthogonalize(gs, outs=None, *, coefficients=None, ns_steps=5, eps=1e-7, prec="bf16",
                     backend="direct", restart_iterations=None, workspace=None, stream=None):
    """dmuon_ns_orthogonalize: outs[i] = NS(gs[i]) in gs[i]'s dtype.
    `outs` defaults to new tensors; passing `outs=gs` works in place."""
    import torch
    gs = list(gs)
    if outs is None:
        outs = [torch.empty_like(g) for g in gs]
    outs = list(outs)
    bg, kg = make_batch(gs)
    bo, ko = make_batch(outs)
    cfg, kc = make_cfg(coefficients, ns_steps, eps, prec, backend, restart_iterations)
    device = gs[0].device if gs else "cuda"
    ws, wptr, wbytes = _ws(workspace, [tuple(g.shape) for g in gs], prec, device, backend,
                           stream)
    _check(lib().dmuon_ns_orthogonalize(ctypes.byref(bg), ctypes.byref(bo), ctypes.byref(cfg),
                                        wptr, wbytes, _stream_handle(stream)))
    return outs


def muon_step(params, grads, bufs, *, lr=0.02, momentum=0.95, weight_decay=0.0, nesterov=True,
              coefficients=None, ns_steps=5, eps=1e-7, prec="bf16", backend="direct",
              restart_iterations=None, workspace=None, stream=None):
    """dmuon_muon_step: in-place update of `params` and `bufs` (defaults as
    in DMuon's Muon signature)."""
    params, grads, bufs = list(params), list(grads), list(bufs)
    bp, kp = make_batch(params)
    bg, kg = make_batch(grads)
    bb, kb = make_batch(bufs)
    cfg, kc = make_cfg(coefficients, ns_steps, eps, prec, backend, restart_iterations)
    device = grads[0].device if grads else "cuda"
    ws, wptr, wbytes = _ws(workspace, [tuple(g.shape) for g in grads], prec, device, backend,
                           stream)
    _check(lib().dmuon_muon_step(ctypes.byref(bp), ctypes.byref(bg), ctypes.byref(bb),
                                 ctypes.byref(cfg), float(momentum), float(lr),
                                 float(weight_decay), int(bool(nesterov)), wptr, wbytes,
                                 _stream_handle(stream)))


def muon_step_noalloc(params, grads, bufs, *, lr=0.02, momentum=0.95, weight_decay=0.0,
                      nesterov=True, coefficients=None, ns_steps=5, eps=1e-7, prec="bf16",
                      stream=None):
    """dmuon_muon_step_noalloc: as :func:`muon_step`, with the library's
    static device scratch instead of a workspace (nothing is allocated)."""
    params, grads, bufs = list(params), list(grads), list(bufs)
    bp, kp = make_batch(params)
    bg, kg = make_batch(grads)
    bb, kb = make_batch(bufs)
    cfg, kc = make_cfg(coefficients, ns_steps, eps, prec, "direct", None)
    _check(lib().dmuon_muon_step_noalloc(ctypes.byref(bp), ctypes.byref(bg), ctypes.byref(bb),
                                         ctypes.byref(cfg), float(momentum), float(lr),
                                         float(weight_decay), int(bool(nesterov)),
                                         _stream_handle(stream)))


KINDS = ("momentum", "input", "norm", "syrk", "poly", "update_x", "clip_norm", "clip_scale",
         "adamw", "gram_mul", "gram_x")


class profile:
    """Context manager around dmuon_profile_begin / dmuon_profile_end.
    ``kinds``: kernel names to time (default all).  After exit, ``rows``
    maps kernel name -> dict(launches, ms, flops, bytes)."""

    def __init__(self, kinds=None):
        self.mask = 0
        for k in kinds or ():
            self.mask |= 1 << KINDS.index(k)

    def __enter__(self):
        self.rows = {}
        lib().dmuon_profile_begin(self.mask)
        return self

    def __exit__(self, *exc):
        out = (ProfileRow * 16)()
        n = lib().dmuon_profile_end(out, 16)
        if n < 0:
            _check(DMUON_E_HIP)
        for r in out[:n]:
            self.rows[r.name.decode()] = dict(launches=r.launches, ms=r.ms, flops=r.flops,
                                              bytes=r.bytes)
        return False


class Graph:
    """A recorded call (dmuon_muon_step_graph / dmuon_ns_orthogonalize_graph):
    ``g(stream=None)`` enqueues one replay (dmuon_graph_launch); the graph is
    destroyed with this object.  ``keep`` holds the recorded buffers."""

    def __init__(self, handle, keep):
        self.handle = handle
        self._keep = keep
        self._destroy = lib().dmuon_graph_destroy

    def __call__(self, stream=None):
        st = lib().dmuon_graph_launch(self.handle, _stream_handle(stream))
        if st:
            _check(st)

    def close(self):
        if self.handle:
            self._destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def muon_step_graph(params, grads, bufs, *, lr=0.02, momentum=0.95, weight_decay=0.0,
                    nesterov=True, coefficients=None, ns_steps=5, eps=1e-7, prec="bf16",
                    backend="direct", restart_iterations=None, workspace=None):
    """dmuon_muon_step_graph: records one Muon step on these buffers; call
    the returned :class:`Graph` to run it."""
    params, grads, bufs = list(params), list(grads), list(bufs)
    bp, kp = make_batch(params)
    bg, kg = make_batch(grads)
    bb, kb = make_batch(bufs)
    cfg, kc = make_cfg(coefficients, ns_steps, eps, prec, backend, restart_iterations)
    ws, wptr, wbytes = _ws(workspace, [tuple(g.shape) for g in grads], prec, grads[0].device,
                           backend)
    h = ctypes.c_void_p()
    _check(lib().dmuon_muon_step_graph(ctypes.byref(bp), ctypes.byref(bg), ctypes.byref(bb),
                                       ctypes.byref(cfg), float(momentum), float(lr),
                                       float(weight_decay), int(bool(nesterov)), wptr, wbytes,
                                       ctypes.byref(h)))
    return Graph(h, (params, grads, bufs, ws))


def ns_orthogonalize_graph(gs, outs, *, coefficients=None, ns_steps=5, eps=1e-7, prec="bf16",
                           backend="direct", restart_iterations=None, workspace=None):
    """dmuon_ns_orthogonalize_graph: records outs[i] = NS(gs[i]); call the
    returned :class:`Graph` to run it."""
    gs, outs = list(gs), list(outs)
    bg, kg = make_batch(gs)
    bo, ko = make_batch(outs)
    cfg, kc = make_cfg(coefficients, ns_steps, eps, prec, backend, restart_iterations)
    ws, wptr, wbytes = _ws(workspace, [tuple(g.shape) for g in gs], prec, gs[0].device, backend)
    h = ctypes.c_void_p()
    _check(lib().dmuon_ns_orthogonalize_graph(ctypes.byref(bg), ctypes.byref(bo),
                                              ctypes.byref(cfg), wptr, wbytes, ctypes.byref(h)))
    return Graph(h, (gs, outs, ws))


class PreparedMuonStep:
    """dmuon_muon_step with the descriptors marshalled once, for repeated
    calls on fixed buffers (one gradient batch per call, chosen by index).
    ``graph=True`` records each gradient batch's step once
    (dmuon_muon_step_graph) and replays it on later calls."""

    def __init__(self, params, bufs, grad_sets, *, lr=0.02, momentum=0.95, weight_decay=0.0,
                 nesterov=True, coefficients=None, ns_steps=5, eps=1e-7, prec="bf16",
                 backend="direct", restart_iterations=None, workspace=None, stream=None,
                 graph=False):
        self._keep = []
        self.bp, k = make_batch(params); self._keep.append(k)
        self.bb, k = make_batch(bufs); self._keep.append(k)
        self.bgs = []
        for gs in grad_sets:
            b, k = make_batch(gs)
            self.bgs.append(b)
            self._keep.append(k)
        self.cfg, k = make_cfg(coefficients, ns_steps, eps, prec, backend, restart_iterations)
        self._keep.append(k)
        shapes = [tuple(p.shape) for p in params]
        self.ws, self.wptr, self.wbytes = _ws(workspace, shapes, prec, params[0].device, backend,
                                              stream)
        self.stream = _stream_handle(stream)
        self.scalars = (ctypes.c_float(momentum), ctypes.c_float(lr),
                        ctypes.c_float(weight_decay), ctypes.c_int32(int(bool(nesterov))))
        self.fn = lib().dmuon_muon_step
        self.graphs = [None] * len(self.bgs) if graph else None
        self._launch = lib().dmuon_graph_launch

    def record(self):
        """Records every gradient batch's graph now (graph=True), so that
        later calls only replay."""
        for i in range(len(self.bgs)):
            if self.graphs[i] is None:
                self._graph(i)

    def _graph(self, i):
        h = ctypes.c_void_p()
        _check(lib().dmuon_muon_step_graph(ctypes.byref(self.bp), ctypes.byref(self.bgs[i]),
                                           ctypes.byref(self.bb), ctypes.byref(self.cfg),
                                           *self.scalars, self.wptr, self.wbytes,
                                           ctypes.byref(h)))
        self.graphs[i] = Graph(h, None)
        return self.graphs[i]

    def __call__(self, i=0):
        if self.graphs is not None:
            g = self.graphs[i] or self._graph(i)
            st = self._launch(g.handle, self.stream)
        else:
            st = self.fn(ctypes.byref(self.bp), ctypes.byref(self.bgs[i]), ctypes.byref(self.bb),
                         ctypes.byref(self.cfg), *self.scalars, self.wptr, self.wbytes,
                         self.stream)
        if st:
            _check(st)


class PreparedNs:
    """dmuon_ns_orthogonalize with the descriptors marshalled once."""

    def __init__(self, gs, outs, *, coefficients=None, ns_steps=5, eps=1e-7, prec="bf16",
                 backend="direct", restart_iterations=None, workspace=None, stream=None,
                 graph=False):
        self.bg, self._kg = make_batch(gs)
        self.bo, self._ko = make_batch(outs)
        self.cfg, self._kc = make_cfg(coefficients, ns_steps, eps, prec, backend,
                                      restart_iterations)
        shapes = [tuple(g.shape) for g in gs]
        self.ws, self.wptr, self.wbytes = _ws(workspace, shapes, prec, gs[0].device, backend,
                                              stream)
        self.stream = _stream_handle(stream)
        self.fn = lib().dmuon_ns_orthogonalize
        self.graph = None
        if graph:
            h = ctypes.c_void_p()
            _check(lib().dmuon_ns_orthogonalize_graph(ctypes.byref(self.bg), ctypes.byref(self.bo),
                                                      ctypes.byref(self.cfg), self.wptr,
                                                      self.wbytes, ctypes.byref(h)))
            self.graph = Graph(h, None)
        self._launch = lib().dmuon_graph_launch

    def __call__(self):
        if self.graph is not None:
            st = self._launch(self.graph.handle, self.stream)
        else:
            st = self.fn(ctypes.byref(self.bg), ctypes.byref(self.bo), ctypes.byref(self.cfg),
                         self.wptr, self.wbytes, self.stream)
        if st:
            _check(st)


# --------------------------------------------- Gram-space NS on shards --

def gram_local_workspace_size(shapes, transposed, prec="f32") -> int:
    """dmuon_gram_local_workspace_size for blocks of these (m, n) shapes."""
    b, keep = shape_batch(shapes)
    cfg, ck = make_cfg(prec=prec, backend="gram")
    out = ctypes.c_size_t(0)
    _check(lib().dmuon_gram_local_workspace_size(ctypes.byref(b), int(transposed),
                                                 ctypes.byref(cfg), ctypes.byref(out)))
    return int(out.value)


def gram_local_bucket(shapes, transposed, *, coefficients=None, ns_steps=5, prec="f32",
                      restart_iterations=None):
    """dmuon_gram_local_bucket: (byte offset, float count, windows)."""
    b, keep = shape_batch(shapes)
    cfg, ck = make_cfg(coefficients, ns_steps, 1e-7, prec, "gram", restart_iterations)
    off, cnt, win = ctypes.c_size_t(0), ctypes.c_int64(0), ctypes.c_int32(0)
    _check(lib().dmuon_gram_local_bucket(ctypes.byref(b), int(transposed), ctypes.byref(cfg),
                                         ctypes.byref(off), ctypes.byref(cnt), ctypes.byref(win)))
    return int(off.value), int(cnt.value), int(win.value)


class GramLocal:
    """dmuon_gram_local_begin / dmuon_gram_local_advance on fixed buffers:
    Gram-space NS of this rank's blocks (DMuon "API Reference",
    gram_newton_schulz_distributed_local, batched).  ``bucket`` is a float32
    view of the workspace that must be summed over the shard group before
    each ``advance``; ``__call__`` runs the whole sequence with an optional
    ``all_reduce(bucket)`` (None: one rank, the block is the whole matrix)."""

    def __init__(self, g_locals, outs, *, transposed, coefficients=None, ns_steps=5, eps=1e-7,
                 prec="f32", restart_iterations=None, workspace=None, stream=None):
        import torch
        self.bg, self._kg = make_batch(g_locals)
        self.bo, self._ko = make_batch(outs)
        self.transposed = int(bool(transposed))
        self.cfg, self._kc = make_cfg(coefficients, ns_steps, eps, prec, "gram",
                                      restart_iterations)
        shapes = [tuple(g.shape) for g in g_locals]
        if workspace is None:
            device = g_locals[0].device if g_locals else "cuda"
            nbytes = max(1, gram_local_workspace_size(shapes, transposed, prec))
            # allocated with the launch stream current (see _ws)
            with torch.cuda.stream(stream if stream is not None
                                   else torch.cuda.current_stream(device)):
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.ws = workspace
        self.wptr = ctypes.c_void_p(int(workspace.data_ptr()))
        self.wbytes = int(workspace.numel())
        off, cnt, self.windows = gram_local_bucket(
            shapes, transposed, coefficients=coefficients, ns_steps=ns_steps, prec=prec,
            restart_iterations=restart_iterations)
        self.bucket = workspace[off:off + 4 * cnt].view(torch.float32)
        self.stream = _stream_handle(stream)
        self.L = lib()

    def begin(self):
        _check(self.L.dmuon_gram_local_begin(ctypes.byref(self.bg), ctypes.byref(self.bo),
                                             self.transposed, ctypes.byref(self.cfg), self.wptr,
                                             self.wbytes, self.stream))

    def advance(self, window):
        _check(self.L.dmuon_gram_local_advance(ctypes.byref(self.bg), ctypes.byref(self.bo),
                                               self.transposed, ctypes.byref(self.cfg),
                                               int(window), self.wptr, self.wbytes,
                                               self.stream))

    def __call__(self, all_reduce=None):
        self.begin()
        for w in range(self.windows):
            if all_reduce is not None:
                all_reduce(self.bucket)
            self.advance(w)


def gram_ns_distributed_local(g_locals, outs=None, *, transposed, all_reduce=None,
                              coefficients=None, ns_steps=5, eps=1e-7, prec="f32",
                              restart_iterations=None, workspace=None, stream=None):
    """Gram-space NS of this rank's column blocks (see :class:`GramLocal`);
    returns ``outs`` (new tensors by default; ``outs=g_locals`` works in
    place)."""
    import torch
    g_locals = list(g_locals)
    outs = [torch.empty_like(g) for g in g_locals] if outs is None else list(outs)
    GramLocal(g_locals, outs, transposed=transposed, coefficients=coefficients,
              ns_steps=ns_steps, eps=eps, prec=prec, restart_iterations=restart_iterations,
              workspace=workspace, stream=stream)(all_reduce)
    return outs


# ------------------------------------------------- element-wise companions --

def clip_workspace_size(shapes, nbuckets=1) -> int:
    """dmuon_clip_workspace_size for gradients of these (m, n) shapes."""
    b, keep = shape_batch(shapes)
    out = ctypes.c_size_t(0)
    _check(lib().dmuon_clip_workspace_size(ctypes.byref(b), int(nbuckets), ctypes.byref(out)))
    return int(out.value)


class PreparedClip:
    """dmuon_clip_grad_norm with the descriptors marshalled once.  Calling it
    enqueues the clipping on the stream; ``stats()`` waits for the stream and
    returns one dict per bucket (total_norm, clip_coef, clipped, found_inf,
    param_count)."""

    def __init__(self, grads, max_norm, *, norm_type=2.0, buckets=None, stream=None):
        import torch
        grads = list(grads)
        self.bg, self._kg = make_flat_batch(grads)
        self.nb = 1 if buckets is None else max(buckets) + 1
        self._bk = None
        bptr = None
        if buckets is not None:
            if len(buckets) != len(grads):
                raise DmuonValueError(DMUON_E_INVALID, "one bucket index per gradient")
            self._bk = (ctypes.c_int32 * len(buckets))(*[int(b) for b in buckets])
            bptr = ctypes.cast(self._bk, ctypes.POINTER(ctypes.c_int32))
        self.bptr = bptr
        self.stats_only = max_norm is None
        self.max_norm = 0.0 if max_norm is None else float(max_norm)
        self.norm_type = float(norm_type)
        device = grads[0].device if grads else "cuda"
        shapes = [(self.bg.mats[i].m, self.bg.mats[i].n) for i in range(len(grads))]
        self.ws = torch.empty(max(1, clip_workspace_size(shapes, self.nb)), dtype=torch.uint8,
                              device=device)
        self.dev_stats = torch.empty(ctypes.sizeof(ClipStats) * self.nb, dtype=torch.uint8,
                                     device=device)
        self.stream = _stream_handle(stream)
        self.fn = lib().dmuon_clip_grad_norm

    def __call__(self, max_norm=None):
        """Enqueues the clipping; ``max_norm`` overrides the prepared value."""
        mx = self.max_norm if max_norm is None else float(max_norm)
        st = self.fn(ctypes.byref(self.bg), self.bptr, self.nb, mx,
                     int(self.stats_only), self.norm_type, int(self.dev_stats.data_ptr()),
                     int(self.ws.data_ptr()), int(self.ws.numel()), self.stream)
        if st:
            _check(st)

    def stats(self):
        raw = bytes(self.dev_stats.cpu().numpy())
        out = []
        for b in range(self.nb):
            r = ClipStats.from_buffer_copy(raw, b * ctypes.sizeof(ClipStats))
            out.append(dict(total_norm=r.total_norm, clip_coef=r.clip_coef,
                            clipped=bool(r.clipped), found_inf=bool(r.found_inf),
                            param_count=int(r.param_count)))
        return out


def clip_grad_norm(grads, max_norm, *, norm_type=2.0, buckets=None, stream=None):
    """dmuon_clip_grad_norm on `grads` (in place); returns the per-bucket
    stats (waits for the stream).  ``max_norm=None`` only measures."""
    c = PreparedClip(grads, max_norm, norm_type=norm_type, buckets=buckets, stream=stream)
    c()
    return c.stats()


ADAMW_DEFAULTS = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)


class PreparedAdamW:
    """dmuon_adamw_step with the descriptors marshalled once; ``__call__(step)``
    enqueues one update with the given 1-based step count."""

    def __init__(self, params, grads, exp_avg, exp_avg_sq, *, lr=1e-3, betas=(0.9, 0.999),
                 eps=1e-8, weight_decay=0.01, stream=None):
        self._k = []
        self.b = []
        for ts in (params, grads, exp_avg, exp_avg_sq):
            b, k = make_flat_batch(ts)
            self.b.append(b)
            self._k.append(k)
        self.hp = (float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay))
        self.stream = _stream_handle(stream)
        self.fn = lib().dmuon_adamw_step

    def __call__(self, step):
        st = self.fn(*[ctypes.byref(b) for b in self.b], int(step), *self.hp, self.stream)
        if st:
            _check(st)


def adamw_step(params, grads, exp_avg, exp_avg_sq, step, *, lr=1e-3, betas=(0.9, 0.999),
               eps=1e-8, weight_decay=0.01, stream=None):
    """dmuon_adamw_step: in-place AdamW update of `params`, `exp_avg` and
    `exp_avg_sq` (defaults as in the adamw_* arguments of DMuon's Muon)."""
    PreparedAdamW(params, grads, exp_avg, exp_avg_sq, lr=lr, betas=betas, eps=eps,
                  weight_decay=weight_decay, stream=stream)(step)
