"""Python binding of libmita.so, the MiTA forward pass for MI355X (gfx950).

Argument marshalling only: every step of the pass runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the stream; the
functions here check that tensors are contiguous device tensors of the right
dtype and shape, allocate outputs and workspace with torch, and pass raw
pointers through ctypes.  The names mirror the C entry points of
``include/mita.h``.  If the library is not built, every call raises: there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmita.so")

MITA_OK, MITA_ERR_INVALID_ARG, MITA_ERR_UNSUPPORTED, MITA_ERR_WORKSPACE, MITA_ERR_HIP = range(5)
MITA_F32, MITA_BF16 = 0, 1
PATHS = {"auto": 0, "fused": 1, "staged": 2}

# Every symbol include/mita.h declares.
EXPORTS = [
    "mita_status_string", "mita_last_error", "mita_version", "mita_workspace_bytes",
    "mita_workspace_bytes_ex", "mita_schedule", "mita_kernel_names", "mita_sync_event_create",
    "mita_forward", "mita_forward_ex", "mita_forward_noalloc", "mita_backward",
    "mita_backward_workspace_bytes", "mita_pool", "mita_landmark_workspace_bytes",
    "mita_landmark", "mita_route_workspace_bytes", "mita_route", "mita_attend",
]


class MitaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class _Extras(ctypes.Structure):
    _fields_ = [("ql", ctypes.c_void_p), ("vl", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("path", ctypes.c_int),
                ("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int),
                ("side_stream", ctypes.c_void_p), ("fork_event", ctypes.c_void_p),
                ("join_event", ctypes.c_void_p), ("s", ctypes.c_int), ("route_only", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmita.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m "
                               "efficient_attention_avg_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int
        L.mita_status_string.restype = ctypes.c_char_p
        L.mita_status_string.argtypes = [I]
        L.mita_last_error.restype = ctypes.c_char_p
        L.mita_last_error.argtypes = []
        L.mita_version.restype = ctypes.c_char_p
        L.mita_version.argtypes = []
        L.mita_workspace_bytes.restype = Z
        L.mita_workspace_bytes.argtypes = [I] * 8 + [I]
        L.mita_workspace_bytes_ex.restype = Z
        L.mita_workspace_bytes_ex.argtypes = [I] * 8 + [I, ctypes.POINTER(_Extras)]
        L.mita_schedule.restype = I
        L.mita_schedule.argtypes = [I] * 8 + [I]
        L.mita_kernel_names.restype = I
        L.mita_kernel_names.argtypes = [I] * 8 + [I, ctypes.POINTER(_Extras),
                                                 ctypes.POINTER(ctypes.c_char_p),
                                                 ctypes.POINTER(ctypes.c_int), I]
        L.mita_sync_event_create.restype = S
        L.mita_sync_event_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.mita_forward.restype = S
        L.mita_forward.argtypes = [P, P, P] + [I] * 8 + [I, P, P, P, P, Z, P]
        L.mita_backward_workspace_bytes.restype = Z
        L.mita_backward_workspace_bytes.argtypes = [I] * 8 + [I, ctypes.POINTER(_Extras)]
        L.mita_backward.restype = S
        L.mita_backward.argtypes = [P, P, P, P] + [I] * 8 + [I, P, P, P,
                                                            ctypes.POINTER(_Extras), P, Z, P]
        L.mita_forward_noalloc.restype = S
        L.mita_forward_noalloc.argtypes = [P, P, P] + [I] * 8 + [I, P, P, P, P]
        L.mita_forward_ex.restype = S
        L.mita_forward_ex.argtypes = [P, P, P] + [I] * 8 + [I, P, P, P, ctypes.POINTER(_Extras),
                                                            P, Z, P]
        L.mita_pool.restype = S
        L.mita_pool.argtypes = [P] + [I] * 7 + [I, P, P]
        L.mita_landmark_workspace_bytes.restype = Z
        L.mita_landmark_workspace_bytes.argtypes = [I] * 6 + [I]
        L.mita_landmark.restype = S
        L.mita_landmark.argtypes = [P, P, P] + [I] * 6 + [I, P, P, P, Z, P]
        L.mita_route_workspace_bytes.restype = Z
        L.mita_route_workspace_bytes.argtypes = [I] * 5 + [I]
        L.mita_route.restype = S
        L.mita_route.argtypes = [P, P] + [I] * 5 + [I, P, P, P, P, P, Z, P]
        L.mita_attend.restype = S
        L.mita_attend.argtypes = [P] * 9 + [I] * 6 + [I, P, P]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != MITA_OK:
        L = lib()
        raise MitaError(status, f"{L.mita_status_string(status).decode()}: "
                                f"{L.mita_last_error().decode()}")


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MITA_BF16
    if t.dtype == torch.float32:
        return MITA_F32
    raise TypeError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream=None):
    torch = _torch()
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _qkv(q, k, v):
    torch = _torch()
    _dev(q, "Q")
    if q.dim() != 4:
        raise ValueError("Q, K, V must be [B, H, N, d]")
    _dev(k, "K", q.dtype, q.shape)
    _dev(v, "V", q.dtype, q.shape)
    return _dtype_code(q), torch


def _grid(q, grid_h, grid_w):
    """The library takes N from the grid; tensors sized from q must agree with it."""
    if q.dim() != 4:
        raise ValueError("Q must be [B, H, N, d]")
    if q.shape[2] != grid_h * grid_w:
        raise ValueError(f"Q has N={q.shape[2]} tokens but the grid is {grid_h}x{grid_w} "
                         f"= {grid_h * grid_w}")


def mita_workspace_bytes(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code, path="auto", s=1,
                         route_only=False) -> int:
    """Device workspace bytes a call with this path and variant needs (0: none)."""
    ex = _Extras(path=PATHS[path], s=s, route_only=1 if route_only else 0)
    return int(lib().mita_workspace_bytes_ex(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code,
                                             ctypes.byref(ex)))


def mita_schedule(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code) -> str:
    """'fused' or 'staged': the schedule mita_forward picks for this shape."""
    r = int(lib().mita_schedule(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code))
    if r < 0:
        raise MitaError(MITA_ERR_INVALID_ARG, "invalid shape")
    return {1: "fused", 2: "staged"}[r]


def mita_forward(q, k, v, grid_h, grid_w, m_h, m_w, topk, *, out=None, idx=None, route=None,
                 workspace=None, stream=None):
    """Whole pass; returns out [B,H,N,d] fp32.  idx/route are optional int32 outputs."""
    return mita_forward_ex(q, k, v, grid_h, grid_w, m_h, m_w, topk, out=out, idx=idx,
                           route=route, workspace=workspace, stream=stream)["out"]


def mita_forward_noalloc(q, k, v, grid_h, grid_w, m_h, m_w, topk, *, out=None, idx=None,
                         route=None, stream=None):
    """The plain pass through mita_forward_noalloc (no workspace: the library's static
    device scratch).  Returns dict(out, idx, route); idx/route as in mita_forward_ex."""
    code, torch = _qkv(q, k, v)
    _grid(q, grid_h, grid_w)
    B, H, N, d = q.shape
    m = m_h * m_w
    i32 = torch.int32

    def alloc(x, shape, dtype, name):
        if x is True:
            return torch.empty(shape, dtype=dtype, device=q.device)
        return _dev(x, name, dtype, shape) if x is not None else None

    out = alloc(True if out is None else out, (B, H, N, d), torch.float32, "out")
    idx = alloc(idx, (B, H, m, topk), i32, "idx")
    route = alloc(route, (B, H, N), i32, "route")
    _check(lib().mita_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), B, H, grid_h, grid_w, d, m_h,
                                      m_w, topk, code, _ptr(out), _ptr(idx), _ptr(route),
                                      _stream(q, stream)))
    return dict(out=out, idx=idx, route=route)


def mita_backward(q, k, v, dout, grid_h, grid_w, m_h, m_w, topk, *, s=1, route_only=False,
                  workspace=None, stream=None):
    """Gradients (dQ, dK, dV), fp32 [B, H, N, d], of sum(dout * out) with the top-k sets
    and routes of the forward held fixed."""
    code, torch = _qkv(q, k, v)
    _grid(q, grid_h, grid_w)
    B, H, N, d = q.shape
    _dev(dout, "dout", torch.float32, q.shape)
    ex = _Extras(s=s, route_only=1 if route_only else 0)
    nbytes = int(lib().mita_backward_workspace_bytes(B, H, grid_h, grid_w, d, m_h, m_w, topk,
                                                     code, ctypes.byref(ex)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    grads = [torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3)]
    _check(lib().mita_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, grid_h, grid_w, d,
                               m_h, m_w, topk, code, *[_ptr(x) for x in grads], ctypes.byref(ex),
                               _ptr(workspace), workspace.numel(), _stream(q, stream)))
    return tuple(grads)


def mita_kernel_schedule(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code, path="auto",
                         overlap=False, s=1, route_only=False) -> list:
    """The kernels mita_forward_ex launches, in the order of its timing events, as
    (name, start) pairs: kernel i runs between events[start] and events[i + 1];
    ``overlap``: the call runs routing on a side stream (host only)."""
    names = (ctypes.c_char_p * 8)()
    starts = (ctypes.c_int * 8)()
    # a non-null side stream marks the forked schedule (never dereferenced here)
    ex = _Extras(path=PATHS[path], s=s, route_only=1 if route_only else 0,
                 side_stream=1 if overlap else None)
    n = int(lib().mita_kernel_names(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code,
                                    ctypes.byref(ex), names, starts, 8))
    if n < 0:
        _check(-n)
    return [(names[i].decode(), int(starts[i])) for i in range(n)]


def mita_kernel_names(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code, path="auto", s=1,
                      route_only=False) -> list:
    """The kernels mita_forward_ex launches, in the order of its timing events (host only)."""
    return [nm for nm, _ in mita_kernel_schedule(B, H, grid_h, grid_w, d, m_h, m_w, k, dtype_code,
                                                 path, s=s, route_only=route_only)]


_sides = {}
_sides_lock = threading.Lock()


class _SyncEvent:
    """A fork / join event from mita_sync_event_create (kept for the process)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().mita_sync_event_create(ctypes.byref(h)))
        self.cuda_event = h.value


def _side(device):
    """The calling thread's side stream and fork/join events for `device` (created once).

    Each host thread gets its own set: two calls in flight at once must not
    share the fork and join events (one call's record could otherwise be
    waited on by the other's side stream)."""
    import torch
    key = (torch.device(device).index, threading.get_ident())
    with _sides_lock:
        if key not in _sides:
            with torch.cuda.device(device):
                s = torch.cuda.Stream(device=device)
                f, j = _SyncEvent(), _SyncEvent()
            _sides[key] = (s, f, j)
        return _sides[key]


def mita_forward_ex(q, k, v, grid_h, grid_w, m_h, m_w, topk, *, out=None, idx=None, route=None,
                    extras=False, path="auto", workspace=None, stream=None, events=None,
                    overlap=False, s=1, route_only=False):
    """Whole pass with optional intermediates.

    ``idx`` / ``route``: a preallocated int32 tensor, True (allocate) or None;
    route is [B, H, N] for s = 1 and [B, H, N, s] otherwise.
    ``extras=True`` also returns ql, vl, counts, offsets and perm (perm and
    counts over the N*s (query, rank) items when s > 1).
    ``overlap=True``: the staged schedule runs routing and grouping on the
    calling thread's side stream for the device, beside the landmark pass.
    ``s``: experts per query; ``route_only``: the variant without the shared
    expert.
    ``events``: torch.cuda.Event objects (enable_timing=True): events[0] before
    the first kernel, events[i + 1] after the i-th kernel of
    mita_kernel_schedule, whose start index gives the event the kernel's
    interval opens with; each must have been recorded once already so that its
    HIP event exists.
    """
    code, torch = _qkv(q, k, v)
    _grid(q, grid_h, grid_w)
    B, H, N, d = q.shape
    m = m_h * m_w
    dev = q.device
    i32 = torch.int32

    def alloc(x, shape, dtype, name):
        if x is True:
            return torch.empty(shape, dtype=dtype, device=dev)
        return _dev(x, name, dtype, shape) if x is not None else None

    out = alloc(True if out is None else out, (B, H, N, d), torch.float32, "out")
    idx = alloc(idx, (B, H, m, topk), i32, "idx")
    route = alloc(route, (B, H, N) if s == 1 else (B, H, N, s), i32, "route")
    res = dict(out=out, idx=idx, route=route)
    ex = _Extras(path=PATHS[path], s=s, route_only=1 if route_only else 0)
    if overlap:
        side, fork, join = _side(dev)
        ex.side_stream, ex.fork_event, ex.join_event = side.cuda_stream, fork.cuda_event, \
            join.cuda_event
    if events:
        handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        ex.events = ctypes.cast(handles, ctypes.POINTER(ctypes.c_void_p))
        ex.n_events = len(events)
    if extras:
        res.update(ql=alloc(True, (B, H, m, d), torch.float32, "ql"),
                   vl=alloc(True, (B, H, m, d), torch.float32, "vl"),
                   counts=alloc(True, (B, H, m), i32, "counts"),
                   offsets=alloc(True, (B, H, m + 1), i32, "offsets"),
                   perm=alloc(True, (B, H, N * s), i32, "perm"))
        for name in ("ql", "vl", "counts", "offsets", "perm"):
            setattr(ex, name, res[name].data_ptr())
    nbytes = int(lib().mita_workspace_bytes_ex(B, H, grid_h, grid_w, d, m_h, m_w, topk, code,
                                               ctypes.byref(ex)))
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
    _check(lib().mita_forward_ex(_ptr(q), _ptr(k), _ptr(v), B, H, grid_h, grid_w, d, m_h, m_w,
                                 topk, code, _ptr(out), _ptr(idx), _ptr(route), ctypes.byref(ex),
                                 _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                 _stream(q, stream)))
    return res


def mita_pool(q, grid_h, grid_w, m_h, m_w, *, ql=None, stream=None):
    torch = _torch()
    _dev(q, "Q")
    _grid(q, grid_h, grid_w)
    B, H, N, d = q.shape
    ql = torch.empty((B, H, m_h * m_w, d), dtype=torch.float32, device=q.device) if ql is None \
        else _dev(ql, "ql", torch.float32, (B, H, m_h * m_w, d))
    _check(lib().mita_pool(_ptr(q), B, H, grid_h, grid_w, d, m_h, m_w, _dtype_code(q), _ptr(ql),
                           _stream(q, stream)))
    return ql


def mita_landmark(ql, k, v, topk, *, stream=None):
    code, torch = _qkv(k, k, v)
    B, H, N, d = k.shape
    m = ql.shape[2]
    _dev(ql, "ql", torch.float32, (B, H, m, d))
    idx = torch.empty((B, H, m, topk), dtype=torch.int32, device=k.device)
    vl = torch.empty((B, H, m, d), dtype=torch.float32, device=k.device)
    nbytes = int(lib().mita_landmark_workspace_bytes(B, H, N, d, m, topk, code))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=k.device)
    _check(lib().mita_landmark(_ptr(ql), _ptr(k), _ptr(v), B, H, N, d, m, topk, code, _ptr(idx),
                               _ptr(vl), _ptr(ws), ws.numel(), _stream(k, stream)))
    return idx, vl


def mita_route(q, ql, *, stream=None):
    torch = _torch()
    _dev(q, "Q")
    B, H, N, d = q.shape
    m = ql.shape[2]
    _dev(ql, "ql", torch.float32, (B, H, m, d))
    i32 = dict(dtype=torch.int32, device=q.device)
    route = torch.empty((B, H, N), **i32)
    counts = torch.empty((B, H, m), **i32)
    offsets = torch.empty((B, H, m + 1), **i32)
    perm = torch.empty((B, H, N), **i32)
    nbytes = int(lib().mita_route_workspace_bytes(B, H, N, d, m, _dtype_code(q)))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().mita_route(_ptr(q), _ptr(ql), B, H, N, d, m, _dtype_code(q), _ptr(route),
                            _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(ws), ws.numel(),
                            _stream(q, stream)))
    return route, counts, offsets, perm


def mita_attend(q, k, v, ql, vl, idx, route, offsets, perm, *, stream=None):
    code, torch = _qkv(q, k, v)
    B, H, N, d = q.shape
    m, topk = idx.shape[2], idx.shape[3]
    i32 = torch.int32
    _dev(ql, "ql", torch.float32, (B, H, m, d))
    _dev(vl, "vl", torch.float32, (B, H, m, d))
    _dev(idx, "idx", i32, (B, H, m, topk))
    _dev(route, "route", i32, (B, H, N))
    _dev(offsets, "offsets", i32, (B, H, m + 1))
    _dev(perm, "perm", i32, (B, H, N))
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    _check(lib().mita_attend(_ptr(q), _ptr(k), _ptr(v), _ptr(ql), _ptr(vl), _ptr(idx),
                             _ptr(route), _ptr(offsets), _ptr(perm), B, H, N, d, m, topk, code,
                             _ptr(out), _stream(q, stream)))
    return out


forward = mita_forward
