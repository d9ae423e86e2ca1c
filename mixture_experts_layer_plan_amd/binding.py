"""ctypes binding of libmoe.so (include/moe.h), same names as the C entry points.

Marshalling only: torch tensors become device pointers, ``None`` becomes NULL and
the current torch stream becomes the hipStream_t.  Every step of the layer runs in
the library's HIP kernels; there is no Python or CPU fallback.  A missing library
raises ``MoeLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8}


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: status {code} ({msg})")
        self.code = code


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("T_minibatch", ctypes.c_int32), ("flags", ctypes.c_int32)]


class moe_plan_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("counts", "offsets", "src_token", "src_slot", "pos",
                                                "tiles", "n_tiles", "err_flag", "active",
                                                "n_active", "tile_first", "wtiles",
                                                "n_wtiles", "scratch",
                                                "sub_plan_bytes", "total_bytes")] + \
               [(n, ctypes.c_int32) for n in ("tile_m", "max_tiles", "chunk_pairs", "n_chunks",
                                              "n_minibatch", "T_minibatch", "wtile_m",
                                              "max_wtiles")]


_P = ctypes.c_void_p
_S = ctypes.POINTER(moe_shape)
_Z = ctypes.c_size_t
_I = ctypes.c_int

class moe_trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)),
                ("names", ctypes.POINTER(ctypes.c_char_p)),
                ("capacity", ctypes.c_int32), ("count", ctypes.c_int32)]


# name -> (restype, argtypes)
_SIGS = {
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_trace_set": (None, [ctypes.POINTER(moe_trace)]),
    "moe_set_cu_budget": (None, [ctypes.c_int32]),
    "moe_plan_layout_of": (ctypes.c_int, [_S, ctypes.POINTER(moe_plan_layout)]),
    "moe_plan_bytes": (_Z, [_S]),
    "moe_saved_bytes": (_Z, [_S, _I]),
    "moe_workspace_bytes": (_Z, [_S, _I, _I]),
    "moe_router_logits_f32": (_I, [_S, _P, _P, _P, _P]),
    "moe_route": (_I, [_S, _P, _P, _P, _P]),
    "moe_route_backward": (_I, [_S, _P, _P, _P, _P, _P]),
    "moe_router_backward_f32": (_I, [_S, _P, _P, _P, _P, _P, _P]),
    "moe_plan": (_I, [_S, _P, _P, _P]),
    "moe_dispatch_bf16": (_I, [_S, _P, _P, _P, _P]),
    "moe_dispatch_f32": (_I, [_S, _P, _P, _P, _P]),
    "moe_combine_bf16": (_I, [_S, _P, _P, _P, _P, _P, _P]),
    "moe_combine_f32": (_I, [_S, _P, _P, _P, _P, _P, _P]),
    "moe_reverse_combine_bf16": (_I, [_S, _P, _P, _P, _P]),
    "moe_reverse_dispatch_bf16": (_I, [_S, _P, _P, _P, _P, _P]),
    "moe_forward_bf16": (_I, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_forward_f32": (_I, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_forward_bf16_noalloc": (_I, [_S] + [_P] * 12),
    "moe_backward_bf16": (_I, [_S] + [_P] * 20 + [_Z, _P]),
    "moe_backward_f32": (_I, [_S] + [_P] * 20 + [_Z, _P]),
    "moe_mx_weights_bytes": (_Z, [_S]),
    "moe_quantize_weights_mxfp8": (_I, [_S, _P, _P, _P, _P, _P]),
    "moe_quantize_mxfp8": (_I, [_P, ctypes.c_int64, ctypes.c_int64, _I, _P, _P, _P]),
    "moe_quantize_mxfp8_f32": (_I, [_P, ctypes.c_int64, ctypes.c_int64, _I, _P, _P, _P]),
    "moe_forward_mxfp8": (_I, [_S] + [_P] * 10 + [_Z, _P]),
    "moe_backward_mxfp8": (_I, [_S] + [_P] * 18 + [_Z, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeLibraryMissing(
                f"{LIB_PATH} is missing: build it with `python -m mixture_experts_layer_plan_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_names() -> list[str]:
    return list(_SIGS)


MOE_REPLAY = 1
MOE_FUSED_FORWARD = 2


def shape(T, H, I, E, k, I_shared=0, T_minibatch=0, flags=0) -> moe_shape:
    return moe_shape(int(T), int(H), int(I), int(E), int(k), int(I_shared), int(T_minibatch),
                     int(flags))


def _ptr(t, dtype=None, numel=None):
    """Device pointer of a contiguous tensor (None -> NULL).  ``dtype`` and ``numel``,
    when given, are checked: the library reads and writes through raw pointers, so a
    tensor of another element type or size would be over-read or overrun."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected a {dtype} tensor, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"expected {numel} elements, got {t.numel()}")
    return t.data_ptr()


_F32 = torch.float32
_BF16 = torch.bfloat16


def _f32(t, numel=None):
    return _ptr(t, _F32, numel)


def _bf16(t, numel=None):
    return _ptr(t, _BF16, numel)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise MoeError(name, rc, lib().moe_status_str(rc).decode())


def moe_set_cu_budget(cus: int) -> None:
    lib().moe_set_cu_budget(int(cus))


def moe_status_str(code: int) -> str:
    return lib().moe_status_str(code).decode()


def moe_plan_layout_of(s: moe_shape) -> moe_plan_layout:
    out = moe_plan_layout()
    _call("moe_plan_layout_of", ctypes.byref(s), ctypes.byref(out))
    return out


def moe_plan_bytes(s: moe_shape) -> int:
    return lib().moe_plan_bytes(ctypes.byref(s))


def moe_saved_bytes(s: moe_shape, dtype: int) -> int:
    return lib().moe_saved_bytes(ctypes.byref(s), dtype)


def moe_workspace_bytes(s: moe_shape, dtype: int, backward: bool) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(s), dtype, int(backward))


def moe_router_logits_f32(s, x, w_router, logits, stream=None):
    _call("moe_router_logits_f32", ctypes.byref(s), _f32(x, s.T * s.H), _f32(w_router, s.E * s.H),
          _f32(logits, s.T * s.E), _stream(stream))


def moe_route(s, logits, topk_idx, topk_w, stream=None):
    _call("moe_route", ctypes.byref(s), _f32(logits, s.T * s.E), _ptr(topk_idx, torch.int32, s.T * s.k),
          _f32(topk_w, s.T * s.k), _stream(stream))


def moe_route_backward(s, topk_idx, topk_w, d_topk_w, d_logits, stream=None):
    _call("moe_route_backward", ctypes.byref(s), _ptr(topk_idx, torch.int32, s.T * s.k),
          _f32(topk_w, s.T * s.k), _f32(d_topk_w, s.T * s.k), _f32(d_logits, s.T * s.E),
          _stream(stream))


def moe_router_backward_f32(s, x, w_router, d_logits, dw_router, dx, stream=None):
    _call("moe_router_backward_f32", ctypes.byref(s), _f32(x, s.T * s.H), _f32(w_router, s.E * s.H),
          _f32(d_logits, s.T * s.E), _f32(dw_router, s.E * s.H), _f32(dx, s.T * s.H),
          _stream(stream))


def moe_plan(s, topk_idx, plan, stream=None):
    _call("moe_plan", ctypes.byref(s), _ptr(topk_idx), _ptr(plan), _stream(stream))


def moe_dispatch_bf16(s, plan, x, X, stream=None):
    _call("moe_dispatch_bf16", ctypes.byref(s), _ptr(plan), _ptr(x), _ptr(X), _stream(stream))


def moe_dispatch_f32(s, plan, x, X, stream=None):
    _call("moe_dispatch_f32", ctypes.byref(s), _ptr(plan), _f32(x, s.T * s.H), _f32(X, s.T * s.k * s.H),
          _stream(stream))


def moe_combine_bf16(s, plan, Y, topk_w, shared_out, y, stream=None):
    _call("moe_combine_bf16", ctypes.byref(s), _ptr(plan), _ptr(Y), _ptr(topk_w),
          _ptr(shared_out), _ptr(y), _stream(stream))


def moe_combine_f32(s, plan, Y, topk_w, shared_out, y, stream=None):
    _call("moe_combine_f32", ctypes.byref(s), _ptr(plan), _f32(Y, s.T * s.k * s.H),
          _f32(topk_w, s.T * s.k), _f32(shared_out, s.T * s.H), _f32(y, s.T * s.H), _stream(stream))


def moe_reverse_combine_bf16(s, plan, dy, dYu, stream=None):
    _call("moe_reverse_combine_bf16", ctypes.byref(s), _ptr(plan), _ptr(dy), _ptr(dYu),
          _stream(stream))


def moe_reverse_dispatch_bf16(s, plan, dX, shared_dx, dx, stream=None):
    _call("moe_reverse_dispatch_bf16", ctypes.byref(s), _ptr(plan), _ptr(dX), _ptr(shared_dx),
          _ptr(dx), _stream(stream))


def _fwd(name, s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y, saved, ws,
         stream):
    dt = _F32 if name.endswith("_f32") else _BF16
    nw, ns = s.E * s.I * s.H, s.I_shared * s.H
    _call(name, ctypes.byref(s), _ptr(plan), _ptr(x, dt, s.T * s.H), _f32(topk_w, s.T * s.k),
          _ptr(w_gate, dt, nw), _ptr(w_up, dt, nw), _ptr(w_down, dt, nw), _ptr(s_gate, dt, ns),
          _ptr(s_up, dt, ns), _ptr(s_down, dt, ns), _ptr(y, dt, s.T * s.H), _ptr(saved), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_forward_bf16(s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y, saved,
                     ws, stream=None):
    _fwd("moe_forward_bf16", s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
         saved, ws, stream)


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_bf16_noalloc(s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
                             saved, stream=None):
    nw, ns, nt = s.E * s.I * s.H, s.I_shared * s.H, s.T * s.H
    _call("moe_forward_bf16_noalloc", ctypes.byref(s), _ptr(plan), _bf16(x, nt),
          _f32(topk_w, s.T * s.k), _bf16(w_gate, nw), _bf16(w_up, nw), _bf16(w_down, nw),
          _bf16(s_gate, ns), _bf16(s_up, ns), _bf16(s_down, ns), _bf16(y, nt), _ptr(saved),
          _stream(stream))


def moe_forward_f32(s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y, saved,
                    ws, stream=None):
    _fwd("moe_forward_f32", s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
         saved, ws, stream)


def _bwd(name, s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, saved, dy, dx,
         dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w, ws, stream):
    dt = _F32 if name.endswith("_f32") else _BF16
    nw, ns, nt = s.E * s.I * s.H, s.I_shared * s.H, s.T * s.H
    _call(name, ctypes.byref(s), _ptr(plan), _ptr(x, dt, nt), _f32(topk_w, s.T * s.k),
          _ptr(w_gate, dt, nw), _ptr(w_up, dt, nw), _ptr(w_down, dt, nw), _ptr(s_gate, dt, ns),
          _ptr(s_up, dt, ns), _ptr(s_down, dt, ns), _ptr(saved), _ptr(dy, dt, nt), _ptr(dx, dt, nt),
          _ptr(dw_gate, dt, nw), _ptr(dw_up, dt, nw), _ptr(dw_down, dt, nw), _ptr(ds_gate, dt, ns),
          _ptr(ds_up, dt, ns), _ptr(ds_down, dt, ns), _f32(d_topk_w, s.T * s.k), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_backward_bf16(s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, saved, dy,
                      dx, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w, ws,
                      stream=None):
    _bwd("moe_backward_bf16", s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down,
         saved, dy, dx, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w, ws, stream)


def moe_backward_f32(s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down, saved, dy,
                     dx, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w, ws,
                     stream=None):
    _bwd("moe_backward_f32", s, plan, x, topk_w, w_gate, w_up, w_down, s_gate, s_up, s_down,
         saved, dy, dx, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w, ws, stream)


def moe_mx_weights_bytes(s: moe_shape) -> int:
    return lib().moe_mx_weights_bytes(ctypes.byref(s))


def moe_quantize_weights_mxfp8(s, w_gate, w_up, w_down, wq, stream=None):
    nw = s.E * s.I * s.H
    _call("moe_quantize_weights_mxfp8", ctypes.byref(s), _bf16(w_gate, nw), _bf16(w_up, nw),
          _bf16(w_down, nw), _ptr(wq, torch.uint8, moe_mx_weights_bytes(s)), _stream(stream))


def moe_quantize_mxfp8(src, rows, cols, axis, q, scales, stream=None):
    _call("moe_quantize_mxfp8", _ptr(src), int(rows), int(cols), int(axis), _ptr(q), _ptr(scales),
          _stream(stream))


def moe_quantize_mxfp8_f32(src, rows, cols, axis, q, scales, stream=None):
    n = int(rows) * int(cols)
    _call("moe_quantize_mxfp8_f32", _f32(src, n), int(rows), int(cols), int(axis),
          _ptr(q, torch.uint8, n), _ptr(scales, torch.uint8, n // 32), _stream(stream))


def moe_forward_mxfp8(s, plan, x, topk_w, wq, s_gate, s_up, s_down, y, saved, ws, stream=None):
    ns, nt = s.I_shared * s.H, s.T * s.H
    _call("moe_forward_mxfp8", ctypes.byref(s), _ptr(plan), _bf16(x, nt), _f32(topk_w, s.T * s.k),
          _ptr(wq, torch.uint8, moe_mx_weights_bytes(s)), _bf16(s_gate, ns), _bf16(s_up, ns),
          _bf16(s_down, ns), _bf16(y, nt), _ptr(saved), _ptr(ws),
          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


def moe_backward_mxfp8(s, plan, x, topk_w, wq, s_gate, s_up, s_down, saved, dy, dx, dw_gate,
                       dw_up, dw_down, ds_gate, ds_up, ds_down, d_topk_w, ws, stream=None):
    nw, ns, nt = s.E * s.I * s.H, s.I_shared * s.H, s.T * s.H
    _call("moe_backward_mxfp8", ctypes.byref(s), _ptr(plan), _bf16(x, nt), _f32(topk_w, s.T * s.k),
          _ptr(wq, torch.uint8, moe_mx_weights_bytes(s)), _bf16(s_gate, ns), _bf16(s_up, ns),
          _bf16(s_down, ns), _ptr(saved), _bf16(dy, nt), _bf16(dx, nt), _bf16(dw_gate, nw),
          _bf16(dw_up, nw), _bf16(dw_down, nw), _bf16(ds_gate, ns), _bf16(ds_up, ns),
          _bf16(ds_down, ns), _f32(d_topk_w, s.T * s.k), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


# ------------------------------------------------------------ kernel timing
_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        _hip = h
    return _hip


class KernelTrace:
    """Per-kernel HIP events around every launch the library makes from this
    thread while active (``with KernelTrace(n) as tr: ...``); ``records()`` gives
    (name, milliseconds) per launch after the stream has been synchronised."""

    def __init__(self, capacity: int):
        h = _hiprt()
        self.capacity = capacity
        self._events = (ctypes.c_void_p * (2 * capacity))()
        ev = ctypes.c_void_p()
        for i in range(2 * capacity):
            if h.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self._events[i] = ev.value
        self._names = (ctypes.c_char_p * capacity)()
        self.t = moe_trace(ctypes.cast(self._events, ctypes.POINTER(ctypes.c_void_p)),
                           ctypes.cast(self._names, ctypes.POINTER(ctypes.c_char_p)),
                           capacity, 0)

    def __enter__(self):
        self.t.count = 0
        lib().moe_trace_set(ctypes.byref(self.t))
        return self

    def __exit__(self, *exc):
        lib().moe_trace_set(None)
        return False

    def records(self):
        h = _hiprt()
        out = []
        ms = ctypes.c_float()
        for i in range(self.t.count):
            if h.hipEventElapsedTime(ctypes.byref(ms), self._events[2 * i], self._events[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((self._names[i].decode(), ms.value))
        return out

    def close(self):
        h = _hiprt()
        for i in range(2 * self.capacity):
            h.hipEventDestroy(self._events[i])
        self.capacity = 0


# ------------------------------------------------------------ buffer helpers
def plan_views(s: moe_shape, plan: torch.Tensor, minibatch: int = 0) -> dict:
    """int32 views of the arrays of one minibatch's table inside a plan buffer
    (uint8 tensor); ``T`` is that minibatch's token count."""
    L = moe_plan_layout_of(s)
    T = min(L.T_minibatch, s.T - minibatch * L.T_minibatch)
    R = T * s.k
    sub = plan[minibatch * L.sub_plan_bytes:(minibatch + 1) * L.sub_plan_bytes]

    def view(off, n):
        return sub[off:off + 4 * n].view(torch.int32)

    return {"counts": view(L.counts, s.E), "offsets": view(L.offsets, s.E + 1),
            "src_token": view(L.src_token, R), "src_slot": view(L.src_slot, R),
            "pos": view(L.pos, R).view(T, s.k), "tiles": view(L.tiles, 2 * L.max_tiles).view(-1, 2),
            "n_tiles": view(L.n_tiles, 1), "err_flag": view(L.err_flag, 1),
            "active": view(L.active, s.E), "n_active": view(L.n_active, 1),
            "tile_first": view(L.tile_first, s.E + 1), "tile_m": L.tile_m,
            "wtiles": view(L.wtiles, 2 * L.max_wtiles).view(-1, 2),
            "n_wtiles": view(L.n_wtiles, 1), "wtile_m": L.wtile_m, "T": T}
