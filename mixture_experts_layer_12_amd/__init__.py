"""Python binding of libcolibri_moe.so, the gfx950 MoE layer forward pass.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/colibri_moe.h``.  torch tensors are
used for device memory and streams; their data pointers and the current HIP
stream are handed to the library unchanged.  There is no fallback: if the
library is not built, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcolibri_moe.so")

COLIBRI_OK, COLIBRI_ERR_INVALID_ARG, COLIBRI_ERR_WORKSPACE, COLIBRI_ERR_UNSUPPORTED, COLIBRI_ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
RELU, GELU, SWIGLU = 0, 1, 2
ACT_CODES = {"relu": RELU, "gelu": GELU, "swiglu": SWIGLU}
GATE_PAIR, GATE_SOFTMAX, GATE_LINEAR = 0, 1, 2
GATE_CODES = {"pair": GATE_PAIR, "softmax": GATE_SOFTMAX, "linear": GATE_LINEAR}

EXPORTED = [
    "colibri_moe_workspace_size", "colibri_moe_route", "colibri_moe_dispatch", "colibri_moe_dispatch_workspace_size",
    "colibri_moe_expert_ffn", "colibri_moe_expert_ffn_up", "colibri_moe_expert_ffn_down", "colibri_moe_combine", "colibri_moe_layer_forward",
    "colibri_moe_layer_forward_noalloc", "colibri_moe_workspace_layout",
    "colibri_moe_quantize_q8", "colibri_moe_expert_ffn_q8", "colibri_moe_layer_forward_q8",
    "colibri_moe_quantize_q4", "colibri_moe_expert_ffn_q4", "colibri_moe_layer_forward_q4",
    "colibri_moe_workspace_size_ex", "colibri_moe_route_ex", "colibri_moe_combine_ex",
    "colibri_moe_layer_forward_ex", "colibri_moe_step_workspace_size", "colibri_moe_step_forward",
    "colibri_moe_graph_create", "colibri_moe_graph_launch", "colibri_moe_graph_destroy",
    "colibri_moe_status_string",
]


class ColibriError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class _Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("h", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32)]


class _Experts(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("b1", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


class _ExpertsQ8(ctypes.Structure):
    _fields_ = [("q1", ctypes.c_void_p), ("q3", ctypes.c_void_p), ("q2", ctypes.c_void_p),
                ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p),
                ("b1", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


class _ExpertsQ4(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q1", "q3", "q2", "s1", "s3", "s2", "z1", "z3", "z2", "b1", "b2")]


class _WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("topk_idx", "topk_gate", "expert_counts", "expert_offsets",
                                                "sorted_assign", "assign_pos")]


class _Opts(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_int), ("shared", ctypes.POINTER(_Experts)), ("shared_h", ctypes.c_int32),
                ("residual", ctypes.c_void_p), ("combine", ctypes.c_int32)]


COMBINE = {"auto": 0, "separate": 1, "fold": 2}


class _LayerParams(ctypes.Structure):
    _fields_ = [("w_r", ctypes.c_void_p), ("b_r", ctypes.c_void_p), ("experts", _Experts), ("gate", ctypes.c_int),
                ("shared", ctypes.POINTER(_Experts)), ("shared_h", ctypes.c_int32)]


@dataclass(frozen=True)
class Shape:
    T: int
    d: int
    h: int
    E: int
    dtype: int = BF16
    act: int = SWIGLU
    k: int = 2

    def c(self) -> _Shape:
        return _Shape(self.T, self.d, self.h, self.E, self.k, self.dtype, self.act)

    def with_T(self, T: int) -> "Shape":
        return Shape(T, self.d, self.h, self.E, self.dtype, self.act, self.k)


_lib = None


def build() -> str:
    from . import _build
    return _build.build()


def load(build_if_missing: bool = False):
    """Load the HIP library.  Raises if it is not built (unless asked to build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise ImportError(f"{LIB_PATH} is not built; run mixture_experts_layer_12_amd.build() "
                              "(or __graft_entry__.build()) first")
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    SP = ctypes.POINTER(_Shape)
    lib.colibri_moe_workspace_size.argtypes = [SP]
    lib.colibri_moe_workspace_size.restype = Z
    lib.colibri_moe_route.argtypes = [SP, P, P, P, P, P, P, P]
    lib.colibri_moe_dispatch_workspace_size.argtypes = [SP]
    lib.colibri_moe_dispatch_workspace_size.restype = Z
    lib.colibri_moe_dispatch.argtypes = [SP, P, P, P, P, P, P, P, P, Z, P]
    lib.colibri_moe_expert_ffn.argtypes = [SP, P, P, P, ctypes.POINTER(_Experts), P, P, Z, P]
    lib.colibri_moe_expert_ffn_up.argtypes = [SP, P, P, P, ctypes.POINTER(_Experts), P, P, Z, P]
    lib.colibri_moe_expert_ffn_down.argtypes = [SP, P, P, ctypes.POINTER(_Experts), P, P, Z, P]
    lib.colibri_moe_combine.argtypes = [SP, P, P, P, P, P]
    lib.colibri_moe_layer_forward.argtypes = [SP, P, P, P, ctypes.POINTER(_Experts), P, P, P, P, P, Z, P]
    lib.colibri_moe_layer_forward_noalloc.argtypes = [SP, P, P, P, ctypes.POINTER(_Experts), P, P, P, P, P]
    lib.colibri_moe_workspace_layout.argtypes = [SP, ctypes.POINTER(_WsLayout)]
    i32 = ctypes.c_int32
    lib.colibri_moe_quantize_q8.argtypes = [P, I, i32, i32, i32, P, P, P]
    lib.colibri_moe_expert_ffn_q8.argtypes = [SP, P, P, P, ctypes.POINTER(_ExpertsQ8), P, P, Z, P]
    lib.colibri_moe_layer_forward_q8.argtypes = [SP, P, P, P, ctypes.POINTER(_ExpertsQ8), P, P, P, P, P, Z, P]
    lib.colibri_moe_quantize_q4.argtypes = [P, I, i32, i32, i32, P, P, P, P]
    lib.colibri_moe_expert_ffn_q4.argtypes = [SP, P, P, P, ctypes.POINTER(_ExpertsQ4), P, P, Z, P]
    lib.colibri_moe_layer_forward_q4.argtypes = [SP, P, P, P, ctypes.POINTER(_ExpertsQ4), P, P, P, P, P, Z, P]
    OP = ctypes.POINTER(_Opts)
    lib.colibri_moe_workspace_size_ex.argtypes = [SP, OP]
    lib.colibri_moe_workspace_size_ex.restype = Z
    lib.colibri_moe_route_ex.argtypes = [SP, P, P, P, I, P, P, P, P]
    lib.colibri_moe_combine_ex.argtypes = [SP, P, P, P, P, P, P, P]
    lib.colibri_moe_layer_forward_ex.argtypes = [SP, P, P, P, ctypes.POINTER(_Experts), OP, P, P, P, P, P, Z, P]
    LP = ctypes.POINTER(_LayerParams)
    lib.colibri_moe_step_workspace_size.argtypes = [SP, i32, LP]
    lib.colibri_moe_step_workspace_size.restype = Z
    lib.colibri_moe_step_forward.argtypes = [SP, i32, LP, i32, P, P, Z, P]
    lib.colibri_moe_graph_create.argtypes = [SP, i32, LP, i32, P, P, Z, ctypes.POINTER(P)]
    lib.colibri_moe_graph_launch.argtypes = [P, P]
    lib.colibri_moe_graph_destroy.argtypes = [P]
    for f in ("colibri_moe_route", "colibri_moe_dispatch", "colibri_moe_expert_ffn", "colibri_moe_expert_ffn_up",
              "colibri_moe_expert_ffn_down", "colibri_moe_combine", "colibri_moe_layer_forward",
              "colibri_moe_layer_forward_noalloc", "colibri_moe_workspace_layout", "colibri_moe_quantize_q8",
              "colibri_moe_expert_ffn_q8", "colibri_moe_layer_forward_q8",
              "colibri_moe_quantize_q4", "colibri_moe_expert_ffn_q4", "colibri_moe_layer_forward_q4",
              "colibri_moe_route_ex", "colibri_moe_combine_ex", "colibri_moe_layer_forward_ex",
              "colibri_moe_step_forward", "colibri_moe_graph_create", "colibri_moe_graph_launch",
              "colibri_moe_graph_destroy"):
        getattr(lib, f).restype = I
    lib.colibri_moe_status_string.argtypes = [I]
    lib.colibri_moe_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().colibri_moe_status_string(int(status)).decode()


# ------------------------------------------------------------------ marshalling
def _ptr(t, nbytes: int = 0, es: int = 0, name: str = "tensor") -> Optional[int]:
    """Device pointer of a tensor (or None), after checking that the tensor can
    be what the call reads or writes there: contiguous, on a GPU, elements of
    es bytes (0: any) and at least nbytes long.  A raw integer is passed as it
    is (tests hand the library addresses directly)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if t.device.type != "cuda":
        raise ValueError(f"{name}: a GPU tensor is needed, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (the library reads it densely, row-major)")
    if es and t.element_size() != es:
        raise TypeError(f"{name}: elements of {es} bytes expected, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: holds {have} bytes, the call's shape needs {nbytes}")
    return t.data_ptr()


def _ws(ws, ws_bytes: Optional[int]):
    """Workspace pointer and byte count: by default the tensor's own size; a
    count larger than the tensor is refused."""
    if ws is None or isinstance(ws, int):
        return ws, int(ws_bytes or 0)
    have = ws.numel() * ws.element_size()
    if ws_bytes is None:
        ws_bytes = have
    if ws_bytes > have:
        raise ValueError(f"ws_bytes = {ws_bytes} exceeds the workspace tensor's {have} bytes")
    return _ptr(ws, name="ws"), int(ws_bytes)


def _es(shape) -> int:
    return 4 if shape.dtype == F32 else 2


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != COLIBRI_OK:
        raise ColibriError(status, where)


def _experts(w1, w2, w3=None, b1=None, b2=None, shape=None, h=None) -> _Experts:
    """Expert weights [E][d][h] / [E][h][d] and biases; with a shape, each
    tensor is checked against it (h: a hidden width other than the shape's)."""
    if shape is None:
        return _Experts(_ptr(w1), _ptr(w3), _ptr(w2), _ptr(b1), _ptr(b2))
    E, d, h, es = shape.E, shape.d, h or shape.h, _es(shape)
    return _Experts(_ptr(w1, E * d * h * es, es, "w1"), _ptr(w3, E * d * h * es, es, "w3"),
                    _ptr(w2, E * h * d * es, es, "w2"), _ptr(b1, E * h * es, es, "b1"), _ptr(b2, E * d * es, es, "b2"))


def workspace_size(shape: Shape) -> int:
    s = shape.c()
    return int(load().colibri_moe_workspace_size(ctypes.byref(s)))


def workspace_layout(shape: Shape) -> dict:
    """Byte offsets of the routing and dispatch results a layer call leaves in
    its workspace (colibri_moe_workspace_layout)."""
    s = shape.c()
    lay = _WsLayout()
    _check(load().colibri_moe_workspace_layout(ctypes.byref(s), ctypes.byref(lay)), "colibri_moe_workspace_layout")
    return {n: int(getattr(lay, n)) for n, _ in _WsLayout._fields_}


def dispatch_workspace_size(shape: Shape) -> int:
    s = shape.c()
    return int(load().colibri_moe_dispatch_workspace_size(ctypes.byref(s)))


def _router_args(shape: Shape, x, w_r, b_r):
    es = _es(shape)
    return (_ptr(x, shape.T * shape.d * es, es, "x"), _ptr(w_r, shape.d * shape.E * es, es, "w_r"),
            _ptr(b_r, shape.E * 4, 4, "b_r"))


def _routing_outs(shape: Shape, topk_idx, topk_gate, counts):
    T = shape.T
    return (_ptr(topk_idx, 2 * T * 4, 4, "topk_idx"), _ptr(topk_gate, 2 * T * 4, 4, "topk_gate"),
            _ptr(counts, shape.E * 4, 4, "counts"))


def route(shape: Shape, x, w_r, b_r, topk_idx, topk_gate, logits=None, stream=None):
    s = shape.c()
    idx, gate, _ = _routing_outs(shape, topk_idx, topk_gate, None)
    _check(load().colibri_moe_route(ctypes.byref(s), *_router_args(shape, x, w_r, b_r), idx, gate,
                                    _ptr(logits, shape.T * shape.E * 4, 4, "logits"), _stream(stream)),
           "colibri_moe_route")


def dispatch(shape: Shape, topk_idx, counts, offsets, sorted_assign, assign_pos, x=None, x_sorted=None,
             ws=None, ws_bytes: Optional[int] = None, stream=None):
    s = shape.c()
    A, es = 2 * shape.T, _es(shape)
    wsp, wsb = _ws(ws, ws_bytes)
    _check(load().colibri_moe_dispatch(ctypes.byref(s), _ptr(topk_idx, A * 4, 4, "topk_idx"),
                                       _ptr(counts, shape.E * 4, 4, "counts"),
                                       _ptr(offsets, (shape.E + 1) * 4, 4, "offsets"),
                                       _ptr(sorted_assign, A * 4, 4, "sorted_assign"),
                                       _ptr(assign_pos, A * 4, 4, "assign_pos"),
                                       _ptr(x, shape.T * shape.d * es, es, "x"),
                                       _ptr(x_sorted, A * shape.d * es, es, "x_sorted"), wsp, wsb, _stream(stream)),
           "colibri_moe_dispatch")


def _rows_args(shape: Shape, x_rows, sorted_assign, offsets, K: int):
    """A operand rows: X [T, K] read through sorted_assign, or sorted rows [2T, K]."""
    A, es = 2 * shape.T, _es(shape)
    return (_ptr(x_rows, (shape.T if sorted_assign is not None else A) * K * es, es, "x_rows"),
            _ptr(sorted_assign, A * 4, 4, "sorted_assign"), _ptr(offsets, (shape.E + 1) * 4, 4, "offsets"))


def expert_ffn(shape: Shape, x_rows, sorted_assign, offsets, w1, w2, y_sorted, ws, ws_bytes: Optional[int] = None,
               w3=None, b1=None, b2=None, stream=None):
    s = shape.c()
    e = _experts(w1, w2, w3, b1, b2, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_expert_ffn(ctypes.byref(s), *_rows_args(shape, x_rows, sorted_assign, offsets, shape.d),
                                         ctypes.byref(e), _ptr(y_sorted, 2 * shape.T * shape.d * es, es, "y_sorted"),
                                         *_ws(ws, ws_bytes), _stream(stream)), "colibri_moe_expert_ffn")


def expert_ffn_up(shape: Shape, x_rows, sorted_assign, offsets, w1, h_rows, ws=None, ws_bytes: Optional[int] = None,
                  w3=None, b1=None, stream=None):
    s = shape.c()
    e = _experts(w1, None, w3, b1, None, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_expert_ffn_up(ctypes.byref(s), *_rows_args(shape, x_rows, sorted_assign, offsets,
                                                                        shape.d), ctypes.byref(e),
                                            _ptr(h_rows, 2 * shape.T * shape.h * es, es, "h_rows"),
                                            *_ws(ws, ws_bytes), _stream(stream)), "colibri_moe_expert_ffn_up")


def expert_ffn_down(shape: Shape, h_rows, offsets, w2, y_sorted, ws=None, ws_bytes: Optional[int] = None, b2=None,
                    stream=None):
    s = shape.c()
    e = _experts(None, w2, None, None, b2, shape=shape)
    es = _es(shape)
    h, _, off = _rows_args(shape, h_rows, None, offsets, shape.h)
    _check(load().colibri_moe_expert_ffn_down(ctypes.byref(s), h, off, ctypes.byref(e),
                                              _ptr(y_sorted, 2 * shape.T * shape.d * es, es, "y_sorted"),
                                              *_ws(ws, ws_bytes), _stream(stream)), "colibri_moe_expert_ffn_down")


def _combine_args(shape: Shape, y_sorted, assign_pos, topk_gate, out):
    A, es = 2 * shape.T, _es(shape)
    return (_ptr(y_sorted, A * shape.d * es, es, "y_sorted"), _ptr(assign_pos, A * 4, 4, "assign_pos"),
            _ptr(topk_gate, A * 4, 4, "topk_gate"), _ptr(out, shape.T * shape.d * es, es, "out"))


def combine(shape: Shape, y_sorted, assign_pos, topk_gate, out, stream=None):
    s = shape.c()
    _check(load().colibri_moe_combine(ctypes.byref(s), *_combine_args(shape, y_sorted, assign_pos, topk_gate, out),
                                      _stream(stream)), "colibri_moe_combine")


def layer_forward(shape: Shape, x, w_r, b_r, w1, w2, out, ws, ws_bytes: Optional[int] = None, w3=None, b1=None,
                  b2=None, topk_idx=None, topk_gate=None, counts=None, stream=None):
    s = shape.c()
    e = _experts(w1, w2, w3, b1, b2, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_layer_forward(ctypes.byref(s), *_router_args(shape, x, w_r, b_r), ctypes.byref(e),
                                            _ptr(out, shape.T * shape.d * es, es, "out"),
                                            *_routing_outs(shape, topk_idx, topk_gate, counts), *_ws(ws, ws_bytes),
                                            _stream(stream)), "colibri_moe_layer_forward")


NOALLOC_SCRATCH_BYTES = 32 << 20  # COLIBRI_MOE_NOALLOC_SCRATCH_BYTES


def layer_forward_noalloc(shape: Shape, x, w_r, b_r, w1, w2, out, w3=None, b1=None, b2=None, topk_idx=None,
                          topk_gate=None, counts=None, stream=None):
    """colibri_moe_layer_forward on the library's own device scratch array (no
    workspace argument, nothing allocated).  Calls that overlap on one GPU race."""
    s = shape.c()
    e = _experts(w1, w2, w3, b1, b2, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_layer_forward_noalloc(ctypes.byref(s), *_router_args(shape, x, w_r, b_r),
                                                    ctypes.byref(e), _ptr(out, shape.T * shape.d * es, es, "out"),
                                                    *_routing_outs(shape, topk_idx, topk_gate, counts),
                                                    _stream(stream)), "colibri_moe_layer_forward_noalloc")


# ------------------------------------------------------------------ gating variants, shared expert, residual
def _gate_code(gate) -> int:
    return GATE_CODES[gate] if isinstance(gate, str) else int(gate)


def _opts(gate="pair", shared=None, shared_h: int = 0, residual=None, shape=None, combine="auto"):
    """ctypes options and the experts struct it points to (keep both alive).
    ``shared``: dict with the shared expert's w1, w2 (and w3, b1, b2); with a
    shape the tensors are checked against it (the shared expert is one expert
    of hidden width shared_h, 0 = the shape's h).  ``combine``: "auto" (the
    library's choice), "separate" (a kernel of its own) or "fold" (in the
    second layer's epilogue where that layer is a grouped GEMM)."""
    sh = None
    one = None if shape is None else Shape(shape.T, shape.d, shape.h, 1, shape.dtype, shape.act)
    if shared is not None:
        sh = _experts(shared["w1"], shared["w2"], shared.get("w3"), shared.get("b1"), shared.get("b2"), shape=one,
                      h=int(shared_h) or None)
    res = _ptr(residual) if shape is None else _ptr(residual, shape.T * shape.d * _es(shape), _es(shape), "residual")
    if combine not in COMBINE:
        raise ValueError(f"combine must be one of {sorted(COMBINE)}, not {combine!r}")
    o = _Opts(_gate_code(gate), ctypes.pointer(sh) if sh is not None else None, int(shared_h), res, COMBINE[combine])
    return o, sh


def workspace_size_ex(shape: Shape, gate="pair", shared=None, shared_h: int = 0, residual=None) -> int:
    s = shape.c()
    o, keep = _opts(gate, shared, shared_h, residual)
    return int(load().colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(o)))


def route_ex(shape: Shape, x, w_r, b_r, gate, topk_idx, topk_gate, logits=None, stream=None):
    s = shape.c()
    idx, g, _ = _routing_outs(shape, topk_idx, topk_gate, None)
    _check(load().colibri_moe_route_ex(ctypes.byref(s), *_router_args(shape, x, w_r, b_r), _gate_code(gate), idx, g,
                                       _ptr(logits, shape.T * shape.E * 4, 4, "logits"), _stream(stream)),
           "colibri_moe_route_ex")


def combine_ex(shape: Shape, y_sorted, assign_pos, topk_gate, out, shared_y=None, residual=None, stream=None):
    s = shape.c()
    y, ap, g, o = _combine_args(shape, y_sorted, assign_pos, topk_gate, out)
    n, es = shape.T * shape.d * _es(shape), _es(shape)
    _check(load().colibri_moe_combine_ex(ctypes.byref(s), y, ap, g, _ptr(shared_y, n, es, "shared_y"),
                                         _ptr(residual, n, es, "residual"), o, _stream(stream)),
           "colibri_moe_combine_ex")


def layer_forward_ex(shape: Shape, x, w_r, b_r, w1, w2, out, ws, ws_bytes: Optional[int] = None, w3=None, b1=None,
                     b2=None, gate="pair", shared=None, shared_h: int = 0, residual=None, topk_idx=None,
                     topk_gate=None, counts=None, stream=None, combine="auto"):
    s = shape.c()
    e = _experts(w1, w2, w3, b1, b2, shape=shape)
    o, keep = _opts(gate, shared, shared_h, residual, shape=shape, combine=combine)
    es = _es(shape)
    _check(load().colibri_moe_layer_forward_ex(ctypes.byref(s), *_router_args(shape, x, w_r, b_r), ctypes.byref(e),
                                               ctypes.byref(o), _ptr(out, shape.T * shape.d * es, es, "out"),
                                               *_routing_outs(shape, topk_idx, topk_gate, counts), *_ws(ws, ws_bytes),
                                               _stream(stream)), "colibri_moe_layer_forward_ex")


# ------------------------------------------------------------------ multi-layer step, graph replay
def _layer_params(layers, shape=None):
    """layers: list of dicts with w_r, w1, w2 (and b_r, w3, b1, b2, gate, shared,
    shared_h).  Returns the ctypes array and the structs it points to; with a
    shape every tensor is checked against it."""
    arr = (_LayerParams * len(layers))()
    keep = []
    for i, l in enumerate(layers):
        o, sh = _opts(l.get("gate", "pair"), l.get("shared"), int(l.get("shared_h", 0)), None, shape=shape)
        if sh is not None:
            keep.append(sh)
        if shape is None:
            w_r, b_r = _ptr(l["w_r"]), _ptr(l.get("b_r"))
        else:
            _, w_r, b_r = _router_args(shape.with_T(0), None, l["w_r"], l.get("b_r"))
        arr[i] = _LayerParams(w_r, b_r, _experts(l["w1"], l["w2"], l.get("w3"), l.get("b1"), l.get("b2"), shape=shape),
                              o.gate, o.shared, o.shared_h)
    return arr, keep


def step_workspace_size(shape: Shape, layers) -> int:
    s = shape.c()
    arr, keep = _layer_params(layers)
    return int(load().colibri_moe_step_workspace_size(ctypes.byref(s), len(layers), arr))


def step_forward(shape: Shape, layers, x, ws, ws_bytes: Optional[int] = None, residual: bool = True, stream=None):
    """x <- layer_l(x) (+ x) for every layer, in place on x."""
    s = shape.c()
    arr, keep = _layer_params(layers, shape)
    es = _es(shape)
    _check(load().colibri_moe_step_forward(ctypes.byref(s), len(layers), arr, int(bool(residual)),
                                           _ptr(x, shape.T * shape.d * es, es, "x"), *_ws(ws, ws_bytes),
                                           _stream(stream)), "colibri_moe_step_forward")


class Graph:
    """A multi-layer step captured into a HIP graph (colibri_moe_graph_*).

    The caller keeps x, ws and the weights alive while the graph exists."""

    def __init__(self, shape: Shape, layers, x, ws, ws_bytes: Optional[int] = None, residual: bool = True):
        s = shape.c()
        arr, keep = _layer_params(layers, shape)
        h = ctypes.c_void_p()
        es = _es(shape)
        _check(load().colibri_moe_graph_create(ctypes.byref(s), len(layers), arr, int(bool(residual)),
                                               _ptr(x, shape.T * shape.d * es, es, "x"), *_ws(ws, ws_bytes),
                                               ctypes.byref(h)), "colibri_moe_graph_create")
        self._h = h

    def launch(self, stream=None):
        if self._h is None:
            raise ValueError("graph is destroyed")
        _check(load().colibri_moe_graph_launch(self._h, _stream(stream)), "colibri_moe_graph_launch")

    def destroy(self):
        if self._h is not None:
            h, self._h = self._h, None
            _check(load().colibri_moe_graph_destroy(h), "colibri_moe_graph_destroy")


# ------------------------------------------------------------------ int8 expert weights
def _experts_q8(q1, s1, q2, s2, q3=None, s3=None, b1=None, b2=None, shape=None) -> _ExpertsQ8:
    if shape is None:
        return _ExpertsQ8(_ptr(q1), _ptr(q3), _ptr(q2), _ptr(s1), _ptr(s3), _ptr(s2), _ptr(b1), _ptr(b2))
    E, d, h, es = shape.E, shape.d, shape.h, _es(shape)
    return _ExpertsQ8(_ptr(q1, E * d * h, 1, "q1"), _ptr(q3, E * d * h, 1, "q3"), _ptr(q2, E * h * d, 1, "q2"),
                      _ptr(s1, E * h * 4, 4, "s1"), _ptr(s3, E * h * 4, 4, "s3"), _ptr(s2, E * d * 4, 4, "s2"),
                      _ptr(b1, E * h * es, es, "b1"), _ptr(b2, E * d * es, es, "b2"))


def quantize_q8(w, dtype: int, E: int, K: int, N: int, q, scale, stream=None):
    """Per-column int8 codes q [E, K, N] and fp32 scales [E, N] of w [E, K, N]."""
    n, es = E * K * N, 4 if dtype == F32 else 2
    _check(load().colibri_moe_quantize_q8(_ptr(w, n * es, es, "w"), int(dtype), int(E), int(K), int(N),
                                          _ptr(q, n, 1, "q"), _ptr(scale, E * N * 4, 4, "scale"), _stream(stream)),
           "colibri_moe_quantize_q8")


def expert_ffn_q8(shape: Shape, x_rows, sorted_assign, offsets, q1, s1, q2, s2, y_sorted, ws,
                  ws_bytes: Optional[int] = None, q3=None, s3=None, b1=None, b2=None, stream=None):
    s = shape.c()
    e = _experts_q8(q1, s1, q2, s2, q3, s3, b1, b2, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_expert_ffn_q8(ctypes.byref(s), *_rows_args(shape, x_rows, sorted_assign, offsets,
                                                                        shape.d), ctypes.byref(e),
                                            _ptr(y_sorted, 2 * shape.T * shape.d * es, es, "y_sorted"),
                                            *_ws(ws, ws_bytes), _stream(stream)), "colibri_moe_expert_ffn_q8")


def layer_forward_q8(shape: Shape, x, w_r, b_r, q1, s1, q2, s2, out, ws, ws_bytes: Optional[int] = None, q3=None,
                     s3=None, b1=None, b2=None, topk_idx=None, topk_gate=None, counts=None, stream=None):
    s = shape.c()
    e = _experts_q8(q1, s1, q2, s2, q3, s3, b1, b2, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_layer_forward_q8(ctypes.byref(s), *_router_args(shape, x, w_r, b_r), ctypes.byref(e),
                                               _ptr(out, shape.T * shape.d * es, es, "out"),
                                               *_routing_outs(shape, topk_idx, topk_gate, counts), *_ws(ws, ws_bytes),
                                               _stream(stream)), "colibri_moe_layer_forward_q8")


# ------------------------------------------------------------------ 4-bit expert weights
def _experts_q4(w1q, w2q, w3q=None, b1=None, b2=None, shape=None) -> _ExpertsQ4:
    t = lambda w: (None, None, None) if w is None else w
    (q1, s1, z1), (q2, s2, z2), (q3, s3, z3) = t(w1q), t(w2q), t(w3q)
    if shape is None:
        return _ExpertsQ4(_ptr(q1), _ptr(q3), _ptr(q2), _ptr(s1), _ptr(s3), _ptr(s2), _ptr(z1), _ptr(z3), _ptr(z2),
                          _ptr(b1), _ptr(b2))
    E, d, h, es = shape.E, shape.d, shape.h, _es(shape)
    up, dn = E * d * h, E * h * d  # weights per layer
    return _ExpertsQ4(_ptr(q1, up // 2, 4, "q1"), _ptr(q3, up // 2, 4, "q3"), _ptr(q2, dn // 2, 4, "q2"),
                      _ptr(s1, up // 128 * 4, 4, "s1"), _ptr(s3, up // 128 * 4, 4, "s3"), _ptr(s2, dn // 128 * 4, 4, "s2"),
                      _ptr(z1, up // 128, 1, "z1"), _ptr(z3, up // 128, 1, "z3"), _ptr(z2, dn // 128, 1, "z2"),
                      _ptr(b1, E * h * es, es, "b1"), _ptr(b2, E * d * es, es, "b2"))


def quantize_q4(w, dtype: int, E: int, K: int, N: int, q, scale, zero, stream=None):
    """4-bit codes q [E, K/8, N] (uint32 words of 8 codes: k = 8j + 2m in bits
    4m..4m+3, k = 8j + 2m + 1 in bits 16+4m..16+4m+3), fp32 scales and uint8
    zero points [E, K/128, N] of w [E, K, N]."""
    n, es = E * K * N, 4 if dtype == F32 else 2
    _check(load().colibri_moe_quantize_q4(_ptr(w, n * es, es, "w"), int(dtype), int(E), int(K), int(N),
                                          _ptr(q, n // 2, 4, "q"), _ptr(scale, n // 128 * 4, 4, "scale"),
                                          _ptr(zero, n // 128, 1, "zero"), _stream(stream)), "colibri_moe_quantize_q4")


def expert_ffn_q4(shape: Shape, x_rows, sorted_assign, offsets, w1q, w2q, y_sorted, ws,
                  ws_bytes: Optional[int] = None, w3q=None, b1=None, b2=None, stream=None):
    """w1q, w2q, w3q: (codes, scales, zero points) device triples."""
    s = shape.c()
    e = _experts_q4(w1q, w2q, w3q, b1, b2, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_expert_ffn_q4(ctypes.byref(s), *_rows_args(shape, x_rows, sorted_assign, offsets,
                                                                        shape.d), ctypes.byref(e),
                                            _ptr(y_sorted, 2 * shape.T * shape.d * es, es, "y_sorted"),
                                            *_ws(ws, ws_bytes), _stream(stream)), "colibri_moe_expert_ffn_q4")


def layer_forward_q4(shape: Shape, x, w_r, b_r, w1q, w2q, out, ws, ws_bytes: Optional[int] = None, w3q=None,
                     b1=None, b2=None, topk_idx=None, topk_gate=None, counts=None, stream=None):
    s = shape.c()
    e = _experts_q4(w1q, w2q, w3q, b1, b2, shape=shape)
    es = _es(shape)
    _check(load().colibri_moe_layer_forward_q4(ctypes.byref(s), *_router_args(shape, x, w_r, b_r), ctypes.byref(e),
                                               _ptr(out, shape.T * shape.d * es, es, "out"),
                                               *_routing_outs(shape, topk_idx, topk_gate, counts), *_ws(ws, ws_bytes),
                                               _stream(stream)), "colibri_moe_layer_forward_q4")


class MoELayer:
    """Device-resident layer: weights and a workspace sized for up to max_T tokens.

    Holds torch tensors (memory only) and calls colibri_moe_layer_forward."""

    def __init__(self, shape: Shape, w_r, w1, w2, w3=None, b1=None, b2=None, b_r=None):
        import torch
        self.shape = shape
        self.w_r, self.w1, self.w2, self.w3, self.b1, self.b2, self.b_r = w_r, w1, w2, w3, b1, b2, b_r
        self.ws_bytes = workspace_size(shape)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=w1.device)

    def forward(self, x, out, topk_idx=None, topk_gate=None, counts=None, stream=None):
        T = x.shape[0]
        if T > self.shape.T:
            raise ValueError(f"T={T} exceeds the workspace's T={self.shape.T}")
        sh = self.shape.with_T(T)
        layer_forward(sh, x, self.w_r, self.b_r, self.w1, self.w2, out, self.ws, self.ws_bytes, w3=self.w3,
                      b1=self.b1, b2=self.b2, topk_idx=topk_idx, topk_gate=topk_gate, counts=counts, stream=stream)
        return out
