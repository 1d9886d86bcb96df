"""fp64 CPU oracle of the MoE layer forward pass (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it.

Thin ctypes wrapper over ``colibri_oracle.cpp``: numpy arrays in, numpy
arrays out.  Inputs are the stored tensors (float32, or bf16 bit patterns as
uint16); results are float64 (values) or int32 (indices).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "colibri_oracle.cpp")
_SO = os.path.join(_HERE, "liboracle.so")

DT_F32, DT_BF16 = 0, 1
ACT = {"relu": 0, "gelu": 1, "swiglu": 2}
# gating of the chosen pair: pair softmax, softmax over all experts (unnormalised
# pair), or the raw logits
GATE = {"pair": 0, "softmax": 1, "linear": 2}

# -ffp-contract=off: no fused multiply-add, so every product and sum is rounded
# exactly as written; no fast-math.
CFLAGS = ["-O3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c++17"]


def build(extra_flags=()) -> str:
    cmd = ["g++", *CFLAGS, *extra_flags, _SRC, "-o", _SO + ".tmp"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None
_P = ctypes.c_void_p


def load_library(path: Optional[str] = None):
    """Load the oracle (building it if absent).  A path loads a separate build."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    so = path or _SO
    if path is None and not os.path.exists(so):
        build()
    lib = ctypes.CDLL(so)
    i, d, z = ctypes.c_int, ctypes.c_double, ctypes.c_size_t
    lib.oracle_set_threads.argtypes = [i]
    lib.oracle_max_threads.restype = i
    lib.oracle_logits.argtypes = [i, i, i, i, _P, _P, _P, _P]
    lib.oracle_top2.argtypes = [i, i, _P, _P]
    lib.oracle_gates.argtypes = [i, i, _P, _P, _P]
    lib.oracle_gates_mode.argtypes = [i, i, i, _P, _P, _P]
    lib.oracle_combine_ex.argtypes = [i, i, i, _P, _P, _P, _P, _P, _P]
    lib.oracle_dispatch.argtypes = [i, i, _P, _P, _P, _P, _P]
    lib.oracle_ffn_rows.argtypes = [i, i, i, i, i, _P, i, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_combine.argtypes = [i, i, i, _P, _P, _P, _P]
    lib.oracle_layer.argtypes = [i, i, i, i, i, i, i] + [_P] * 8 + [_P] * 9
    lib.oracle_round.argtypes = [_P, _P, z, i]
    lib.oracle_quantize_q8.argtypes = [_P, i, i, i, i, _P, _P]
    lib.oracle_ffn_rows_q8.argtypes = [i, i, i, i, i, _P, i, _P, _P] + [_P] * 8 + [_P]
    lib.oracle_quantize_q4.argtypes = [_P, i, i, i, i, _P, _P, _P]
    lib.oracle_ffn_rows_q4.argtypes = [i, i, i, i, i, _P, i, _P, _P] + [_P] * 11 + [_P]
    for f in ("oracle_set_threads", "oracle_logits", "oracle_top2", "oracle_gates", "oracle_dispatch",
              "oracle_ffn_rows", "oracle_combine", "oracle_layer", "oracle_round", "oracle_quantize_q8",
              "oracle_ffn_rows_q8", "oracle_gates_mode", "oracle_combine_ex", "oracle_quantize_q4",
              "oracle_ffn_rows_q4"):
        getattr(lib, f).restype = None
    if path is None:
        _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    raise TypeError(f"oracle inputs are float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


def set_threads(n: int, lib=None):
    (lib or load_library()).oracle_set_threads(int(n))


def max_threads(lib=None) -> int:
    return int((lib or load_library()).oracle_max_threads())


def logits(x, w_r, b_r=None, lib=None) -> np.ndarray:
    lib = lib or load_library()
    x, w_r = _c(x), _c(w_r)
    T, d = x.shape
    E = w_r.shape[1]
    b_r = _c(b_r, np.float32)
    out = np.empty((T, E), np.float64)
    lib.oracle_logits(T, d, E, _dt(x), _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(out))
    return out


def top2(lg: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load_library()
    lg = _c(lg, np.float64)
    T, E = lg.shape
    idx = np.empty((T, 2), np.int32)
    lib.oracle_top2(T, E, _ptr(lg), _ptr(idx))
    return idx


def gates(lg: np.ndarray, idx: np.ndarray, mode: str = "pair", lib=None) -> np.ndarray:
    lib = lib or load_library()
    lg = _c(lg, np.float64)
    idx = _c(idx, np.int32)
    T, E = lg.shape
    g = np.empty((T, 2), np.float64)
    if mode == "pair":
        lib.oracle_gates(T, E, _ptr(lg), _ptr(idx), _ptr(g))
    else:
        lib.oracle_gates_mode(T, E, GATE[mode], _ptr(lg), _ptr(idx), _ptr(g))
    return g


def dispatch(idx: np.ndarray, E: int, lib=None) -> Dict[str, np.ndarray]:
    lib = lib or load_library()
    idx = _c(idx, np.int32)
    T = idx.shape[0]
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sa = np.empty(2 * T, np.int32)
    ap = np.empty(2 * T, np.int32)
    lib.oracle_dispatch(T, E, _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(sa), _ptr(ap))
    return {"counts": counts, "offsets": offsets, "sorted_assign": sa, "assign_pos": ap}


def ffn_rows(x, rows_token, rows_expert, w1, w2, act: str, w3=None, b1=None, b2=None, mirror=True,
             lib=None) -> np.ndarray:
    lib = lib or load_library()
    x, w1, w2, w3, b1, b2 = (_c(a) for a in (x, w1, w2, w3, b1, b2))
    dt = _dt(x)
    for a in (w1, w2, w3, b1, b2):
        if a is not None and _dt(a) != dt:
            raise TypeError("all layer tensors share one dtype")
    E, d, h = w1.shape
    rt = _c(rows_token, np.int32)
    re = _c(rows_expert, np.int32)
    n = rt.shape[0]
    if act == "swiglu" and w3 is None:
        raise ValueError("swiglu needs w3")
    y = np.empty((n, d), np.float64)
    lib.oracle_ffn_rows(d, h, dt, ACT[act], int(bool(mirror)), _ptr(x), n, _ptr(rt), _ptr(re), _ptr(w1),
                        _ptr(w3), _ptr(w2), _ptr(b1), _ptr(b2), _ptr(y))
    return y


def combine(y_sorted, assign_pos, gate, dtype: int, shared_y=None, residual=None, lib=None) -> np.ndarray:
    """Gate-weighted pair; with ``shared_y`` [T, d] (float64) and/or ``residual``
    [T, d] (stored dtype) added before the rounding."""
    lib = lib or load_library()
    y = _c(y_sorted, np.float64)
    ap = _c(assign_pos, np.int32)
    g = _c(gate, np.float64)
    T = ap.shape[0] // 2
    d = y.shape[1]
    out = np.empty((T, d), np.float64)
    if shared_y is None and residual is None:
        lib.oracle_combine(T, d, dtype, _ptr(y), _ptr(ap), _ptr(g), _ptr(out))
        return out
    sh = _c(shared_y, np.float64)
    res = _c(residual)
    if res is not None and _dt(res) != dtype:
        raise TypeError("residual must be stored in the layer dtype")
    lib.oracle_combine_ex(T, d, dtype, _ptr(y), _ptr(ap), _ptr(g), _ptr(sh), _ptr(res), _ptr(out))
    return out


def layer(x, w_r, w1, w2, act: str, b_r=None, w3=None, b1=None, b2=None, mirror=True,
          lib=None) -> Dict[str, np.ndarray]:
    lib = lib or load_library()
    x, w_r, w1, w2, w3, b1, b2 = (_c(a) for a in (x, w_r, w1, w2, w3, b1, b2))
    b_r = _c(b_r, np.float32)
    T, d = x.shape
    E, _, h = w1.shape
    dt = _dt(x)
    r = {
        "logits": np.empty((T, E), np.float64), "idx": np.empty((T, 2), np.int32),
        "gate": np.empty((T, 2), np.float64), "counts": np.empty(E, np.int32),
        "offsets": np.empty(E + 1, np.int32), "sorted_assign": np.empty(2 * T, np.int32),
        "assign_pos": np.empty(2 * T, np.int32), "y_sorted": np.empty((2 * T, d), np.float64),
        "out": np.empty((T, d), np.float64),
    }
    lib.oracle_layer(T, d, h, E, dt, ACT[act], int(bool(mirror)), _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(w1),
                     _ptr(w3), _ptr(w2), _ptr(b1), _ptr(b2), *(_ptr(r[k]) for k in (
                         "logits", "idx", "gate", "counts", "offsets", "sorted_assign", "assign_pos",
                         "y_sorted", "out")))
    return r


def layer_tokens(x, w_r, w1, w2, act: str, tokens, b_r=None, w3=None, b1=None, b2=None, mirror=True,
                 idx_override=None, gate="pair", shared=None, residual=None, lib=None) -> Dict[str, np.ndarray]:
    """Layer outputs for a sample of tokens only (each token's row depends only on
    that token).  ``idx_override`` [len(tokens), 2] forces the chosen experts
    (gates are then taken from the oracle's own logits for that pair).

    ``gate``: "pair" | "softmax" | "linear" (see ``gates``).  ``shared``: a dict
    with the shared expert's w1, w2 (and w3, b1, b2), each with a leading expert
    axis of 1; its output (rounded to the dtype when ``mirror``) is added with
    weight one.  ``residual`` [T, d] (all tokens, stored dtype) is added last."""
    lib = lib or load_library()
    tokens = np.asarray(tokens, np.int64)
    xs = _c(np.asarray(x)[tokens])
    lg = logits(xs, w_r, b_r, lib=lib)
    idx = top2(lg, lib=lib) if idx_override is None else _c(idx_override, np.int32)
    g = gates(lg, idx, mode=gate, lib=lib)
    n = len(tokens)
    rt = np.repeat(np.arange(n, dtype=np.int32), 2)
    re = idx.reshape(-1)
    y = ffn_rows(xs, rt, re, w1, w2, act, w3=w3, b1=b1, b2=b2, mirror=mirror, lib=lib)
    ap = np.arange(2 * n, dtype=np.int32)
    ysh = None
    if shared is not None:
        ysh = ffn_rows(xs, np.arange(n, dtype=np.int32), np.zeros(n, np.int32), shared["w1"], shared["w2"], act,
                       w3=shared.get("w3"), b1=shared.get("b1"), b2=shared.get("b2"), mirror=mirror, lib=lib)
    res = None if residual is None else _c(np.asarray(residual)[tokens])
    out = combine(y, ap, g, _dt(xs), shared_y=ysh, residual=res, lib=lib)
    r = {"logits": lg, "idx": idx, "gate": g, "y": y.reshape(n, 2, -1), "out": out}
    if ysh is not None:
        r["y_shared"] = ysh
    return r


# ------------------------------------------------------------------ int8 expert weights
def quantize_q8(w, lib=None):
    """Per-column int8 codes and fp32 scales of w [E, K, N] (float32 or bf16 bits)."""
    lib = lib or load_library()
    w = _c(w)
    E, K, N = w.shape
    q = np.empty((E, K, N), np.int8)
    s = np.empty((E, N), np.float32)
    lib.oracle_quantize_q8(_ptr(w), _dt(w), E, K, N, _ptr(q), _ptr(s))
    return q, s


def ffn_rows_q8(x, rows_token, rows_expert, q1, s1, q2, s2, act: str, q3=None, s3=None, b1=None, b2=None,
                mirror=True, lib=None) -> np.ndarray:
    """ffn_rows with int8 weights q* and per-column scales s* (dequantized as s * q)."""
    lib = lib or load_library()
    x, b1, b2 = _c(x), _c(b1), _c(b2)
    q1, q2, q3 = _c(q1, np.int8), _c(q2, np.int8), _c(q3, np.int8)
    s1, s2, s3 = _c(s1, np.float32), _c(s2, np.float32), _c(s3, np.float32)
    dt = _dt(x)
    for a in (b1, b2):
        if a is not None and _dt(a) != dt:
            raise TypeError("x and the biases share one dtype")
    E, d, h = q1.shape
    rt = _c(rows_token, np.int32)
    re = _c(rows_expert, np.int32)
    n = rt.shape[0]
    if act == "swiglu" and (q3 is None or s3 is None):
        raise ValueError("swiglu needs q3 and s3")
    y = np.empty((n, d), np.float64)
    lib.oracle_ffn_rows_q8(d, h, dt, ACT[act], int(bool(mirror)), _ptr(x), n, _ptr(rt), _ptr(re), _ptr(q1),
                           _ptr(s1), _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(b1), _ptr(b2), _ptr(y))
    return y


def layer_tokens_q8(x, w_r, q1, s1, q2, s2, act: str, tokens, b_r=None, q3=None, s3=None, b1=None, b2=None,
                    mirror=True, idx_override=None, lib=None) -> Dict[str, np.ndarray]:
    """layer_tokens with int8 expert weights."""
    lib = lib or load_library()
    tokens = np.asarray(tokens, np.int64)
    xs = _c(np.asarray(x)[tokens])
    lg = logits(xs, w_r, b_r, lib=lib)
    idx = top2(lg, lib=lib) if idx_override is None else _c(idx_override, np.int32)
    g = gates(lg, idx, lib=lib)
    n = len(tokens)
    rt = np.repeat(np.arange(n, dtype=np.int32), 2)
    y = ffn_rows_q8(xs, rt, idx.reshape(-1), q1, s1, q2, s2, act, q3=q3, s3=s3, b1=b1, b2=b2, mirror=mirror,
                    lib=lib)
    out = combine(y, np.arange(2 * n, dtype=np.int32), g, _dt(xs), lib=lib)
    return {"logits": lg, "idx": idx, "gate": g, "y": y.reshape(n, 2, -1), "out": out}


# ------------------------------------------------------------------ 4-bit expert weights
Q4_GROUP = 128


def quantize_q4(w, lib=None):
    """4-bit codes [E, K, N] (uint8, 0..15), fp32 scales and uint8 zero points
    [E, K/128, N] of w [E, K, N] (float32 or bf16 bits); W = s * (q - z)."""
    lib = lib or load_library()
    w = _c(w)
    E, K, N = w.shape
    if K % Q4_GROUP:
        raise ValueError("K must be a multiple of 128")
    q = np.empty((E, K, N), np.uint8)
    s = np.empty((E, K // Q4_GROUP, N), np.float32)
    z = np.empty((E, K // Q4_GROUP, N), np.uint8)
    lib.oracle_quantize_q4(_ptr(w), _dt(w), E, K, N, _ptr(q), _ptr(s), _ptr(z))
    return q, s, z


def ffn_rows_q4(x, rows_token, rows_expert, w1q, w2q, act: str, w3q=None, b1=None, b2=None, mirror=True,
                lib=None) -> np.ndarray:
    """ffn_rows with 4-bit weights; each w*q is a (codes, scales, zeros) triple
    as quantize_q4 returns it."""
    lib = lib or load_library()
    x, b1, b2 = _c(x), _c(b1), _c(b2)
    dt = _dt(x)
    for a in (b1, b2):
        if a is not None and _dt(a) != dt:
            raise TypeError("x and the biases share one dtype")
    if act == "swiglu" and w3q is None:
        raise ValueError("swiglu needs w3q")
    f = lambda t: (None, None, None) if t is None else (_c(t[0], np.uint8), _c(t[1], np.float32), _c(t[2], np.uint8))
    (q1, s1, z1), (q2, s2, z2), (q3, s3, z3) = f(w1q), f(w2q), f(w3q)
    E, d, h = q1.shape
    rt = _c(rows_token, np.int32)
    re = _c(rows_expert, np.int32)
    n = rt.shape[0]
    y = np.empty((n, d), np.float64)
    lib.oracle_ffn_rows_q4(d, h, dt, ACT[act], int(bool(mirror)), _ptr(x), n, _ptr(rt), _ptr(re), _ptr(q1),
                           _ptr(s1), _ptr(z1), _ptr(q3), _ptr(s3), _ptr(z3), _ptr(q2), _ptr(s2), _ptr(z2),
                           _ptr(b1), _ptr(b2), _ptr(y))
    return y


def layer_tokens_q4(x, w_r, w1q, w2q, act: str, tokens, b_r=None, w3q=None, b1=None, b2=None, mirror=True,
                    idx_override=None, lib=None) -> Dict[str, np.ndarray]:
    """layer_tokens with 4-bit expert weights."""
    lib = lib or load_library()
    tokens = np.asarray(tokens, np.int64)
    xs = _c(np.asarray(x)[tokens])
    lg = logits(xs, w_r, b_r, lib=lib)
    idx = top2(lg, lib=lib) if idx_override is None else _c(idx_override, np.int32)
    g = gates(lg, idx, lib=lib)
    n = len(tokens)
    rt = np.repeat(np.arange(n, dtype=np.int32), 2)
    y = ffn_rows_q4(xs, rt, idx.reshape(-1), w1q, w2q, act, w3q=w3q, b1=b1, b2=b2, mirror=mirror, lib=lib)
    out = combine(y, np.arange(2 * n, dtype=np.int32), g, _dt(xs), lib=lib)
    return {"logits": lg, "idx": idx, "gate": g, "y": y.reshape(n, 2, -1), "out": out}


def round_to(a: np.ndarray, dtype: int, lib=None) -> np.ndarray:
    lib = lib or load_library()
    a = _c(a, np.float64)
    o = np.empty_like(a)
    lib.oracle_round(_ptr(a), _ptr(o), a.size, dtype)
    return o
