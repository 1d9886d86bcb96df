"""Seeded synthetic inputs for the MoE layer (shared by tests, bench and smoke).

This module only draws random numbers and lays them out; it contains none of
the layer's arithmetic.  The draw is Philox-4x32-10 + Box-Muller
(``philox_gen.c``), keyed by (seed, tensor id), one stream per tensor, with the
flat element index as the counter.  A prefix of a stream is therefore the same
whatever length is requested, so T=1 decode inputs are the first row of the
T=32 inputs.

Workload recipes follow the layer shapes of the models the Colibri write-ups
talk about (see ``CONFIGS``); "N(0, v)" reads v as the variance.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox_gen.c")
_SO = os.path.join(_HERE, "libgen.so")

# tensor ids (Philox key word 1); the seed is key word 0
TID_X, TID_WR, TID_W1, TID_B1, TID_W3, TID_W2, TID_B2 = 1, 2, 10, 11, 12, 13, 14
TID_SH_W1, TID_SH_B1, TID_SH_W3, TID_SH_W2, TID_SH_B2 = 20, 21, 22, 23, 24  # shared expert
TID_RES = 30  # residual rows

F32, BF16 = 0, 1


def build() -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.gen_normal.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.gen_normal.restype = None
        lib.gen_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        lib.gen_philox4x32_10.restype = None
        lib.gen_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]
        lib.gen_f32_to_bf16.restype = None
        _lib = lib
    return _lib


def philox4x32_10(ctr, key):
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib.gen_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def normal(seed: int, tensor_id: int, shape, std: float, dtype: int, begin: int = 0) -> np.ndarray:
    """Elements [begin, begin+prod(shape)) of stream (seed, tensor_id), times std.

    dtype F32 returns float32; BF16 returns the bf16 bit patterns as uint16."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    if n:
        _load().gen_normal(seed, tensor_id, begin, n, float(std), dtype, out.ctypes.data)
    return out.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().gen_f32_to_bf16(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Config:
    key: str
    title: str
    E: int
    d: int
    h: int
    act: str           # "relu" | "gelu" | "swiglu"
    dtype: int         # F32 | BF16
    Ts: List[int]
    biases: bool       # b1/b2 present
    router_bias: Optional[str] = None   # None | "zipf"
    zipf_s: float = 0.0
    seed: int = 0
    shared_h: int = 0      # hidden width of an always-on shared expert (0: none)
    gate: str = "pair"     # gating of the chosen pair: "pair" | "softmax" | "linear"


CONFIGS: Dict[str, Config] = {
    # the 4-expert demo model the first write-up runs (two-layer FFN experts)
    "tiny": Config("tiny", "tiny-moe-4e2r layer", E=4, d=64, h=128, act="relu", dtype=F32,
                   Ts=[32], biases=True),
    # 1.3B-class 8-expert MoE layer
    "e8": Config("e8", "8-expert 1.3B-class layer", E=8, d=2048, h=5632, act="gelu", dtype=BF16,
                 Ts=[1, 64, 512], biases=True),
    # Mixtral-8x7B-shaped layer, decode batch sizes
    "mixtral_decode": Config("mixtral_decode", "Mixtral-shaped decode layer", E=8, d=4096, h=14336,
                             act="swiglu", dtype=BF16, Ts=[1, 4, 16, 32], biases=False),
    # Mixtral-8x7B-shaped layer, one 4096-token prefill
    "mixtral_prefill": Config("mixtral_prefill", "Mixtral-shaped prefill layer", E=8, d=4096, h=14336,
                              act="swiglu", dtype=BF16, Ts=[4096], biases=False),
    # 16 experts with Zipf(1.2) expert popularity set by a fitted router bias
    "skew16": Config("skew16", "16-expert Zipf-skewed layer", E=16, d=3584, h=2560, act="swiglu",
                     dtype=BF16, Ts=[8192], biases=False, router_bias="zipf", zipf_s=1.2),
    # 1 shared + 15 routed experts (the Qwen2-MoE split), softmax over all
    # experts without renormalising the pair; widths of a 2.7B-active layer
    # (routed h 1408, shared h 4 x 1408)
    "shared15": Config("shared15", "15 routed + 1 shared expert layer", E=15, d=2048, h=1408, act="swiglu",
                       dtype=BF16, Ts=[1, 64, 512], biases=False, shared_h=5632, gate="softmax"),
}

ACT_CODE = {"relu": 0, "gelu": 1, "swiglu": 2}

_GOLDEN = os.path.join(os.path.dirname(_HERE), "tests", "golden")


def router_bias(cfg: Config) -> Optional[np.ndarray]:
    """Router bias b_r [E] fp32, or None.  The Zipf-fitted bias is a stored input
    written by tests/golden/make_skew16_router_bias.py."""
    if cfg.router_bias is None:
        return None
    path = os.path.join(_GOLDEN, f"{cfg.key}_router_bias.txt")
    vals = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals.append(float.fromhex(line.split()[0]))
    b = np.array(vals, dtype=np.float32)
    assert b.shape == (cfg.E,), b.shape
    return b


def make_x(cfg: Config, T: int) -> np.ndarray:
    return normal(cfg.seed, TID_X, (T, cfg.d), 1.0, cfg.dtype)


def make_router(cfg: Config) -> np.ndarray:
    return normal(cfg.seed, TID_WR, (cfg.d, cfg.E), 1.0 / math.sqrt(cfg.d), cfg.dtype)


def make_experts(cfg: Config) -> Dict[str, Optional[np.ndarray]]:
    E, d, h, dt = cfg.E, cfg.d, cfg.h, cfg.dtype
    w = {
        "w1": normal(cfg.seed, TID_W1, (E, d, h), 1.0 / math.sqrt(d), dt),
        "w3": normal(cfg.seed, TID_W3, (E, d, h), 1.0 / math.sqrt(d), dt) if cfg.act == "swiglu" else None,
        "w2": normal(cfg.seed, TID_W2, (E, h, d), 1.0 / math.sqrt(h), dt),
        "b1": normal(cfg.seed, TID_B1, (E, h), 0.1, dt) if cfg.biases else None,
        "b2": normal(cfg.seed, TID_B2, (E, d), 0.1, dt) if cfg.biases else None,
    }
    return w


def make_shared_expert(cfg: Config) -> Dict[str, Optional[np.ndarray]]:
    """The shared expert's weights, laid out as one expert: w1 [1, d, shared_h] ..."""
    d, h, dt = cfg.d, cfg.shared_h or cfg.h, cfg.dtype
    return {
        "w1": normal(cfg.seed, TID_SH_W1, (1, d, h), 1.0 / math.sqrt(d), dt),
        "w3": normal(cfg.seed, TID_SH_W3, (1, d, h), 1.0 / math.sqrt(d), dt) if cfg.act == "swiglu" else None,
        "w2": normal(cfg.seed, TID_SH_W2, (1, h, d), 1.0 / math.sqrt(h), dt),
        "b1": normal(cfg.seed, TID_SH_B1, (1, h), 0.1, dt) if cfg.biases else None,
        "b2": normal(cfg.seed, TID_SH_B2, (1, d), 0.1, dt) if cfg.biases else None,
    }


def make_residual(cfg: Config, T: int) -> np.ndarray:
    """Residual rows [T, d] ~ N(0, 1), in the layer dtype."""
    return normal(cfg.seed, TID_RES, (T, cfg.d), 1.0, cfg.dtype)


def layer_of(cfg: Config, l: int) -> Config:
    """Layer l of a multi-layer stack of this shape: its own weights (seed
    cfg.seed + 1000 l; layer 0 is the single-layer workload itself)."""
    import dataclasses
    return cfg if l == 0 else dataclasses.replace(cfg, seed=cfg.seed + 1000 * l)


def make_all(cfg: Config, T: int) -> Dict[str, Optional[np.ndarray]]:
    out = {"x": make_x(cfg, T), "w_r": make_router(cfg), "b_r": router_bias(cfg)}
    out.update(make_experts(cfg))
    return out
