"""Helpers for the GPU parity tests: device copies of seeded inputs, the
tolerance rules, and the near-tie bookkeeping."""
from __future__ import annotations

import functools
import json
import os
from typing import Dict, Optional

import numpy as np

import gen
import mixture_experts_layer_12_amd as moe
import oracle

NEAR_TIE = 1e-6  # logit margin below which a token's expert choice is exempt


def torch():
    import torch as _t
    return _t


def dev(a: Optional[np.ndarray]):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).cuda().view(t.bfloat16)
    if a.dtype == np.uint32:  # packed 4-bit codes: carried as int32
        return t.from_numpy(a.view(np.int32)).cuda()
    return t.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    """device tensor -> numpy (bf16 widened exactly to float32)."""
    T = torch()
    if t.dtype == T.bfloat16:
        return gen.bf16_bits_to_f32(t.view(T.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def empty(shape, dtype):
    T = torch()
    return T.empty(shape, dtype=dtype, device="cuda")


def tdtype(dt: int):
    T = torch()
    return T.float32 if dt == gen.F32 else T.bfloat16


# ------------------------------------------------------------------ tolerances
def fp32_rel_err(a, b) -> float:
    """Largest per-row relative error: max over rows r of
    max_c |a_rc - b_rc| / max_c |b_rc|  (a 1-D array is one row).

    fp32 accumulation error scales with the magnitude of the summands, i.e.
    with the row's scale, not with each element, so an elementwise ratio is
    unbounded where a sum cancels to near zero; each output vector (a token's
    logits, gates or hidden/output row) is therefore judged against its own
    largest element."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return 0.0
    a2 = a.reshape(a.shape[0], -1) if a.ndim >= 2 else a.reshape(1, -1)
    b2 = b.reshape(b.shape[0], -1) if b.ndim >= 2 else b.reshape(1, -1)
    scale = np.maximum(np.abs(b2).max(axis=1), 1e-30)
    return float((np.abs(a2 - b2).max(axis=1) / scale).max())


def assert_fp32_close(a, b, what, tol=1e-4):
    err = fp32_rel_err(a, b)
    assert err <= tol, f"{what}: max relative error {err:.3e} > {tol:.0e}"


def assert_bf16_close(a, b, what, atol=1e-2, rtol=2e-2):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    bad = np.abs(a - b) > atol + rtol * np.abs(b)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside |a-b| <= {atol} + {rtol}|b|; "
                           f"worst |a-b| = {np.abs(a - b).max():.3e}")


def assert_close(a, b, dt, what):
    if dt == gen.F32:
        assert_fp32_close(a, b, what)
    else:
        assert_bf16_close(a, b, what)


def assert_layer_close(a, ref, dt, what, residual=None):
    """Layer outputs with a shared expert, a residual or raw-logit gates.

    fp32: the row rule.  bf16: |a - b| <= 1e-2 + 2e-2 M per element, where M is
    the largest magnitude among b and the summands of the combine (g0 y0, g1 y1,
    the shared row, the residual row).  Both sides store the expert rows in
    bf16; where an fp32 sum lands on a rounding boundary the two round a row to
    neighbouring values, and that one-ulp step is relative to the row, not to
    the sum, which may cancel to far less.  With no addends and convex gates M
    is at most the larger gated row."""
    if dt == gen.F32:
        assert_fp32_close(a, ref["out"], what)
        return
    a = np.asarray(a, np.float64)
    b = np.asarray(ref["out"], np.float64)
    g, y = ref["gate"], ref["y"]
    M = np.maximum(np.abs(b), np.abs(g[:, :1] * y[:, 0]))
    M = np.maximum(M, np.abs(g[:, 1:] * y[:, 1]))
    if "y_shared" in ref:
        M = np.maximum(M, np.abs(ref["y_shared"]))
    if residual is not None:
        M = np.maximum(M, np.abs(np.asarray(residual, np.float64)))
    bad = np.abs(a - b) > 1e-2 + 2e-2 * M
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside |a-b| <= 1e-2 + 2e-2 M; "
                           f"worst |a-b| = {np.abs(a - b).max():.3e}")


# ------------------------------------------------------------------ near ties
def near_tie_mask(lg: np.ndarray) -> np.ndarray:
    """Tokens whose 1st/2nd or 2nd/3rd logit margin (oracle fp64) is < NEAR_TIE."""
    s = -np.sort(-lg, axis=1)
    m12 = s[:, 0] - s[:, 1]
    m23 = s[:, 1] - s[:, 2] if lg.shape[1] > 2 else np.full(lg.shape[0], np.inf)
    return np.minimum(m12, m23) < NEAR_TIE


def report(record: Dict):
    """Append one line to the parity report (path from COLIBRI_PARITY_REPORT, if set)."""
    path = os.environ.get("COLIBRI_PARITY_REPORT")
    line = json.dumps(record, sort_keys=True)
    print(line, flush=True)
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


# ------------------------------------------------------------------ seeded layers
def weight_key(key: str) -> str:
    """Configs that draw identical weights (same shapes, activation, dtype, seed)
    share one cached copy: the Mixtral decode and prefill layers do."""
    c = gen.CONFIGS[key]
    for k, o in gen.CONFIGS.items():
        if (o.E, o.d, o.h, o.act, o.dtype, o.biases, o.seed) == (c.E, c.d, c.h, c.act, c.dtype, c.biases, c.seed):
            return k
    return key


@functools.lru_cache(maxsize=8)
def host_router(key: str):
    cfg = gen.CONFIGS[key]
    return {"w_r": gen.make_router(cfg), "b_r": gen.router_bias(cfg)}


@functools.lru_cache(maxsize=8)
def device_router(key: str):
    return {k: dev(v) for k, v in host_router(key).items()}


@functools.lru_cache(maxsize=1)
def _host_experts(wkey: str):
    return gen.make_experts(gen.CONFIGS[wkey])


@functools.lru_cache(maxsize=1)
def _device_experts(wkey: str):
    return {k: dev(v) for k, v in _host_experts(wkey).items()}


@functools.lru_cache(maxsize=1)
def _host_experts_q8(wkey: str):
    """int8 codes and per-column scales of the seeded weights, from the oracle's quantizer."""
    w = _host_experts(wkey)
    out = {"b1": w["b1"], "b2": w["b2"]}
    for name, qn, sn in (("w1", "q1", "s1"), ("w3", "q3", "s3"), ("w2", "q2", "s2")):
        if w[name] is None:
            out[qn] = out[sn] = None
        else:
            out[qn], out[sn] = oracle.quantize_q8(w[name])
    return out


@functools.lru_cache(maxsize=1)
def _device_experts_q8(wkey: str):
    return {k: dev(v) for k, v in _host_experts_q8(wkey).items()}


# bit offset of the code of k = 8j + i inside word j: 4m for k = 8j + 2m, 16 + 4m for k = 8j + 2m + 1
Q4_SHIFT = np.array([4 * (i // 2) + 16 * (i % 2) for i in range(8)], np.uint32)


def pack_q4(codes: np.ndarray) -> np.ndarray:
    """Codes [E, K, N] (0..15) -> the library's words [E, K/8, N]."""
    E, K, N = codes.shape
    c = codes.reshape(E, K // 8, 8, N).astype(np.uint32)
    return np.bitwise_or.reduce(c << Q4_SHIFT[None, None, :, None], axis=2)


def unpack_q4(words: np.ndarray) -> np.ndarray:
    E, KB, N = words.shape
    w = words.astype(np.uint32)[:, :, None, :] >> Q4_SHIFT[None, None, :, None]
    return (w & 0xF).astype(np.uint8).reshape(E, KB * 8, N)


@functools.lru_cache(maxsize=1)
def _host_experts_q4(wkey: str):
    """4-bit codes (unpacked and packed), scales and zero points of the seeded
    weights, from the oracle's quantizer."""
    w = _host_experts(wkey)
    out = {"b1": w["b1"], "b2": w["b2"]}
    for name, t in (("w1", "1"), ("w3", "3"), ("w2", "2")):
        if w[name] is None:
            out["w" + t + "q"] = None
        else:
            q, sc, z = oracle.quantize_q4(w[name])
            out["w" + t + "q"] = (q, sc, z)
    return out


@functools.lru_cache(maxsize=1)
def _device_experts_q4(wkey: str):
    h = _host_experts_q4(wkey)
    out = {"b1": dev(h["b1"]), "b2": dev(h["b2"])}
    for k in ("w1q", "w3q", "w2q"):
        out[k] = None if h[k] is None else (dev(pack_q4(h[k][0])), dev(h[k][1]), dev(h[k][2]))
    return out


class Layer:
    """Seeded inputs of one config at T tokens; expert weights load on first use."""

    def __init__(self, key: str, T: int):
        self.key = key
        self.cfg = gen.CONFIGS[key]
        self.T = T
        self.x = gen.make_x(self.cfg, T)

    @property
    def hw(self) -> Dict:
        w = dict(_host_experts(weight_key(self.key)))
        w.update(host_router(self.key))
        return w

    @property
    def dw(self) -> Dict:
        w = dict(_device_experts(weight_key(self.key)))
        w.update(device_router(self.key))
        return w

    @property
    def shape(self) -> moe.Shape:
        c = self.cfg
        return moe.Shape(self.T, c.d, c.h, c.E, c.dtype, gen.ACT_CODE[c.act])

    def oracle_tokens(self, tokens, idx_override=None):
        w = self.hw
        return oracle.layer_tokens(self.x, w["w_r"], w["w1"], w["w2"], self.cfg.act, tokens, b_r=w["b_r"],
                                   w3=w["w3"], b1=w["b1"], b2=w["b2"], mirror=True, idx_override=idx_override)


    @property
    def hq8(self) -> Dict:
        w = dict(_host_experts_q8(weight_key(self.key)))
        w.update(host_router(self.key))
        return w

    @property
    def dq8(self) -> Dict:
        w = dict(_device_experts_q8(weight_key(self.key)))
        w.update(device_router(self.key))
        return w

    def oracle_tokens_q8(self, tokens, idx_override=None):
        w = self.hq8
        return oracle.layer_tokens_q8(self.x, w["w_r"], w["q1"], w["s1"], w["q2"], w["s2"], self.cfg.act, tokens,
                                      b_r=w["b_r"], q3=w["q3"], s3=w["s3"], b1=w["b1"], b2=w["b2"], mirror=True,
                                      idx_override=idx_override)


    @property
    def hq4(self) -> Dict:
        w = dict(_host_experts_q4(weight_key(self.key)))
        w.update(host_router(self.key))
        return w

    @property
    def dq4(self) -> Dict:
        w = dict(_device_experts_q4(weight_key(self.key)))
        w.update(device_router(self.key))
        return w

    def oracle_tokens_q4(self, tokens, idx_override=None):
        w = self.hq4
        return oracle.layer_tokens_q4(self.x, w["w_r"], w["w1q"], w["w2q"], self.cfg.act, tokens, b_r=w["b_r"],
                                      w3q=w["w3q"], b1=w["b1"], b2=w["b2"], mirror=True, idx_override=idx_override)

    # ---- gating variants, shared expert, residual
    @property
    def h_shared(self) -> Dict:
        return _host_shared(self.key)

    @property
    def d_shared(self) -> Dict:
        return _device_shared(self.key)

    @property
    def residual(self) -> np.ndarray:
        return gen.make_residual(self.cfg, self.T)

    def oracle_tokens_ex(self, tokens, idx_override=None, gate="pair", shared=False, residual=False):
        w = self.hw
        return oracle.layer_tokens(self.x, w["w_r"], w["w1"], w["w2"], self.cfg.act, tokens, b_r=w["b_r"],
                                   w3=w["w3"], b1=w["b1"], b2=w["b2"], mirror=True, idx_override=idx_override,
                                   gate=gate, shared=self.h_shared if shared else None,
                                   residual=self.residual if residual else None)


@functools.lru_cache(maxsize=2)
def _host_shared(key: str):
    cfg = gen.CONFIGS[key]
    return gen.make_shared_expert(cfg)


@functools.lru_cache(maxsize=2)
def _device_shared(key: str):
    return {k: dev(v) for k, v in _host_shared(key).items()}


def seeded_layer(key: str, T: int) -> Layer:
    return Layer(key, T)
