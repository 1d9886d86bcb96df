"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function takes a loaded oracle library (the real one, or a
deliberately broken copy built by the mutation test) and raises
AssertionError when the oracle disagrees with the pin.  The pins use:
brute force on tiny inputs, exhaustive tie patterns, values the pages print,
hand-worked examples (``tests/golden``), closed forms, numpy/scipy library
routines, and whole-layer invariants.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
from scipy.special import erf, softmax

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def _brute_top2(l):
    """O(E^2) brute force: an expert's rank is the number of experts that beat
    it under (logit descending, index ascending); NaN ranks below numbers."""
    E = len(l)

    def beats(a, b):
        la, lb = l[a], l[b]
        if math.isnan(la) != math.isnan(lb):
            return math.isnan(lb)
        if not math.isnan(la) and la != lb:
            return la > lb
        return a < b

    rank = [sum(1 for o in range(E) if o != e and beats(o, e)) for e in range(E)]
    return rank.index(0), rank.index(1)


def _read_kv(path):
    d = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            d[k] = [float(x) for x in v]
    return d


def _np_ffn(x, w1, b1, w2, b2, act, w3=None):
    """fp64 two-layer FFN via numpy matmul (library routine)."""
    u = x @ w1
    if act == "swiglu":
        v = x @ w3
        H = (u / (1.0 + np.exp(-u))) * v
    else:
        z = u + (b1 if b1 is not None else 0.0)
        H = np.maximum(z, 0.0) if act == "relu" else 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))
    y = H @ w2
    if act != "swiglu" and b2 is not None:
        y = y + b2
    return y


def _rand_f32(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


# ----------------------------------------------------------------- top-2
def pin_top2_bruteforce(lib):
    rng = np.random.default_rng(1)
    for E in (2, 3, 4, 5, 8, 16, 33, 64):
        # few distinct values -> many ties; plus continuous values
        for lg in (rng.integers(-2, 3, size=(200, E)).astype(np.float64), rng.standard_normal((200, E))):
            idx = oracle.top2(lg, lib=lib)
            for t in range(lg.shape[0]):
                assert tuple(idx[t]) == _brute_top2(list(lg[t])), (E, lg[t], idx[t])


def pin_top2_exhaustive_ties(lib):
    for E in range(2, 7):
        lg = np.array(list(itertools.product((0.0, 1.0, 2.0), repeat=E)))
        idx = oracle.top2(lg, lib=lib)
        for t in range(lg.shape[0]):
            assert tuple(idx[t]) == _brute_top2(list(lg[t])), (lg[t], idx[t])


def pin_top2_special_cases(lib):
    # all-equal logits (e.g. an all-zero padding token): lowest indices win
    for E in (2, 4, 16, 64):
        idx = oracle.top2(np.zeros((1, E)), lib=lib)
        assert tuple(idx[0]) == (0, 1)
        g = oracle.gates(np.zeros((1, E)), idx, lib=lib)
        assert g[0, 0] == 0.5 and g[0, 1] == 0.5
    # NaN ranks below every number, -inf included
    idx = oracle.top2(np.array([[np.nan, 1.0, 0.0]]), lib=lib)
    assert tuple(idx[0]) == (1, 2)
    idx = oracle.top2(np.array([[np.nan, -np.inf, np.nan]]), lib=lib)
    assert tuple(idx[0]) == (1, 0)
    # slot 0 holds the larger logit
    idx = oracle.top2(np.array([[0.0, 3.0, 1.0, 2.0]]), lib=lib)
    assert tuple(idx[0]) == (1, 3)


# ----------------------------------------------------------------- gates
def pin_gates_closed_form(lib):
    rng = np.random.default_rng(2)
    for E in (2, 3, 8, 16, 64):
        lg = rng.standard_normal((300, E)) * 3
        idx = oracle.top2(lg, lib=lib)
        g = oracle.gates(lg, idx, lib=lib)
        l0 = lg[np.arange(300), idx[:, 0]]
        l1 = lg[np.arange(300), idx[:, 1]]
        g0 = 1.0 / (1.0 + np.exp(l1 - l0))  # logistic of the logit gap
        np.testing.assert_allclose(g[:, 0], g0, rtol=1e-13)
        np.testing.assert_allclose(g[:, 1], 1.0 - g0, rtol=1e-12, atol=1e-15)
        assert np.all(np.abs(g.sum(1) - 1.0) < 1e-14)
        assert np.all(g[:, 0] >= 0.5)


def pin_gates_two_way_softmax(lib):
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((100, 2)) * 2
    idx = oracle.top2(lg, lib=lib)
    g = oracle.gates(lg, idx, lib=lib)
    p = softmax(lg, axis=1)  # scipy library softmax
    np.testing.assert_allclose(g[:, 0], p[np.arange(100), idx[:, 0]], rtol=1e-13)
    np.testing.assert_allclose(g[:, 1], p[np.arange(100), idx[:, 1]], rtol=1e-13)


def pin_gates_page_pairs(lib):
    with open(os.path.join(GOLDEN, "gate_pairs.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for E, e0, e1, w0, w1 in rows:
        E, e0, e1, w0, w1 = int(E), int(e0), int(e1), float(w0), float(w1)
        lg = np.full((1, E), -4.0)
        lg[0, e1] = 0.0
        lg[0, e0] = math.log(w0 / w1)
        idx = oracle.top2(lg, lib=lib)
        assert tuple(idx[0]) == (e0, e1)
        g = oracle.gates(lg, idx, lib=lib)
        np.testing.assert_allclose(g[0], [w0, w1], rtol=1e-12)


# ----------------------------------------------------------------- dispatch
def pin_dispatch_hand_example(lib):
    kv = _read_kv(os.path.join(GOLDEN, "dispatch_hand_example.txt"))
    T, E = int(kv["T"][0]), int(kv["E"][0])
    idx = np.array(kv["idx"], np.int32).reshape(T, 2)
    r = oracle.dispatch(idx, E, lib=lib)
    for k in ("counts", "offsets", "sorted_assign", "assign_pos"):
        assert r[k].tolist() == [int(v) for v in kv[k]], (k, r[k])


def check_dispatch_against_library(idx, E, r):
    """Counts, offsets, permutation and inverse against numpy's stable sort."""
    flat = np.asarray(idx).reshape(-1)
    A = flat.size
    assert r["counts"].tolist() == np.bincount(flat, minlength=E).tolist()
    assert r["offsets"][0] == 0 and r["offsets"][-1] == A
    assert np.all(np.diff(r["offsets"]) == r["counts"])
    order = np.argsort(flat, kind="stable")  # library stable sort
    assert np.array_equal(r["sorted_assign"], order)
    inv = np.empty(A, np.int64)
    inv[order] = np.arange(A)
    assert np.array_equal(r["assign_pos"], inv)


def pin_dispatch_library_sort(lib):
    rng = np.random.default_rng(4)
    cases = []
    for E in (2, 3, 8, 16, 64):
        for T in (1, 2, 7, 64, 1000):
            # two distinct experts per token
            a = rng.integers(0, E, size=T)
            b = (a + rng.integers(1, E, size=T)) % E
            cases.append((np.stack([a, b], 1), E))
    # degenerate: every token picks the same pair; experts left empty
    cases.append((np.tile([[5, 2]], (300, 1)), 8))
    cases.append((np.tile([[0, 63]], (17, 1)), 64))
    for idx, E in cases:
        r = oracle.dispatch(idx, E, lib=lib)
        check_dispatch_against_library(idx, E, r)


# ----------------------------------------------------------------- expert FFN
def pin_ffn_hand_example(lib):
    kv = _read_kv(os.path.join(GOLDEN, "ffn_hand_example.txt"))
    f = lambda k, s: np.array(kv[k], np.float32).reshape(s)
    x, w1, b1, w2, b2 = f("x", (1, 2)), f("w1", (1, 2, 2)), f("b1", (1, 2)), f("w2", (1, 2, 2)), f("b2", (1, 2))
    for mirror in (False, True):
        y = oracle.ffn_rows(x, [0], [0], w1, w2, "relu", b1=b1, b2=b2, mirror=mirror, lib=lib)
        assert y[0].tolist() == kv["y"], y


def pin_ffn_library_matmul(lib):
    rng = np.random.default_rng(5)
    d, h, E = 48, 80, 3
    x = _rand_f32(rng, (4, d))
    for act in ("relu", "gelu", "swiglu"):
        w1 = _rand_f32(rng, (E, d, h), 1 / math.sqrt(d))
        w3 = _rand_f32(rng, (E, d, h), 1 / math.sqrt(d)) if act == "swiglu" else None
        w2 = _rand_f32(rng, (E, h, d), 1 / math.sqrt(h))
        b1 = _rand_f32(rng, (E, h), 0.1) if act != "swiglu" else None
        b2 = _rand_f32(rng, (E, d), 0.1) if act != "swiglu" else None
        rows_t = np.array([0, 1, 2, 3, 1], np.int32)
        rows_e = np.array([0, 2, 1, 1, 0], np.int32)
        y = oracle.ffn_rows(x, rows_t, rows_e, w1, w2, act, w3=w3, b1=b1, b2=b2, mirror=False, lib=lib)
        for r, (t, e) in enumerate(zip(rows_t, rows_e)):
            ref = _np_ffn(x[t].astype(np.float64), w1[e].astype(np.float64),
                          None if b1 is None else b1[e].astype(np.float64), w2[e].astype(np.float64),
                          None if b2 is None else b2[e].astype(np.float64), act,
                          None if w3 is None else w3[e].astype(np.float64))
            np.testing.assert_allclose(y[r], ref, rtol=1e-11, atol=1e-13)


def pin_ffn_activation_values(lib):
    # d = h = 1, W1 = W2 = 1, no biases: y = act(x).  Textbook values:
    # GELU(z) = z * Phi(z) with Phi(1) = 0.8413447460685429, Phi(-1) = 1 - Phi(1);
    # SiLU with W3 = 1: y = z / (1 + e^-z), 1 / (1 + e^-1) = 0.7310585786300049.
    one = np.ones((1, 1, 1), np.float32)
    xs = np.array([[1.0], [-1.0], [0.0], [-30.0], [30.0]], np.float32)
    rt = np.arange(5, dtype=np.int32)
    re = np.zeros(5, np.int32)
    g = oracle.ffn_rows(xs, rt, re, one, one, "gelu", mirror=False, lib=lib)[:, 0]
    np.testing.assert_allclose(g[:3], [0.8413447460685429, -(1 - 0.8413447460685429), 0.0], rtol=1e-14, atol=1e-16)
    assert abs(g[3]) < 1e-150 and g[4] == 30.0
    r = oracle.ffn_rows(xs, rt, re, one, one, "relu", mirror=False, lib=lib)[:, 0]
    assert r.tolist() == [1.0, 0.0, 0.0, 0.0, 30.0]
    s = oracle.ffn_rows(xs, rt, re, one, one, "swiglu", w3=one, mirror=False, lib=lib)[:, 0]
    # y = silu(z) * z
    np.testing.assert_allclose(s[:2], [0.7310585786300049, 1 - 0.7310585786300049], rtol=1e-14)
    assert s[2] == 0.0


def pin_ffn_small_integer_mirror(lib):
    """bf16 "mirror" rounding: with small-integer operands every product and sum
    is an exact integer, so the only rounding is H -> bf16 and y -> bf16.  The
    reference rounds with the generator's own fp32 -> bf16 routine."""
    rng = np.random.default_rng(6)
    d, h, E, T = 64, 128, 2, 6
    ints = lambda s: rng.integers(-8, 9, size=s)
    x, w1, w2 = ints((T, d)), ints((E, d, h)), ints((E, h, d))
    b1, b2 = ints((E, h)), ints((E, d))
    bf = lambda a: gen.f32_to_bf16_bits(np.asarray(a, np.float32))
    rt = np.arange(T, dtype=np.int32)
    re = (np.arange(T) % E).astype(np.int32)
    y = oracle.ffn_rows(bf(x), rt, re, bf(w1), bf(w2), "relu", b1=bf(b1), b2=bf(b2), mirror=True, lib=lib)
    for r in range(T):
        e = re[r]
        u = x[r] @ w1[e] + b1[e]                     # exact int64
        H = gen.bf16_bits_to_f32(bf(np.maximum(u, 0))).astype(np.int64)
        yy = H @ w2[e] + b2[e]                         # exact int64, |yy| < 2^24
        assert np.abs(yy).max() < 2 ** 24
        ref = gen.bf16_bits_to_f32(bf(yy)).astype(np.float64)
        assert np.array_equal(y[r], ref), r
    # the rounding must matter here (otherwise the pin would not see it)
    u_all = np.einsum("td,tdh->th", x, w1[re]) + b1[re]
    assert np.any(np.abs(u_all) > 256)


def pin_rounding(lib):
    # direct fp64 -> bf16 RNE, ties to even, no double rounding via fp32
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8), 2.0 ** -130, 3.5e38])
    got = oracle.round_to(vals, oracle.DT_BF16, lib=lib)
    assert got[0] == 1.0 and got[1] == 1 + 2 ** -6 and got[2] == 1 + 2 ** -7 and got[3] == -1.0
    assert got[4] == 2.0 ** -130 and np.isinf(got[5])
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(10000) * 10.0 ** rng.integers(-30, 30, 10000)).astype(np.float32)
    got = oracle.round_to(f.astype(np.float64), oracle.DT_BF16, lib=lib)
    ref = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(f)).astype(np.float64)
    assert np.array_equal(got, ref)
    got32 = oracle.round_to(np.array([1 + 2 ** -24, 1 + 2 ** -23 + 2 ** -24, 0.1]), oracle.DT_F32, lib=lib)
    assert got32.tolist() == [1.0, 1 + 2 ** -22, float(np.float32(0.1))]


# ----------------------------------------------------------------- router logits
def pin_logits_library(lib):
    rng = np.random.default_rng(8)
    for dt in (gen.F32, gen.BF16):
        x = _rand_f32(rng, (9, 96))
        w = _rand_f32(rng, (96, 7), 0.1)
        b = _rand_f32(rng, (7,), 0.5)
        if dt == gen.BF16:
            x, w = gen.f32_to_bf16_bits(x), gen.f32_to_bf16_bits(w)
            xf, wf = gen.bf16_bits_to_f32(x), gen.bf16_bits_to_f32(w)
        else:
            xf, wf = x, w
        lg = oracle.logits(x, w, b, lib=lib)
        np.testing.assert_allclose(lg, xf.astype(np.float64) @ wf.astype(np.float64) + b, rtol=1e-12, atol=1e-13)
        lg0 = oracle.logits(x, w, None, lib=lib)
        np.testing.assert_allclose(lg0, xf.astype(np.float64) @ wf.astype(np.float64), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- combine
def pin_combine_indexing(lib):
    # y_sorted row p holds the value p in every column; out[t] must be
    # g0 * assign_pos[2t] + g1 * assign_pos[2t+1]
    rng = np.random.default_rng(9)
    T, d = 50, 3
    ap = rng.permutation(2 * T).astype(np.int32)
    g = rng.random((T, 2))
    y = np.repeat(np.arange(2 * T, dtype=np.float64)[:, None], d, 1)
    out = oracle.combine(y, ap, g, oracle.DT_F32, lib=lib)
    ref = g[:, 0] * ap[0::2] + g[:, 1] * ap[1::2]
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-7)


# ----------------------------------------------------------------- whole layer
def _small_layer(rng, act, E=6, d=32, h=48, T=40, dt=gen.F32):
    w = {
        "x": _rand_f32(rng, (T, d)), "w_r": _rand_f32(rng, (d, E), 1 / math.sqrt(d)),
        "b_r": _rand_f32(rng, (E,), 0.3),
        "w1": _rand_f32(rng, (E, d, h), 1 / math.sqrt(d)), "w2": _rand_f32(rng, (E, h, d), 1 / math.sqrt(h)),
        "w3": _rand_f32(rng, (E, d, h), 1 / math.sqrt(d)) if act == "swiglu" else None,
        "b1": _rand_f32(rng, (E, h), 0.1) if act != "swiglu" else None,
        "b2": _rand_f32(rng, (E, d), 0.1) if act != "swiglu" else None,
    }
    if dt == gen.BF16:
        w = {k: (None if v is None else (v if k == "b_r" else gen.f32_to_bf16_bits(v))) for k, v in w.items()}
    return w


def _run_layer(w, act, lib, mirror=False):
    return oracle.layer(w["x"], w["w_r"], w["w1"], w["w2"], act, b_r=w["b_r"], w3=w["w3"], b1=w["b1"],
                        b2=w["b2"], mirror=mirror, lib=lib)


def pin_layer_invariants(lib):
    rng = np.random.default_rng(10)
    for act in ("relu", "gelu", "swiglu"):
        w = _small_layer(rng, act)
        r = _run_layer(w, act, lib)
        T = w["x"].shape[0]
        assert np.all(np.abs(r["gate"].sum(1) - 1.0) < 1e-14)
        assert r["counts"].sum() == 2 * T
        check_dispatch_against_library(r["idx"], w["w_r"].shape[1], r)
        # permuting the tokens permutes the outputs (and nothing else changes)
        perm = rng.permutation(T)
        w2 = dict(w)
        w2["x"] = w["x"][perm]
        r2 = _run_layer(w2, act, lib)
        assert np.array_equal(r2["out"], r["out"][perm])
        assert np.array_equal(r2["idx"], r["idx"][perm])
        assert np.array_equal(r2["counts"], r["counts"])


def pin_layer_identical_experts_dense(lib):
    rng = np.random.default_rng(11)
    for act in ("relu", "gelu", "swiglu"):
        w = _small_layer(rng, act)
        E = w["w1"].shape[0]
        for k in ("w1", "w2", "w3", "b1", "b2"):
            if w[k] is not None:
                w[k] = np.ascontiguousarray(np.repeat(w[k][:1], E, 0))
        r = _run_layer(w, act, lib)
        f64 = lambda a: None if a is None else a[0].astype(np.float64)
        dense = _np_ffn(w["x"].astype(np.float64), f64(w["w1"]), f64(w["b1"]), f64(w["w2"]), f64(w["b2"]), act,
                        f64(w["w3"]))
        ref = oracle.round_to(dense, oracle.DT_F32, lib=lib)
        np.testing.assert_allclose(r["out"], ref, rtol=1e-6, atol=1e-7)


def pin_layer_isolate_one_expert(lib):
    rng = np.random.default_rng(12)
    act = "gelu"
    w = _small_layer(rng, act)
    E = w["w1"].shape[0]
    keep = 3
    for k in ("w2", "b2"):
        z = np.zeros_like(w[k])
        z[keep] = w[k][keep]
        w[k] = z
    r = _run_layer(w, act, lib)
    f64 = lambda a: a[keep].astype(np.float64)
    y = _np_ffn(w["x"].astype(np.float64), f64(w["w1"]), f64(w["b1"]), f64(w["w2"]), f64(w["b2"]), act)
    for t in range(w["x"].shape[0]):
        g = sum(r["gate"][t, s] for s in range(2) if r["idx"][t, s] == keep)
        np.testing.assert_allclose(r["out"][t], g * y[t], rtol=1e-6, atol=1e-7)
    assert np.any(r["idx"] == keep) and np.any(np.all(r["idx"] != keep, axis=1))


def pin_layer_zero_padding(lib):
    rng = np.random.default_rng(13)
    for act in ("relu", "gelu", "swiglu"):
        w = _small_layer(rng, act, d=32, h=48)
        r = _run_layer(w, act, lib)
        pd, ph = 16, 24
        p = dict(w)
        p["x"] = np.pad(w["x"], ((0, 0), (0, pd)))
        p["w_r"] = np.pad(w["w_r"], ((0, pd), (0, 0)))
        p["w1"] = np.pad(w["w1"], ((0, 0), (0, pd), (0, ph)))
        if w["w3"] is not None:
            p["w3"] = np.pad(w["w3"], ((0, 0), (0, pd), (0, ph)))
        p["w2"] = np.pad(w["w2"], ((0, 0), (0, ph), (0, pd)))
        if w["b1"] is not None:
            p["b1"] = np.pad(w["b1"], ((0, 0), (0, ph)))
            p["b2"] = np.pad(w["b2"], ((0, 0), (0, pd)))
        rp = _run_layer(p, act, lib)
        assert np.array_equal(rp["idx"], r["idx"])
        np.testing.assert_allclose(rp["out"][:, :32], r["out"], rtol=1e-12, atol=1e-14)
        assert np.all(rp["out"][:, 32:] == 0.0)


# ----------------------------------------------------------------- int8 expert weights
def pin_q8_quantize_hand_example(lib):
    kv = _read_kv(os.path.join(GOLDEN, "q8_quantize_hand_example.txt"))
    w = np.stack([np.array(kv[f"col{c}_w"], np.float32) for c in range(4)], axis=1)[None]  # [1, 8, 4]
    for dt_w in (w, gen.f32_to_bf16_bits(w)):  # the values are bf16-exact too
        q, sc = oracle.quantize_q8(dt_w, lib=lib)
        for c in range(4):
            assert q[0, :, c].tolist() == [int(v) for v in kv[f"col{c}_q"]], (c, q[0, :, c])
            assert sc[0, c] == np.float32(kv[f"col{c}_s"][0]), (c, sc[0, c])


def pin_q8_ffn_hand_example(lib):
    kv = _read_kv(os.path.join(GOLDEN, "q8_ffn_hand_example.txt"))
    f = lambda k, s, t=np.float32: np.array(kv[k], t).reshape(s)
    x, b1, b2 = f("x", (1, 2)), f("b1", (1, 2)), f("b2", (1, 2))
    q1, q2 = f("q1", (1, 2, 2), np.int8), f("q2", (1, 2, 2), np.int8)
    s1, s2 = f("s1", (1, 2)), f("s2", (1, 2))
    for mirror in (False, True):
        y = oracle.ffn_rows_q8(x, [0], [0], q1, s1, q2, s2, "relu", b1=b1, b2=b2, mirror=mirror, lib=lib)
        assert y[0].tolist() == kv["y"], y


def pin_q8_ffn_unit_scales(lib):
    """With every scale 1 the int8 path is the plain FFN on the integer weights."""
    rng = np.random.default_rng(21)
    d, h, E = 32, 48, 3
    x = _rand_f32(rng, (5, d))
    rows_t = np.array([0, 1, 2, 3, 4, 0], np.int32)
    rows_e = np.array([0, 2, 1, 1, 0, 2], np.int32)
    for act in ("relu", "gelu", "swiglu"):
        q1, q3 = rng.integers(-127, 128, (E, d, h)), rng.integers(-127, 128, (E, d, h))
        q2 = rng.integers(-127, 128, (E, h, d))
        ones_h, ones_d = np.ones((E, h), np.float32), np.ones((E, d), np.float32)
        b1 = _rand_f32(rng, (E, h)) if act != "swiglu" else None
        b2 = _rand_f32(rng, (E, d)) if act != "swiglu" else None
        sw = act == "swiglu"
        y = oracle.ffn_rows_q8(x, rows_t, rows_e, q1, ones_h, q2, ones_d, act, q3=q3 if sw else None,
                               s3=ones_h if sw else None, b1=b1, b2=b2, mirror=False, lib=lib)
        ref = oracle.ffn_rows(x, rows_t, rows_e, q1.astype(np.float32), q2.astype(np.float32), act,
                              w3=q3.astype(np.float32) if sw else None, b1=b1, b2=b2, mirror=False, lib=lib)
        assert np.array_equal(y, ref), act


def pin_q8_ffn_library(lib):
    """Random codes and scales against numpy matmuls on s[None, :] * q (fp64)."""
    rng = np.random.default_rng(22)
    d, h, E = 40, 56, 2
    x = _rand_f32(rng, (3, d))
    for act in ("relu", "gelu", "swiglu"):
        q1, q3, q2 = (rng.integers(-127, 128, s).astype(np.int8) for s in ((E, d, h), (E, d, h), (E, h, d)))
        s1, s3 = (rng.uniform(0.5, 2.0, (E, h)).astype(np.float32) / 127 for _ in range(2))
        s2 = rng.uniform(0.5, 2.0, (E, d)).astype(np.float32) / 127
        b1 = _rand_f32(rng, (E, h), 0.1) if act != "swiglu" else None
        b2 = _rand_f32(rng, (E, d), 0.1) if act != "swiglu" else None
        sw = act == "swiglu"
        rows_t = np.array([0, 1, 2, 1], np.int32)
        rows_e = np.array([1, 0, 1, 1], np.int32)
        y = oracle.ffn_rows_q8(x, rows_t, rows_e, q1, s1, q2, s2, act, q3=q3 if sw else None,
                               s3=s3 if sw else None, b1=b1, b2=b2, mirror=False, lib=lib)
        deq = lambda q, s: q.astype(np.float64) * s.astype(np.float64)[None, :]
        for r, (t, e) in enumerate(zip(rows_t, rows_e)):
            ref = _np_ffn(x[t].astype(np.float64), deq(q1[e], s1[e]),
                          None if b1 is None else b1[e].astype(np.float64), deq(q2[e], s2[e]),
                          None if b2 is None else b2[e].astype(np.float64), act,
                          deq(q3[e], s3[e]) if sw else None)
            np.testing.assert_allclose(y[r], ref, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------- 4-bit expert weights
def pin_q4_quantize_hand_example(lib):
    kv = _read_kv(os.path.join(GOLDEN, "q4_quantize_hand_example.txt"))
    cols = []
    for c in range(4):
        col = np.full(128, kv[f"col{c}_rest"][0], np.float32)
        col[:8] = kv[f"col{c}_head"]
        cols.append(col)
    w = np.stack(cols, axis=1)[None]  # [1, 128, 4]
    for dt_w in (w, gen.f32_to_bf16_bits(w)):  # the values are bf16-exact too
        q, sc, z = oracle.quantize_q4(dt_w, lib=lib)
        for c in range(4):
            want = [int(v) for v in kv[f"col{c}_q"]] + [int(kv[f"col{c}_qrest"][0])] * 120
            assert q[0, :, c].tolist() == want, (c, q[0, :8, c])
            assert sc[0, 0, c] == np.float32(kv[f"col{c}_s"][0]), (c, sc[0, 0, c])
            assert z[0, 0, c] == int(kv[f"col{c}_z"][0]), (c, z[0, 0, c])


def pin_q4_quantize_bounds(lib):
    """Random groups: codes and zero points in [0, 15]; a code that was not
    clamped stands for a weight within s/2 of w, and the group's smallest
    weight gets code 0 whenever its zero point was not clamped; codes are
    monotone in w inside a group; a group is 128 consecutive k of one column
    (changing one weight moves only that group's scale)."""
    rng = np.random.default_rng(31)
    E, K, N = 2, 384, 24
    w = (rng.standard_normal((E, K, N)) * rng.uniform(0.01, 3.0, (E, 1, N))).astype(np.float32)
    w[0, 128:256, 3] += 5.0  # an all-positive group: its zero point clamps to 0
    q, sc, z = oracle.quantize_q4(w, lib=lib)
    assert q.min() >= 0 and q.max() <= 15 and z.min() >= 0 and z.max() <= 15
    s_full = np.repeat(sc, 128, axis=1).astype(np.float64)
    z_full = np.repeat(z, 128, axis=1).astype(np.float64)
    deq = s_full * (q.astype(np.float64) - z_full)
    raw = np.rint((w / np.repeat(sc, 128, axis=1)).astype(np.float32)).astype(np.float64) + z_full
    unclamped = (raw >= 0) & (raw <= 15)
    assert unclamped.mean() > 0.95
    err = np.abs(deq - w.astype(np.float64))
    assert np.all(err[unclamped] <= s_full[unclamped] * (0.5 + 1e-5)), err[unclamped].max()
    g = w.reshape(E, K // 128, 128, N)
    gq = q.reshape(E, K // 128, 128, N)
    zmn = -np.rint((g.min(axis=2) / sc).astype(np.float32))
    for e in range(E):
        for gi in range(K // 128):
            for n in range(N):
                col, cq = g[e, gi, :, n], gq[e, gi, :, n]
                o = np.argsort(col, kind="stable")
                assert np.all(np.diff(cq[o].astype(int)) >= 0), (e, gi, n)
                if 0 <= zmn[e, gi, n] <= 15:
                    assert cq[o[0]] == 0, (e, gi, n)
    assert z[0, 1, 3] == 0
    w2 = w.copy()
    w2[1, 200, 7] = 40.0
    _, sc2, _ = oracle.quantize_q4(w2, lib=lib)
    changed = np.argwhere(sc2 != sc)
    assert changed.tolist() == [[1, 1, 7]], changed


def pin_q4_ffn_library(lib):
    """Random codes, scales and zero points against numpy matmuls on
    s * (q - z) (fp64), groups of 128 along the input channels."""
    rng = np.random.default_rng(32)
    d, h, E = 256, 384, 2
    x = _rand_f32(rng, (3, d))
    for act in ("relu", "gelu", "swiglu"):
        def mk(K, N):
            return (rng.integers(0, 16, (E, K, N)).astype(np.uint8),
                    (rng.uniform(0.5, 2.0, (E, K // 128, N)) / 15 / np.sqrt(K)).astype(np.float32),
                    rng.integers(0, 16, (E, K // 128, N)).astype(np.uint8))
        w1q, w3q, w2q = mk(d, h), mk(d, h), mk(h, d)
        b1 = _rand_f32(rng, (E, h), 0.1) if act != "swiglu" else None
        b2 = _rand_f32(rng, (E, d), 0.1) if act != "swiglu" else None
        sw = act == "swiglu"
        rows_t = np.array([0, 1, 2, 1], np.int32)
        rows_e = np.array([1, 0, 1, 1], np.int32)
        y = oracle.ffn_rows_q4(x, rows_t, rows_e, w1q, w2q, act, w3q=w3q if sw else None, b1=b1, b2=b2,
                               mirror=False, lib=lib)
        deq = lambda t, e: (np.repeat(t[1][e], 128, axis=0).astype(np.float64) *
                            (t[0][e].astype(np.float64) - np.repeat(t[2][e], 128, axis=0).astype(np.float64)))
        for r, (t, e) in enumerate(zip(rows_t, rows_e)):
            ref = _np_ffn(x[t].astype(np.float64), deq(w1q, e), None if b1 is None else b1[e].astype(np.float64),
                          deq(w2q, e), None if b2 is None else b2[e].astype(np.float64), act,
                          deq(w3q, e) if sw else None)
            np.testing.assert_allclose(y[r], ref, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------- gating variants, shared expert, residual
def pin_gate_modes_hand_example(lib):
    kv = _read_kv(os.path.join(GOLDEN, "gate_modes_hand_example.txt"))
    for case in ("a", "b"):
        lg = np.log(np.array([kv[f"{case}_p"]]))
        idx = oracle.top2(lg, lib=lib)
        assert idx[0].tolist() == [int(v) for v in kv[f"{case}_idx"]], (case, idx)
        for mode in ("softmax", "pair"):
            g = oracle.gates(lg, idx, mode=mode, lib=lib)
            np.testing.assert_allclose(g[0], kv[f"{case}_{mode}"], rtol=1e-14, err_msg=f"{case} {mode}")
        g = oracle.gates(lg, idx, mode="linear", lib=lib)
        assert g[0].tolist() == lg[0, idx[0]].tolist()


def pin_gates_softmax_all_library(lib):
    """Softmax over all experts (scipy), read at the chosen pair, unnormalised."""
    rng = np.random.default_rng(31)
    for E in (2, 3, 8, 16, 60, 64):
        lg = rng.standard_normal((200, E)) * 3
        idx = oracle.top2(lg, lib=lib)
        g = oracle.gates(lg, idx, mode="softmax", lib=lib)
        p = softmax(lg, axis=1)
        rows = np.arange(200)
        np.testing.assert_allclose(g[:, 0], p[rows, idx[:, 0]], rtol=1e-13)
        np.testing.assert_allclose(g[:, 1], p[rows, idx[:, 1]], rtol=1e-13)
        # the pair keeps the ratio of the pair softmax; with two experts the modes agree
        gp = oracle.gates(lg, idx, lib=lib)
        np.testing.assert_allclose(g[:, 0] / g.sum(1), gp[:, 0], rtol=1e-13)
        if E == 2:
            np.testing.assert_allclose(g, gp, rtol=1e-14)
        else:
            assert np.all(g.sum(1) < 1.0)


def pin_gates_linear_are_logits(lib):
    rng = np.random.default_rng(32)
    for E in (2, 5, 64):
        lg = rng.standard_normal((100, E)) * 4
        idx = oracle.top2(lg, lib=lib)
        g = oracle.gates(lg, idx, mode="linear", lib=lib)
        rows = np.arange(100)
        assert np.array_equal(g[:, 0], lg[rows, idx[:, 0]])
        assert np.array_equal(g[:, 1], lg[rows, idx[:, 1]])


def pin_combine_addends_hand_example(lib):
    kv = _read_kv(os.path.join(GOLDEN, "combine_addends_hand_example.txt"))
    y = np.array([kv["y0"], kv["y1"]])
    ap = np.array([0, 1], np.int32)
    g = np.array([kv["g"]])
    sh = np.array([kv["shared"]])
    res = np.array([kv["residual"]], np.float32)
    for dt, cast in ((oracle.DT_F32, lambda a: a), (oracle.DT_BF16, gen.f32_to_bf16_bits)):
        out = oracle.combine(y, ap, g, dt, shared_y=sh, residual=cast(res), lib=lib)
        assert out[0].tolist() == kv["out"], out
        assert oracle.combine(y, ap, g, dt, lib=lib)[0].tolist() == kv["out_plain"]
        assert oracle.combine(y, ap, g, dt, shared_y=sh, lib=lib)[0].tolist() == kv["out_shared_only"]


def pin_combine_addends_indexing(lib):
    """Addend rows follow the token: row t of shared_y / residual holds t and
    10 t in every column."""
    rng = np.random.default_rng(33)
    T, d = 30, 4
    ap = rng.permutation(2 * T).astype(np.int32)
    g = rng.random((T, 2))
    y = np.repeat(np.arange(2 * T, dtype=np.float64)[:, None], d, 1)
    sh = np.repeat(np.arange(T, dtype=np.float64)[:, None], d, 1)
    res = np.repeat((10 * np.arange(T, dtype=np.float32))[:, None], d, 1)
    out = oracle.combine(y, ap, g, oracle.DT_F32, shared_y=sh, residual=res, lib=lib)
    ref = g[:, 0] * ap[0::2] + g[:, 1] * ap[1::2] + 11 * np.arange(T)
    for c in range(d):
        np.testing.assert_allclose(out[:, c], ref, rtol=1e-7)


def _shared_expert(rng, act, d, h):
    return {
        "w1": _rand_f32(rng, (1, d, h), 1 / math.sqrt(d)), "w2": _rand_f32(rng, (1, h, d), 1 / math.sqrt(h)),
        "w3": _rand_f32(rng, (1, d, h), 1 / math.sqrt(d)) if act == "swiglu" else None,
        "b1": _rand_f32(rng, (1, h), 0.1) if act != "swiglu" else None,
        "b2": _rand_f32(rng, (1, d), 0.1) if act != "swiglu" else None,
    }


def pin_layer_shared_expert_library(lib):
    """The shared expert is a dense FFN over every token (numpy matmuls), added
    with weight one beside the routed pair and the residual."""
    rng = np.random.default_rng(34)
    for act in ("relu", "gelu", "swiglu"):
        w = _small_layer(rng, act)
        T, d = w["x"].shape
        sh = _shared_expert(rng, act, d, 80)
        res = _rand_f32(rng, (T, d))
        tokens = np.arange(T)
        for gate in ("pair", "softmax", "linear"):
            r = oracle.layer_tokens(w["x"], w["w_r"], w["w1"], w["w2"], act, tokens, b_r=w["b_r"], w3=w["w3"],
                                    b1=w["b1"], b2=w["b2"], mirror=False, gate=gate, shared=sh, residual=res,
                                    lib=lib)
            x64 = w["x"].astype(np.float64)
            f = lambda k: None if sh[k] is None else sh[k][0].astype(np.float64)
            ysh = _np_ffn(x64, f("w1"), f("b1"), f("w2"), f("b2"), act, f("w3"))
            np.testing.assert_allclose(r["y_shared"], ysh, rtol=1e-11, atol=1e-13)
            routed = r["gate"][:, :1] * r["y"][:, 0] + r["gate"][:, 1:] * r["y"][:, 1]
            ref = routed + ysh + res.astype(np.float64)
            np.testing.assert_allclose(r["out"], ref, rtol=3e-7, atol=1e-6)


def pin_layer_zero_addends_are_plain(lib):
    """A shared expert of zero weights and a zero residual leave the layer as it was."""
    rng = np.random.default_rng(35)
    for act in ("relu", "swiglu"):
        for dt in (gen.F32, gen.BF16):
            w = _small_layer(rng, act, dt=dt)
            T, d = w["x"].shape
            zero = lambda shape: np.zeros(shape, w["x"].dtype)
            sh = {"w1": zero((1, d, 64)), "w2": zero((1, 64, d)), "w3": zero((1, d, 64)) if act == "swiglu" else None}
            tokens = np.arange(T)
            kw = dict(b_r=w["b_r"], w3=w["w3"], b1=w["b1"], b2=w["b2"], mirror=True, lib=lib)
            base = oracle.layer_tokens(w["x"], w["w_r"], w["w1"], w["w2"], act, tokens, **kw)
            ex = oracle.layer_tokens(w["x"], w["w_r"], w["w1"], w["w2"], act, tokens, shared=sh,
                                     residual=zero((T, d)), **kw)
            assert np.array_equal(base["out"], ex["out"])
            full = oracle.layer(w["x"], w["w_r"], w["w1"], w["w2"], act, **kw)
            assert np.array_equal(full["out"], base["out"])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
