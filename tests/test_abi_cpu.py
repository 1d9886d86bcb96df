"""C-ABI library: loads, exports what the header declares, and rejects bad
calls on the host before launching anything (CPU only: no call here reaches a
kernel launch)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_12_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "colibri_moe.h")

A16 = 0x7F0000100000  # fake, 256-byte aligned device addresses (never dereferenced)


def fake(i):
    return A16 + i * 0x100000


@pytest.fixture(scope="module")
def lib():
    return moe.load(build_if_missing=True)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(colibri_moe_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(moe.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert moe.status_string(code) != "unknown status"
    assert moe.status_string(-99) == "unknown status"


GOOD = moe.Shape(T=16, d=128, h=256, E=8, dtype=moe.BF16, act=moe.SWIGLU)


def shape_c(**kw):
    base = dict(T=GOOD.T, d=GOOD.d, h=GOOD.h, E=GOOD.E, k=2, dtype=GOOD.dtype, act=GOOD.act)
    base.update(kw)
    return moe._Shape(base["T"], base["d"], base["h"], base["E"], base["k"], base["dtype"], base["act"])


def route_call(lib, s, x=fake(0), w_r=fake(1), b_r=None, idx=fake(2), gate=fake(3), logits=None):
    return lib.colibri_moe_route(ctypes.byref(s), x, w_r, b_r, idx, gate, logits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=1), moe.COLIBRI_ERR_UNSUPPORTED), (dict(k=3), moe.COLIBRI_ERR_UNSUPPORTED),
    (dict(E=1), moe.COLIBRI_ERR_UNSUPPORTED), (dict(E=65), moe.COLIBRI_ERR_UNSUPPORTED),
    (dict(d=100), moe.COLIBRI_ERR_UNSUPPORTED), (dict(h=32), moe.COLIBRI_ERR_UNSUPPORTED),
    (dict(d=0), moe.COLIBRI_ERR_UNSUPPORTED), (dict(dtype=7), moe.COLIBRI_ERR_UNSUPPORTED),
    (dict(act=9), moe.COLIBRI_ERR_UNSUPPORTED), (dict(T=-1), moe.COLIBRI_ERR_INVALID_ARG),
    (dict(T=(1 << 28) + 1), moe.COLIBRI_ERR_UNSUPPORTED),
])
def test_shape_validation(lib, kw, code):
    s = shape_c(**kw)
    assert route_call(lib, s) == code
    assert lib.colibri_moe_workspace_size(ctypes.byref(s)) == 0


def test_empty_batch_is_a_no_op(lib):
    s = shape_c(T=0)
    # T = 0: success with no work, even with null pointers
    assert route_call(lib, s, x=None, w_r=None, idx=None, gate=None) == 0
    e = moe._Experts(None, None, None, None, None)
    assert lib.colibri_moe_layer_forward(ctypes.byref(s), None, None, None, ctypes.byref(e), None, None, None,
                                         None, None, 0, None) == 0
    assert lib.colibri_moe_workspace_size(ctypes.byref(s)) == 0


def test_route_pointer_checks(lib):
    s = shape_c()
    assert route_call(lib, s, x=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert route_call(lib, s, idx=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert route_call(lib, s, x=fake(0) + 8) == moe.COLIBRI_ERR_INVALID_ARG     # not 16-byte aligned
    assert route_call(lib, s, b_r=fake(5) + 2) == moe.COLIBRI_ERR_INVALID_ARG   # fp32 bias misaligned


def test_dispatch_checks(lib):
    s = shape_c()
    args = [fake(0), fake(1), fake(2), fake(3), fake(4)]
    for i in range(5):
        a = list(args)
        a[i] = None
        assert lib.colibri_moe_dispatch(ctypes.byref(s), *a, None, None, None, 0, None) == moe.COLIBRI_ERR_INVALID_ARG
    # x without x_sorted (or the reverse) is an error
    assert lib.colibri_moe_dispatch(ctypes.byref(s), *args, fake(6), None, None, 0, None) == moe.COLIBRI_ERR_INVALID_ARG
    assert lib.colibri_moe_dispatch(ctypes.byref(s), *args, None, fake(6), None, 0, None) == moe.COLIBRI_ERR_INVALID_ARG


def ffn_call(lib, s, e, ws_bytes=1 << 40, ws=fake(9), y=fake(8)):
    return lib.colibri_moe_expert_ffn(ctypes.byref(s), fake(0), fake(1), fake(2), ctypes.byref(e), y, ws,
                                      ws_bytes, None)


def test_ffn_checks(lib):
    s = shape_c()
    sw = moe._Experts(fake(10), fake(11), fake(12), None, None)
    # workspace too small
    assert ffn_call(lib, s, sw, ws_bytes=1024) == moe.COLIBRI_ERR_WORKSPACE
    # SwiGLU needs W3 and takes no biases
    assert ffn_call(lib, s, moe._Experts(fake(10), None, fake(12), None, None)) == moe.COLIBRI_ERR_INVALID_ARG
    assert ffn_call(lib, s, moe._Experts(fake(10), fake(11), fake(12), fake(13), None)) == moe.COLIBRI_ERR_UNSUPPORTED
    # ReLU / GELU take no W3
    sr = shape_c(act=moe.RELU)
    assert ffn_call(lib, sr, moe._Experts(fake(10), fake(11), fake(12), None, None)) == moe.COLIBRI_ERR_UNSUPPORTED
    # misaligned weights / output / workspace
    assert ffn_call(lib, s, moe._Experts(fake(10) + 4, fake(11), fake(12), None, None)) == moe.COLIBRI_ERR_INVALID_ARG
    assert ffn_call(lib, s, sw, y=fake(8) + 2) == moe.COLIBRI_ERR_INVALID_ARG
    assert ffn_call(lib, s, sw, ws=fake(9) + 16) == moe.COLIBRI_ERR_INVALID_ARG


def test_layer_checks(lib):
    s = shape_c()
    e = moe._Experts(fake(10), fake(11), fake(12), None, None)
    need = lib.colibri_moe_workspace_size(ctypes.byref(s))

    def call(ws=fake(20), ws_bytes=need, x=fake(0), out=fake(3)):
        return lib.colibri_moe_layer_forward(ctypes.byref(s), x, fake(1), None, ctypes.byref(e), out, None, None,
                                             None, ws, ws_bytes, None)

    assert call(ws_bytes=need - 1) == moe.COLIBRI_ERR_WORKSPACE
    assert call(ws=fake(20) + 128) == moe.COLIBRI_ERR_INVALID_ARG  # layer workspace must be 256-byte aligned
    assert call(x=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(out=fake(3) + 8) == moe.COLIBRI_ERR_INVALID_ARG


def test_workspace_size_covers_buffers(lib):
    for dt, el in ((moe.F32, 4), (moe.BF16, 2)):
        prev = 0
        for T in (1, 7, 64, 4096):
            s = shape_c(T=T, dtype=dt)
            ws = lib.colibri_moe_workspace_size(ctypes.byref(s))
            # at least H [2T, h] and Y [2T, d] plus the routing arrays
            assert ws >= 2 * T * (GOOD.h + GOOD.d) * el + 4 * (2 * T) * 4
            assert ws % 256 == 0 and ws > prev
            prev = ws


def test_ffn_layer_entry_point_checks(lib):
    s = shape_c()
    up = lambda e: lib.colibri_moe_expert_ffn_up(ctypes.byref(s), fake(0), fake(1), fake(2), ctypes.byref(e),
                                                 fake(3), None, 0, None)
    down = lambda e, sh=s: lib.colibri_moe_expert_ffn_down(ctypes.byref(sh), fake(0), fake(2), ctypes.byref(e),
                                                           fake(3), None, 0, None)
    # the first layer needs W1 (and W3 for SwiGLU), the second needs W2
    assert up(moe._Experts(None, fake(11), None, None, None)) == moe.COLIBRI_ERR_INVALID_ARG
    assert up(moe._Experts(fake(10), None, None, None, None)) == moe.COLIBRI_ERR_INVALID_ARG
    assert down(moe._Experts(None, None, None, None, None)) == moe.COLIBRI_ERR_INVALID_ARG
    assert down(moe._Experts(None, None, fake(12) + 2, None, None)) == moe.COLIBRI_ERR_INVALID_ARG
    # SwiGLU takes no biases; ReLU takes no W3
    assert down(moe._Experts(None, None, fake(12), None, fake(13))) == moe.COLIBRI_ERR_UNSUPPORTED
    assert down(moe._Experts(None, fake(11), fake(12), None, None), shape_c(act=moe.RELU)) == \
        moe.COLIBRI_ERR_UNSUPPORTED
    # misaligned hidden rows
    e = moe._Experts(fake(10), fake(11), None, None, None)
    assert lib.colibri_moe_expert_ffn_up(ctypes.byref(s), fake(0), fake(1), fake(2), ctypes.byref(e), fake(3) + 4,
                                         None, 0, None) == moe.COLIBRI_ERR_INVALID_ARG


# ------------------------------------------------------------------ int8 expert weights
def q8_experts(**kw):
    base = dict(q1=fake(10), q3=fake(11), q2=fake(12), s1=fake(13), s3=fake(14), s2=fake(15), b1=None, b2=None)
    base.update(kw)
    return moe._ExpertsQ8(base["q1"], base["q3"], base["q2"], base["s1"], base["s3"], base["s2"], base["b1"],
                          base["b2"])


def ffn_q8_call(lib, s, e, ws_bytes=1 << 40, ws=fake(9), y=fake(8)):
    return lib.colibri_moe_expert_ffn_q8(ctypes.byref(s), fake(0), fake(1), fake(2), ctypes.byref(e), y, ws,
                                         ws_bytes, None)


def test_q8_ffn_checks(lib):
    s = shape_c()
    e = q8_experts()
    # decode sizes only: bf16 and T <= 64
    assert ffn_q8_call(lib, shape_c(T=65), e) == moe.COLIBRI_ERR_UNSUPPORTED
    assert ffn_q8_call(lib, shape_c(dtype=moe.F32), e) == moe.COLIBRI_ERR_UNSUPPORTED
    assert ffn_q8_call(lib, s, e, ws_bytes=1024) == moe.COLIBRI_ERR_WORKSPACE
    # codes and scales of both layers are required; SwiGLU needs q3/s3 and takes no biases
    for k in ("q1", "q2", "s1", "s2", "q3", "s3"):
        assert ffn_q8_call(lib, s, q8_experts(**{k: None})) == moe.COLIBRI_ERR_INVALID_ARG, k
    assert ffn_q8_call(lib, s, q8_experts(b1=fake(16))) == moe.COLIBRI_ERR_UNSUPPORTED
    # ReLU / GELU take no q3/s3
    sr = shape_c(act=moe.GELU)
    assert ffn_q8_call(lib, sr, q8_experts(s3=None)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert ffn_q8_call(lib, sr, q8_experts(q3=None)) == moe.COLIBRI_ERR_UNSUPPORTED
    # alignment: codes 16 bytes, scales 4 bytes
    assert ffn_q8_call(lib, s, q8_experts(q1=fake(10) + 8)) == moe.COLIBRI_ERR_INVALID_ARG
    assert ffn_q8_call(lib, s, q8_experts(s2=fake(15) + 2)) == moe.COLIBRI_ERR_INVALID_ARG
    # T = 0 is a no-op even with null pointers
    assert lib.colibri_moe_expert_ffn_q8(ctypes.byref(shape_c(T=0)), None, None, None, None, None, None, 0,
                                         None) == 0


def test_q8_layer_checks(lib):
    s = shape_c()
    need = lib.colibri_moe_workspace_size(ctypes.byref(s))

    def call(sh=s, e=q8_experts(), ws_bytes=need, x=fake(0)):
        return lib.colibri_moe_layer_forward_q8(ctypes.byref(sh), x, fake(1), None, ctypes.byref(e), fake(3), None,
                                                None, None, fake(20), ws_bytes, None)

    assert call(ws_bytes=need - 1) == moe.COLIBRI_ERR_WORKSPACE
    assert call(x=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(sh=shape_c(T=100)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(e=q8_experts(q2=None)) == moe.COLIBRI_ERR_INVALID_ARG


def test_quantize_checks(lib):
    def call(w=fake(0), dtype=moe.BF16, E=2, K=64, N=128, q=fake(1), sc=fake(2)):
        return lib.colibri_moe_quantize_q8(w, dtype, E, K, N, q, sc, None)

    assert call(w=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(q=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(sc=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(N=130) == moe.COLIBRI_ERR_UNSUPPORTED  # columns in groups of 4
    assert call(K=0) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(dtype=5) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(w=fake(0) + 8) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(sc=fake(2) + 1) == moe.COLIBRI_ERR_INVALID_ARG


# ------------------------------------------------------------------ 4-bit expert weights
def q4_experts(**kw):
    names = ("q1", "q3", "q2", "s1", "s3", "s2", "z1", "z3", "z2", "b1", "b2")
    base = {n: fake(10 + i) for i, n in enumerate(names[:9])}
    base.update(b1=None, b2=None)
    base.update(kw)
    return moe._ExpertsQ4(*(base[n] for n in names))


def ffn_q4_call(lib, s, e, ws_bytes=1 << 40, ws=fake(9), y=fake(8)):
    return lib.colibri_moe_expert_ffn_q4(ctypes.byref(s), fake(0), fake(1), fake(2), ctypes.byref(e), y, ws,
                                         ws_bytes, None)


def test_q4_ffn_checks(lib):
    s = shape_c()
    assert s.d % 128 == 0 and s.h % 128 == 0
    e = q4_experts()
    # decode sizes only: bf16, T <= 64, d and h multiples of the 128-channel group
    assert ffn_q4_call(lib, shape_c(T=65), e) == moe.COLIBRI_ERR_UNSUPPORTED
    assert ffn_q4_call(lib, shape_c(dtype=moe.F32), e) == moe.COLIBRI_ERR_UNSUPPORTED
    assert ffn_q4_call(lib, shape_c(d=s.d + 64), e) == moe.COLIBRI_ERR_UNSUPPORTED
    assert ffn_q4_call(lib, shape_c(h=s.h + 64), e) == moe.COLIBRI_ERR_UNSUPPORTED
    assert ffn_q4_call(lib, s, e, ws_bytes=1024) == moe.COLIBRI_ERR_WORKSPACE
    # codes, scales and zero points of both layers are required; SwiGLU needs the third and takes no biases
    for k in ("q1", "q2", "s1", "s2", "z1", "z2", "q3", "s3", "z3"):
        assert ffn_q4_call(lib, s, q4_experts(**{k: None})) == moe.COLIBRI_ERR_INVALID_ARG, k
    assert ffn_q4_call(lib, s, q4_experts(b2=fake(20))) == moe.COLIBRI_ERR_UNSUPPORTED
    sr = shape_c(act=moe.GELU)
    assert ffn_q4_call(lib, sr, q4_experts(z3=None, s3=None)) == moe.COLIBRI_ERR_UNSUPPORTED
    # alignment: codes and scales 16 bytes, zero points 4
    assert ffn_q4_call(lib, s, q4_experts(q2=fake(12) + 8)) == moe.COLIBRI_ERR_INVALID_ARG
    assert ffn_q4_call(lib, s, q4_experts(s1=fake(13) + 4)) == moe.COLIBRI_ERR_INVALID_ARG
    assert ffn_q4_call(lib, s, q4_experts(z2=fake(18) + 2)) == moe.COLIBRI_ERR_INVALID_ARG
    assert lib.colibri_moe_expert_ffn_q4(ctypes.byref(shape_c(T=0)), None, None, None, None, None, None, 0,
                                         None) == 0


def test_q4_layer_checks(lib):
    s = shape_c()
    need = lib.colibri_moe_workspace_size(ctypes.byref(s))

    def call(sh=s, e=q4_experts(), ws_bytes=need, x=fake(0)):
        return lib.colibri_moe_layer_forward_q4(ctypes.byref(sh), x, fake(1), None, ctypes.byref(e), fake(3), None,
                                                None, None, fake(20), ws_bytes, None)

    assert call(ws_bytes=need - 1) == moe.COLIBRI_ERR_WORKSPACE
    assert call(x=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(sh=shape_c(T=100)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(e=q4_experts(z1=None)) == moe.COLIBRI_ERR_INVALID_ARG


def test_quantize_q4_checks(lib):
    def call(w=fake(0), dtype=moe.BF16, E=2, K=256, N=128, q=fake(1), sc=fake(2), z=fake(3)):
        return lib.colibri_moe_quantize_q4(w, dtype, E, K, N, q, sc, z, None)

    for k in ("w", "q", "sc", "z"):
        assert call(**{k: None}) == moe.COLIBRI_ERR_INVALID_ARG, k
    assert call(K=192) == moe.COLIBRI_ERR_UNSUPPORTED  # whole groups of 128
    assert call(K=0) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(N=130) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(dtype=5) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(q=fake(1) + 8) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(sc=fake(2) + 4) == moe.COLIBRI_ERR_INVALID_ARG


# ------------------------------------------------------------------ gating variants, shared expert, residual
def opts_c(gate=moe.GATE_PAIR, shared=None, shared_h=0, residual=None):
    return moe._Opts(gate, ctypes.pointer(shared) if shared is not None else None, shared_h, residual)


def layer_ex_call(lib, s, o, ws_bytes=1 << 40, e=None):
    e = e or moe._Experts(fake(4), fake(5), fake(6), None, None)
    return lib.colibri_moe_layer_forward_ex(ctypes.byref(s), fake(0), fake(1), None, ctypes.byref(e),
                                            ctypes.byref(o) if o is not None else None, fake(3), None, None, None,
                                            fake(20), ws_bytes, None)


def test_workspace_size_ex(lib):
    s = shape_c()
    plain = lib.colibri_moe_workspace_size(ctypes.byref(s))
    assert lib.colibri_moe_workspace_size_ex(ctypes.byref(s), None) == plain
    for gate in (moe.GATE_PAIR, moe.GATE_SOFTMAX, moe.GATE_LINEAR):
        o = opts_c(gate=gate, residual=fake(30))
        assert lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(o)) == plain
    sh = moe._Experts(fake(7), fake(8), fake(9), None, None)
    with_shared = lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(opts_c(shared=sh)))
    wider = lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(opts_c(shared=sh, shared_h=4096)))
    assert plain < with_shared < wider
    # invalid options size nothing
    assert lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(opts_c(gate=3))) == 0
    assert lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(opts_c(shared=sh, shared_h=96))) == 0


def test_layer_ex_checks(lib):
    s = shape_c()
    sh = moe._Experts(fake(7), fake(8), fake(9), None, None)
    need = lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(opts_c(shared=sh)))
    assert layer_ex_call(lib, s, opts_c(shared=sh), ws_bytes=need - 1) == moe.COLIBRI_ERR_WORKSPACE
    assert layer_ex_call(lib, s, opts_c(gate=-1)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert layer_ex_call(lib, s, opts_c(gate=3)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert layer_ex_call(lib, s, opts_c(residual=fake(30) + 8)) == moe.COLIBRI_ERR_INVALID_ARG
    assert layer_ex_call(lib, s, opts_c(shared=sh, shared_h=-64)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert layer_ex_call(lib, s, opts_c(shared=sh, shared_h=100)) == moe.COLIBRI_ERR_UNSUPPORTED
    for bad in (-1, 3):  # colibri_combine_t
        o = opts_c()
        o.combine = bad
        assert layer_ex_call(lib, s, o) == moe.COLIBRI_ERR_UNSUPPORTED
        assert lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(o)) == 0
    o = opts_c()
    o.combine = moe.COMBINE["separate"]
    assert lib.colibri_moe_workspace_size_ex(ctypes.byref(s), ctypes.byref(o)) == \
        lib.colibri_moe_workspace_size(ctypes.byref(s))
    # the shared expert is checked like the routed ones (SwiGLU: W1, W3, W2 and no biases)
    for bad, code in ((moe._Experts(None, fake(8), fake(9), None, None), moe.COLIBRI_ERR_INVALID_ARG),
                      (moe._Experts(fake(7), None, fake(9), None, None), moe.COLIBRI_ERR_INVALID_ARG),
                      (moe._Experts(fake(7), fake(8), None, None, None), moe.COLIBRI_ERR_INVALID_ARG),
                      (moe._Experts(fake(7) + 4, fake(8), fake(9), None, None), moe.COLIBRI_ERR_INVALID_ARG),
                      (moe._Experts(fake(7), fake(8), fake(9), fake(10), None), moe.COLIBRI_ERR_UNSUPPORTED)):
        assert layer_ex_call(lib, s, opts_c(shared=bad)) == code
    # the routed experts are still checked
    e = moe._Experts(fake(4), None, fake(6), None, None)
    assert layer_ex_call(lib, s, None, e=e) == moe.COLIBRI_ERR_INVALID_ARG
    # T = 0: a no-op with null pointers, but options are still validated
    z = shape_c(T=0)
    ez = moe._Experts(None, None, None, None, None)
    assert lib.colibri_moe_layer_forward_ex(ctypes.byref(z), None, None, None, ctypes.byref(ez), None, None, None,
                                            None, None, None, 0, None) == 0
    assert lib.colibri_moe_layer_forward_ex(ctypes.byref(z), None, None, None, ctypes.byref(ez),
                                            ctypes.byref(opts_c(gate=7)), None, None, None, None, None, 0,
                                            None) == moe.COLIBRI_ERR_UNSUPPORTED


def test_route_and_combine_ex_checks(lib):
    s = shape_c()
    r = lambda gate, x=fake(0): lib.colibri_moe_route_ex(ctypes.byref(s), x, fake(1), None, gate, fake(2), fake(3),
                                                         None, None)
    assert r(3) == moe.COLIBRI_ERR_UNSUPPORTED
    assert r(-1) == moe.COLIBRI_ERR_UNSUPPORTED
    assert r(moe.GATE_SOFTMAX, x=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert r(moe.GATE_LINEAR, x=fake(0) + 2) == moe.COLIBRI_ERR_INVALID_ARG
    c = lambda sh=None, res=None, y=fake(0): lib.colibri_moe_combine_ex(ctypes.byref(s), y, fake(1), fake(2), sh,
                                                                        res, fake(3), None)
    assert c(sh=fake(4) + 8) == moe.COLIBRI_ERR_INVALID_ARG
    assert c(res=fake(5) + 2) == moe.COLIBRI_ERR_INVALID_ARG
    assert c(y=None) == moe.COLIBRI_ERR_INVALID_ARG


# ------------------------------------------------------------------ multi-layer step, graph
def params_c(n, **kw):
    arr = (moe._LayerParams * n)()
    for i in range(n):
        base = dict(w_r=fake(40 + i), b_r=None, experts=moe._Experts(fake(50 + 3 * i), fake(51 + 3 * i),
                                                                       fake(52 + 3 * i), None, None),
                    gate=moe.GATE_PAIR, shared=None, shared_h=0)
        base.update(kw)
        arr[i] = moe._LayerParams(base["w_r"], base["b_r"], base["experts"], base["gate"], base["shared"],
                                  base["shared_h"])
    return arr


def test_step_and_graph_checks(lib):
    s = shape_c()
    one = lib.colibri_moe_workspace_size(ctypes.byref(s))
    assert lib.colibri_moe_step_workspace_size(ctypes.byref(s), 3, params_c(3)) == one
    sh = moe._Experts(fake(7), fake(8), fake(9), None, None)
    withsh = lib.colibri_moe_step_workspace_size(ctypes.byref(s), 2, params_c(2, shared=ctypes.pointer(sh)))
    assert withsh > one
    assert lib.colibri_moe_step_workspace_size(ctypes.byref(s), 0, params_c(1)) == 0
    assert lib.colibri_moe_step_workspace_size(ctypes.byref(s), 4097, params_c(1)) == 0

    def fwd(L=2, p=None, x=fake(1), ws_bytes=1 << 40, sh=s):
        return lib.colibri_moe_step_forward(ctypes.byref(sh), L, p if p is not None else params_c(L), 1, x,
                                            fake(20), ws_bytes, None)

    assert fwd(L=0) == moe.COLIBRI_ERR_UNSUPPORTED
    assert fwd(x=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert fwd(x=fake(1) + 8) == moe.COLIBRI_ERR_INVALID_ARG
    assert fwd(ws_bytes=one - 1) == moe.COLIBRI_ERR_WORKSPACE
    assert fwd(p=params_c(2, w_r=None)) == moe.COLIBRI_ERR_INVALID_ARG
    assert fwd(p=params_c(2, gate=5)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert fwd(p=params_c(2, experts=moe._Experts(fake(4), None, fake(6), None, None))) == moe.COLIBRI_ERR_INVALID_ARG
    assert fwd(p=params_c(2, shared=ctypes.pointer(sh), shared_h=100)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert fwd(sh=shape_c(T=0)) == 0  # T = 0: no-op
    # graph creation validates the same way before any HIP call; T = 0 has no graph
    h = ctypes.c_void_p(123)

    def create(L=2, p=None, ws_bytes=1 << 40, sh=s, out=ctypes.byref(h)):
        return lib.colibri_moe_graph_create(ctypes.byref(sh), L, p if p is not None else params_c(L), 1, fake(1),
                                            fake(20), ws_bytes, out)

    assert create(out=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert create(ws_bytes=one - 1) == moe.COLIBRI_ERR_WORKSPACE and h.value is None
    assert create(p=params_c(2, gate=-2)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert create(sh=shape_c(T=0)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert lib.colibri_moe_graph_launch(None, None) == moe.COLIBRI_ERR_INVALID_ARG
    assert lib.colibri_moe_graph_destroy(None) == 0


def test_dispatch_workspace_size(lib):
    small = shape_c(T=2047)
    large = shape_c(T=2048)
    assert lib.colibri_moe_dispatch_workspace_size(ctypes.byref(small)) == 0
    need = lib.colibri_moe_dispatch_workspace_size(ctypes.byref(large))
    # two [2T / 64][E] int32 tables (chunk counts, chunk starts), 256-byte aligned
    assert need == 2 * ((64 * 8 * 4 + 255) // 256 * 256)
    assert lib.colibri_moe_dispatch_workspace_size(ctypes.byref(shape_c(T=2048, E=65))) == 0
    # the layer's workspace holds it
    assert lib.colibri_moe_workspace_size(ctypes.byref(large)) > lib.colibri_moe_workspace_size(
        ctypes.byref(shape_c(T=2047))) + need


def test_layer_noalloc_checks(lib):
    """The allocation-free layer validates on the host like the layer, and
    refuses a batch whose workspace exceeds its device array before it touches
    the GPU (no call here reaches the array's lookup)."""
    e = moe._Experts(fake(10), fake(11), fake(12), None, None)
    call = lambda s, x=fake(0), w_r=fake(1), out=fake(2): lib.colibri_moe_layer_forward_noalloc(
        ctypes.byref(s), x, w_r, None, ctypes.byref(e), out, None, None, None, None)
    assert call(shape_c(T=0), x=None, w_r=None, out=None) == moe.COLIBRI_OK
    assert call(shape_c(k=3)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert call(shape_c(), x=None) == moe.COLIBRI_ERR_INVALID_ARG
    assert call(shape_c(), out=fake(2) + 8) == moe.COLIBRI_ERR_INVALID_ARG
    big = shape_c(T=4096, d=4096, h=14336, E=8)
    assert lib.colibri_moe_workspace_size(ctypes.byref(big)) > moe.NOALLOC_SCRATCH_BYTES
    assert call(big) == moe.COLIBRI_ERR_WORKSPACE
    no_w3 = moe._Experts(fake(10), None, fake(12), None, None)
    assert lib.colibri_moe_layer_forward_noalloc(ctypes.byref(shape_c()), fake(0), fake(1), None, ctypes.byref(no_w3),
                                                 fake(2), None, None, None, None) == moe.COLIBRI_ERR_INVALID_ARG


def test_validate_env_rejects_non_device_pointers(lib, monkeypatch):
    """COLIBRI_MOE_VALIDATE=1: every tensor argument must lie inside a device
    allocation; the fake addresses used above are not, so each entry point
    returns INVALID_ARG on the host, before anything is launched."""
    monkeypatch.setenv("COLIBRI_MOE_VALIDATE", "1")
    s = shape_c()
    assert route_call(lib, s) == moe.COLIBRI_ERR_INVALID_ARG
    assert lib.colibri_moe_dispatch(ctypes.byref(s), fake(0), fake(1), fake(2), fake(3), fake(4), None, None, None,
                                    0, None) == moe.COLIBRI_ERR_INVALID_ARG
    assert lib.colibri_moe_combine(ctypes.byref(s), fake(0), fake(1), fake(2), fake(3), None) == \
        moe.COLIBRI_ERR_INVALID_ARG
    e = moe._Experts(fake(10), fake(11), fake(12), None, None)
    ws_bytes = lib.colibri_moe_workspace_size(ctypes.byref(s))
    assert lib.colibri_moe_layer_forward(ctypes.byref(s), fake(0), fake(1), None, ctypes.byref(e), fake(2), None,
                                         None, None, fake(20), ws_bytes, None) == moe.COLIBRI_ERR_INVALID_ARG
    assert lib.colibri_moe_expert_ffn(ctypes.byref(s), fake(0), fake(1), fake(2), ctypes.byref(e), fake(3),
                                      fake(20), ws_bytes, None) == moe.COLIBRI_ERR_INVALID_ARG
    # the shape and pointer checks still come first
    assert route_call(lib, shape_c(k=3)) == moe.COLIBRI_ERR_UNSUPPORTED
    assert route_call(lib, s, x=None) == moe.COLIBRI_ERR_INVALID_ARG


def test_binding_refuses_host_tensors(lib):
    """The binding hands the library device pointers only: a host tensor is refused before the call."""
    torch = pytest.importorskip("torch")
    s = moe.Shape(T=4, d=64, h=64, E=4, dtype=moe.BF16, act=moe.RELU)
    host = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.route(s, host, fake(1), None, fake(2), fake(3))
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.combine(s, fake(0), fake(1), fake(2), host)
