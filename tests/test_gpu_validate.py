"""COLIBRI_MOE_VALIDATE=1 on the GPU: with valid inputs the layer's results
are those of an unvalidated call, bit for bit; non-finite inputs and expert
indices outside [0, E) are refused with COLIBRI_ERR_INVALID_ARG before
anything is launched (the outputs are left untouched).  (Pointers outside any
device allocation are refused the same way; that case runs on the host, in
the ABI tests, since on the GPU a failed check would let a kernel write past
an allocation.)"""
import numpy as np
import pytest

import gen
import mixture_experts_layer_12_amd as moe
from tests import gpu_util as G

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _layer(layer, x=None, dw=None, out=None):
    sh = layer.shape
    dw = dw or layer.dw
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    if out is None:
        out = G.empty((sh.T, sh.d), G.tdtype(sh.dtype))
    idx = G.empty((sh.T, 2), torch.int32)
    moe.layer_forward(sh, G.dev(layer.x) if x is None else x, dw["w_r"], dw["b_r"], dw["w1"], dw["w2"], out, ws,
                      ws_bytes, w3=dw["w3"], b1=dw["b1"], b2=dw["b2"], topk_idx=idx)
    torch.cuda.synchronize()
    return out, idx


@pytest.mark.parametrize("key,T", [("e8", 64), ("mixtral_decode", 4), ("tiny", 32), ("e8", 512)])
def test_validated_layer_is_unchanged(key, T, monkeypatch):
    layer = G.seeded_layer(key, T)
    monkeypatch.delenv("COLIBRI_MOE_VALIDATE", raising=False)
    o0, i0 = _layer(layer)
    monkeypatch.setenv("COLIBRI_MOE_VALIDATE", "1")
    o1, i1 = _layer(layer)
    assert torch.equal(i0, i1)
    bits = (lambda t: t.view(torch.int16)) if o0.dtype == torch.bfloat16 else (lambda t: t)
    assert torch.equal(bits(o0), bits(o1))


def test_validate_refuses_bad_inputs(monkeypatch):
    layer = G.seeded_layer("e8", 64)
    sh = layer.shape
    monkeypatch.setenv("COLIBRI_MOE_VALIDATE", "1")
    sentinel = -12345.0
    # a NaN in x
    x = G.dev(layer.x)
    x[7, 100] = float("nan")
    out = torch.full((sh.T, sh.d), sentinel, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.ColibriError) as ei:
        _layer(layer, x=x, out=out)
    assert ei.value.status == moe.COLIBRI_ERR_INVALID_ARG
    assert bool((out == sentinel).all()), "nothing may be launched"
    # an Inf in one expert's second-layer weights
    dw = dict(layer.dw)
    w2 = dw["w2"].clone()
    w2[5, 3, 11] = float("inf")
    dw["w2"] = w2
    with pytest.raises(moe.ColibriError) as ei:
        _layer(layer, dw=dw, out=out)
    assert ei.value.status == moe.COLIBRI_ERR_INVALID_ARG
    assert bool((out == sentinel).all())
    # the same call without the variable runs (and does not check)
    monkeypatch.delenv("COLIBRI_MOE_VALIDATE")
    _layer(layer, dw=dw, out=out)
    assert not bool((out == sentinel).all())


def test_validate_refuses_out_of_range_indices(monkeypatch):
    T, E = 100, 8
    rng = np.random.default_rng(3)
    idx = rng.integers(0, E, size=(T, 2)).astype(np.int32)
    idx[17, 1] = E  # outside [0, E)
    sh = moe.Shape(T, 64, 64, E, gen.BF16, moe.RELU)
    counts = G.empty((E,), torch.int32)
    offsets = G.empty((E + 1,), torch.int32)
    sa = G.empty((2 * T,), torch.int32)
    ap = G.empty((2 * T,), torch.int32)
    monkeypatch.setenv("COLIBRI_MOE_VALIDATE", "1")
    with pytest.raises(moe.ColibriError) as ei:
        moe.dispatch(sh, G.dev(idx), counts, offsets, sa, ap)
    assert ei.value.status == moe.COLIBRI_ERR_INVALID_ARG
    idx[17, 1] = 3
    moe.dispatch(sh, G.dev(idx), counts, offsets, sa, ap)
    torch.cuda.synchronize()
    assert int(offsets[-1]) == 2 * T


def test_binding_refuses_tensors_that_do_not_fit():
    """The Python binding checks tensors before the call: contiguous, elements
    of the layer's width, large enough for the shape; ws_bytes within ws."""
    layer = G.seeded_layer("e8", 64)
    sh, dw = layer.shape, layer.dw
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    x = G.dev(layer.x)
    out = G.empty((sh.T, sh.d), torch.bfloat16)
    call = lambda **kw: moe.layer_forward(sh, kw.get("x", x), dw["w_r"], dw["b_r"], dw["w1"], dw["w2"],
                                          kw.get("out", out), kw.get("ws", ws), kw.get("ws_bytes", ws_bytes),
                                          b1=dw["b1"], b2=dw["b2"])
    with pytest.raises(ValueError, match="contiguous"):
        call(x=G.empty((sh.d, 2 * sh.T), torch.bfloat16).t()[:sh.T])
    with pytest.raises(ValueError, match="needs"):
        call(out=out[: sh.T - 1])
    with pytest.raises(TypeError, match="bytes"):
        call(out=G.empty((sh.T, sh.d), torch.float32))
    with pytest.raises(ValueError, match="exceeds"):
        call(ws_bytes=ws_bytes + 256)
    call(ws_bytes=None)  # the tensor's own size
    torch.cuda.synchronize()
