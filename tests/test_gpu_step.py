"""Multi-layer step and its HIP-graph replay on the GPU.

Each layer of a step is checked against the fp64 oracle on the GPU's own
input to that layer (the same bar as the single layer: bf16 elements within
1e-2 + 2e-2 |b|, fp32 rows within 1e-4), because a bf16 rounding difference
in one layer's output legitimately moves the next layer's near-tied routings
(the bf16 bound takes the largest summand of the combine as its scale, as
for the other layer variants).
The step entry point must equal the chain of single-layer calls bit for bit,
and every graph replay must equal the eager step bit for bit (replays are
interleaved with eager work on the same buffers).
"""
import numpy as np
import pytest

import gen
import mixture_experts_layer_12_amd as moe
import oracle
from tests import gpu_util as G

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module", autouse=True)
def lib():
    return moe.load(build_if_missing=True)


def stored(t) -> np.ndarray:
    """device tensor -> the stored values (fp32, or bf16 bit patterns as uint16)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def make_stack(key, L, gate, shared):
    base = gen.CONFIGS[key]
    host, devl = [], []
    for l in range(L):
        c = gen.layer_of(base, l)
        h = dict(gen.make_experts(c))
        h["w_r"] = gen.make_router(c)
        h["b_r"] = gen.router_bias(base)
        h["gate"] = gate
        if shared:
            h["shared"] = gen.make_shared_expert(c)
            h["shared_h"] = base.shared_h
        d = {k: (G.dev(v) if isinstance(v, np.ndarray) else v) for k, v in h.items() if k != "shared"}
        if shared:
            d["shared"] = {k: G.dev(v) for k, v in h["shared"].items()}
        host.append(h)
        devl.append(d)
    return host, devl


def layer_chain(shape, devl, x0, residual):
    """The step as single-layer calls; returns every layer's input and indices."""
    xs, idxs = [x0.clone()], []
    for d in devl:
        ws_bytes = moe.workspace_size_ex(shape, gate=d["gate"], shared=d.get("shared"), shared_h=d.get("shared_h", 0))
        ws = G.empty((ws_bytes,), torch.uint8)
        out = torch.empty_like(x0)
        idx = G.empty((shape.T, 2), torch.int32)
        moe.layer_forward_ex(shape, xs[-1], d["w_r"], d.get("b_r"), d["w1"], d["w2"], out, ws, ws_bytes,
                             w3=d.get("w3"), b1=d.get("b1"), b2=d.get("b2"), gate=d["gate"], shared=d.get("shared"),
                             shared_h=d.get("shared_h", 0), residual=xs[-1] if residual else None, topk_idx=idx)
        xs.append(out)
        idxs.append(idx)
    torch.cuda.synchronize()
    return xs, [i.cpu().numpy() for i in idxs]


# key, T, layers, gating, shared expert, residual
STEP_CASES = [
    ("tiny", 32, 3, "pair", False, True),
    ("e8", 1, 4, "pair", False, True),
    ("e8", 64, 3, "softmax", False, True),
    ("e8", 512, 2, "pair", False, False),
    ("e8", 1024, 2, "pair", False, True),  # large-tile GEMMs, the second split in K
    ("shared15", 1, 3, "softmax", True, True),
    ("shared15", 64, 3, "softmax", True, True),
    ("mixtral_decode", 4, 2, "pair", False, True),
]


@pytest.mark.parametrize("key,T,L,gate,shared,residual", STEP_CASES,
                         ids=[f"{c[0]}-T{c[1]}-L{c[2]}-{c[3]}{'-shared' if c[4] else ''}{'-res' if c[5] else ''}"
                              for c in STEP_CASES])
def test_step_and_graph(key, T, L, gate, shared, residual):
    cfg = gen.CONFIGS[key]
    shape = moe.Shape(T, cfg.d, cfg.h, cfg.E, cfg.dtype, gen.ACT_CODE[cfg.act])
    host, devl = make_stack(key, L, gate, shared)
    x0 = G.dev(gen.make_x(cfg, T))
    xs, idxs = layer_chain(shape, devl, x0, residual)

    # each layer against the oracle on that layer's GPU input
    rng = np.random.default_rng(T + L)
    toks = np.arange(T) if T <= 64 else np.sort(rng.choice(T, 24, replace=False))
    for l, h in enumerate(host):
        xin = stored(xs[l])
        ref = oracle.layer_tokens(xin, h["w_r"], h["w1"], h["w2"], cfg.act, toks, b_r=h["b_r"], w3=h["w3"],
                                  b1=h["b1"], b2=h["b2"], mirror=True, idx_override=idxs[l][toks], gate=gate,
                                  shared=h.get("shared"), residual=xin if residual else None)
        lg = oracle.logits(xin, h["w_r"], h["b_r"])
        G.assert_selection(idxs[l], lg, f"layer {l}")
        scale = None
        if cfg.dtype == gen.F32:
            scale = G.layer_scale(xin, h["w_r"], h["b_r"], h["w1"], h["w2"], cfg.act, toks, idxs[l][toks], ref,
                                  w3=h["w3"], b1=h["b1"], b2=h["b2"], gate=gate, shared=h.get("shared"),
                                  residual=xin if residual else None)
        G.assert_layer_close(G.host(xs[l + 1])[toks], ref, cfg.dtype, f"{key} layer {l}",
                             residual=G.host(xs[l])[toks] if residual else None, scale=scale)

    # the step entry point is the chain, bit for bit
    ws_bytes = moe.step_workspace_size(shape, devl)
    assert ws_bytes > 0
    ws = G.empty((ws_bytes,), torch.uint8)
    x = x0.clone()
    moe.step_forward(shape, devl, x, ws, ws_bytes, residual=residual)
    torch.cuda.synchronize()
    assert torch.equal(x, xs[-1]), "step_forward differs from the chain of layer calls"

    # graph replays: x reset by an eager copy, eager layer work between replays
    g = moe.Graph(shape, devl, x, ws, ws_bytes, residual=residual)
    try:
        for rep in range(3):
            x.copy_(x0)
            g.launch()
            torch.cuda.synchronize()
            assert torch.equal(x, xs[-1]), f"graph replay {rep} differs from the eager step"
            moe.step_forward(shape, devl[:1], x, ws, ws_bytes, residual=residual)  # eager work on the same buffers
            torch.cuda.synchronize()
            assert torch.equal(x, layer_chain(shape, devl[:1], xs[-1], residual)[0][-1])
        # on a side stream too
        s = torch.cuda.Stream()
        x.copy_(x0)
        torch.cuda.synchronize()
        g.launch(stream=s)
        s.synchronize()
        assert torch.equal(x, xs[-1])
    finally:
        g.destroy()
    G.report({"check": "step", "case": f"{key}/T={T}/L={L}/{gate}/shared={shared}/residual={residual}",
              "tokens_compared_per_layer": int(len(toks))})
