"""GPU parity: every C-ABI entry point and the whole layer against the fp64
oracle on seeded inputs.

Bar (per the method's reading):
  * expert indices, counts, offsets and the dispatch permutation: bit-exact,
    except that tokens whose oracle logit margin (1st/2nd or 2nd/3rd) is below
    1e-6 are counted, reported and exempt from the index comparison only;
    the oracle's top-2 of the GPU's own fp32 logits must equal the GPU's
    indices, and the oracle's dispatch of the GPU's indices must equal the
    GPU's dispatch, with no exemption;
  * fp32 values: max relative error <= 1e-4, taken per output row (the
    row's largest |error| over its largest |reference|);
  * bf16 values: |a - b| <= 1e-2 + 2e-2 |b| for every element.
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


# ------------------------------------------------------------------ router
def run_route(layer):
    sh = layer.shape
    x = G.dev(layer.x)
    idx = G.empty((sh.T, 2), torch.int32)
    gate = G.empty((sh.T, 2), torch.float32)
    lg = G.empty((sh.T, sh.E), torch.float32)
    r = G.device_router(layer.key)
    moe.route(sh, x, r["w_r"], r["b_r"], idx, gate, lg)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gate.cpu().numpy(), lg.cpu().numpy()


def check_route(layer, idx, gate, lg_gpu, tag):
    w = G.host_router(layer.key)
    lg_ref = oracle.logits(layer.x, w["w_r"], w["b_r"])
    S_lg = G.logits_scale(layer.x, w["w_r"], w["b_r"])
    G.assert_fp32_close(lg_gpu, lg_ref, S_lg, f"{tag} logits")
    # the GPU's selection is exactly the oracle's top-2 of the GPU's own logits
    assert np.array_equal(oracle.top2(lg_gpu.astype(np.float64)), idx), f"{tag}: top-2 of own logits"
    diff, ties = G.assert_selection(idx, lg_ref, tag)
    # gates: fp32 rule against the oracle's gates for the GPU's chosen pair
    g_ref = oracle.gates(lg_ref, idx)
    G.assert_fp32_close(gate, g_ref, G.gates_scale(S_lg, idx, g_ref, lg_ref), f"{tag} gates")
    assert np.all(gate[:, 0] + gate[:, 1] == np.float32(1.0)), f"{tag}: gates must sum to exactly 1 in fp32"
    assert np.all(gate[:, 0] >= 0.5)
    G.report({"check": "route", "case": tag, "tokens": int(layer.T), **ties})


ROUTE_CASES = [("tiny", 32), ("e8", 1), ("e8", 64), ("e8", 512), ("mixtral_decode", 1), ("mixtral_decode", 4),
               ("mixtral_decode", 16), ("mixtral_decode", 32), ("mixtral_prefill", 4096), ("skew16", 8192)]


@pytest.mark.parametrize("key,T", ROUTE_CASES, ids=[f"{k}-T{t}" for k, t in ROUTE_CASES])
def test_route_parity(key, T):
    layer = G.seeded_layer(key, T)
    idx, gate, lg = run_route(layer)
    check_route(layer, idx, gate, lg, f"{key}/T={T}")


@pytest.mark.parametrize("E", [2, 3, 5, 16, 33, 64])
@pytest.mark.parametrize("dt", [gen.F32, gen.BF16])
def test_route_expert_counts_and_ties(E, dt):
    """Every padded expert width, ragged token counts, and exact ties."""
    rng = np.random.default_rng(E * 10 + dt)
    T, d = 77, 192
    x = rng.integers(-2, 3, size=(T, d)).astype(np.float32)       # integer data: exact sums, many ties
    w_r = rng.integers(-1, 2, size=(d, E)).astype(np.float32)
    x[5] = 0.0                                                      # all-zero token: every logit ties
    if dt == gen.BF16:
        x, w_r = gen.f32_to_bf16_bits(x), gen.f32_to_bf16_bits(w_r)
    sh = moe.Shape(T, d, 64, E, dt, moe.RELU)
    idx = G.empty((T, 2), torch.int32)
    gate = G.empty((T, 2), torch.float32)
    lg = G.empty((T, E), torch.float32)
    moe.route(sh, G.dev(x), G.dev(w_r), None, idx, gate, lg)
    torch.cuda.synchronize()
    idx, gate, lg = idx.cpu().numpy(), gate.cpu().numpy(), lg.cpu().numpy()
    lg_ref = oracle.logits(x, w_r)
    assert np.array_equal(lg.astype(np.float64), lg_ref)           # integer sums are exact in fp32
    assert np.array_equal(idx, oracle.top2(lg_ref))                # ties resolved to the lower index
    assert tuple(idx[5]) == (0, 1) and gate[5].tolist() == [0.5, 0.5]
    g_ref = oracle.gates(lg_ref, idx)
    G.assert_fp32_close(gate, g_ref, G.gates_scale(G.logits_scale(x, w_r), idx, g_ref, lg_ref), f"gates E={E}")


def test_route_bias_and_nan_ranking():
    T, d, E = 8, 64, 6
    x = np.zeros((T, d), np.float32)
    w_r = np.zeros((d, E), np.float32)
    b_r = np.array([0.5, 2.0, -1.0, 2.0, 1.0, -np.inf], np.float32)
    sh = moe.Shape(T, d, 64, E, gen.F32, moe.RELU)
    idx = G.empty((T, 2), torch.int32)
    gate = G.empty((T, 2), torch.float32)
    moe.route(sh, G.dev(x), G.dev(w_r), G.dev(b_r), idx, gate)
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == [[1, 3]] * T               # bias only; tie 2.0/2.0 -> lower index first
    b_r[1] = np.nan
    moe.route(sh, G.dev(x), G.dev(w_r), G.dev(b_r), idx, gate)
    torch.cuda.synchronize()
    assert idx.cpu().numpy().tolist() == [[3, 4]] * T               # NaN ranks below every number


# ------------------------------------------------------------------ dispatch
def run_dispatch(idx: np.ndarray, E: int, x=None, dt=gen.BF16, multi=False):
    """multi: hand the entry point scratch, so that large batches take the
    multi-workgroup path (count, scan and scatter kernels)."""
    T = idx.shape[0]
    sh = moe.Shape(T, 64 if x is None else x.shape[1], 64, E, dt, moe.RELU)
    ws, ws_bytes = None, 0
    if multi:
        ws_bytes = moe.dispatch_workspace_size(sh)
        assert ws_bytes > 0 or 2 * T < 4096
        ws = G.empty((max(ws_bytes, 256),), torch.uint8) if ws_bytes else None
    counts = G.empty((E,), torch.int32)
    offsets = G.empty((E + 1,), torch.int32)
    sa = G.empty((2 * T,), torch.int32)
    ap = G.empty((2 * T,), torch.int32)
    xd = G.dev(x) if x is not None else None
    xs = G.empty((2 * T, x.shape[1]), G.tdtype(dt)) if x is not None else None
    moe.dispatch(sh, G.dev(idx.astype(np.int32)), counts, offsets, sa, ap, xd, xs, ws=ws, ws_bytes=ws_bytes)
    torch.cuda.synchronize()
    r = {"counts": counts.cpu().numpy(), "offsets": offsets.cpu().numpy(), "sorted_assign": sa.cpu().numpy(),
         "assign_pos": ap.cpu().numpy()}
    if xs is not None:
        r["x_sorted"] = G.host(xs)
    return r


def _pairs(rng, T, E, p=None):
    a = rng.choice(E, size=T, p=p)
    b = (a + rng.integers(1, E, size=T)) % E
    return np.stack([a, b], 1).astype(np.int32)


DISPATCH_CASES = [(1, 8), (31, 4), (32, 4), (33, 4), (1000, 8), (4096, 8), (8192, 16), (50000, 64), (3, 2),
                  (70001, 16)]


@pytest.mark.parametrize("multi", [False, True], ids=["one-wg", "multi-wg"])
@pytest.mark.parametrize("T,E", DISPATCH_CASES, ids=[f"T{t}-E{e}" for t, e in DISPATCH_CASES])
def test_dispatch_bit_exact(T, E, multi):
    rng = np.random.default_rng(T + E)
    idx = _pairs(rng, T, E)
    r = run_dispatch(idx, E, multi=multi)
    ref = oracle.dispatch(idx, E)
    for k in ("counts", "offsets", "sorted_assign", "assign_pos"):
        assert np.array_equal(r[k], ref[k]), k


@pytest.mark.parametrize("multi", [False, True], ids=["one-wg", "multi-wg"])
def test_dispatch_degenerate_routings(multi):
    # every token to the same pair (other experts empty), and a Zipf-like skew
    for idx, E in ((np.tile([[6, 1]], (5000, 1)).astype(np.int32), 8),
                   (np.tile([[0, 63]], (129, 1)).astype(np.int32), 64),
                   (np.tile([[0, 63]], (2049, 1)).astype(np.int32), 64),
                   (_pairs(np.random.default_rng(9), 20000, 16,
                           p=(np.arange(1, 17) ** -1.2) / (np.arange(1, 17) ** -1.2).sum()), 16)):
        r = run_dispatch(idx, E, multi=multi)
        ref = oracle.dispatch(idx, E)
        for k in ("counts", "offsets", "sorted_assign", "assign_pos"):
            assert np.array_equal(r[k], ref[k]), k


def test_dispatch_multi_skips_out_of_range_indices():
    """The multi-workgroup path with indices outside [0, E) scattered through a
    large batch: the same counts, order and -1 markers as the one-workgroup path."""
    rng = np.random.default_rng(12)
    T, E = 3001, 8
    idx = _pairs(rng, T, E)
    flat = idx.reshape(-1)
    bad = rng.choice(flat.size, 97, replace=False)
    flat[bad] = rng.choice([-1, -7, E, E + 5], size=97)
    one = run_dispatch(idx, E)
    multi = run_dispatch(idx, E, multi=True)
    for k in ("counts", "offsets", "sorted_assign", "assign_pos"):
        assert np.array_equal(one[k], multi[k]), k
    valid = (flat >= 0) & (flat < E)
    assert multi["offsets"][-1] == valid.sum()
    assert np.all(multi["assign_pos"][~valid] == -1)
    assert np.all(multi["sorted_assign"][valid.sum():] == -1)
    order = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    assert np.array_equal(multi["sorted_assign"][:valid.sum()], order)


def test_dispatch_row_gather():
    rng = np.random.default_rng(3)
    T, E, d = 300, 8, 192
    idx = _pairs(rng, T, E)
    x = gen.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    r = run_dispatch(idx, E, x=x)
    xf = gen.bf16_bits_to_f32(x)
    assert np.array_equal(r["x_sorted"], xf[r["sorted_assign"] // 2])


def test_dispatch_skips_out_of_range_indices():
    idx = np.array([[1, 2], [9, 0], [1, -3], [3, 3]], np.int32)   # 9 and -3 are outside [0, 4)
    r = run_dispatch(idx, 4)
    valid = (idx.reshape(-1) >= 0) & (idx.reshape(-1) < 4)
    assert r["counts"].tolist() == np.bincount(idx.reshape(-1)[valid], minlength=4).tolist()
    assert r["offsets"][-1] == valid.sum()
    assert np.all(r["assign_pos"][~valid] == -1)
    assert np.all(r["sorted_assign"][valid.sum():] == -1)
    order = np.flatnonzero(valid)[np.argsort(idx.reshape(-1)[valid], kind="stable")]
    assert np.array_equal(r["sorted_assign"][:valid.sum()], order)


# ------------------------------------------------------------------ expert FFN
def small_ffn_case(act, dt, T=300, E=8, d=256, h=384, skew=None, seed=0):
    rng = np.random.default_rng(seed)
    cvt = (lambda a: a) if dt == gen.F32 else gen.f32_to_bf16_bits
    f = lambda s, sc: cvt((rng.standard_normal(s) * sc).astype(np.float32))
    w = {"x": f((T, d), 1.0), "w1": f((E, d, h), d ** -0.5), "w2": f((E, h, d), h ** -0.5),
         "w3": f((E, d, h), d ** -0.5) if act == "swiglu" else None,
         "b1": f((E, h), 0.1) if act != "swiglu" else None, "b2": f((E, d), 0.1) if act != "swiglu" else None}
    idx = _pairs(rng, T, E, p=skew)
    return w, idx


def run_ffn(w, idx, act, dt, E, gather=True, scale_out=None):
    """y_sorted from the GPU and the oracle; with a list for scale_out, the fp32
    scale of every row is appended to it (None for bf16)."""
    T, d = w["x"].shape
    h = w["w1"].shape[2]
    ref = oracle.dispatch(idx, E)
    sh = moe.Shape(T, d, h, E, dt, moe.ACT_CODES[act])
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    y = G.empty((2 * T, d), G.tdtype(dt))
    if gather:
        x_rows, sa = G.dev(w["x"]), G.dev(ref["sorted_assign"])
    else:
        x_rows, sa = G.dev(np.ascontiguousarray(w["x"][ref["sorted_assign"] // 2])), None
    moe.expert_ffn(sh, x_rows, sa, G.dev(ref["offsets"]), G.dev(w["w1"]), G.dev(w["w2"]), y, ws, ws_bytes,
                   w3=G.dev(w["w3"]), b1=G.dev(w["b1"]), b2=G.dev(w["b2"]))
    torch.cuda.synchronize()
    rows_t = ref["sorted_assign"] // 2
    rows_e = idx.reshape(-1)[ref["sorted_assign"]]
    y_ref = oracle.ffn_rows(w["x"], rows_t, rows_e, w["w1"], w["w2"], act, w3=w["w3"], b1=w["b1"], b2=w["b2"],
                            mirror=True)
    if scale_out is not None:
        scale_out.append(G.ffn_scale(w["x"], rows_t, rows_e, w["w1"], w["w2"], act, w3=w["w3"], b1=w["b1"],
                                     b2=w["b2"]) if dt == gen.F32 else None)
    return G.host(y), y_ref


FFN_CASES = [(a, dt) for a in ("relu", "gelu", "swiglu") for dt in (gen.F32, gen.BF16)]


@pytest.mark.parametrize("act,dt", FFN_CASES, ids=[f"{a}-{'f32' if d == 0 else 'bf16'}" for a, d in FFN_CASES])
def test_ffn_parity_small(act, dt):
    w, idx = small_ffn_case(act, dt)
    sc = []
    y, y_ref = run_ffn(w, idx, act, dt, E=8, scale_out=sc)
    G.assert_close(y, y_ref, dt, f"y_sorted {act}", scale=sc[0])


@pytest.mark.parametrize("dt", [gen.F32, gen.BF16])
def test_ffn_ragged_columns_and_presorted_rows(dt):
    # h = 320 and d = 192: column counts that are not multiples of 128
    w, idx = small_ffn_case("gelu", dt, T=173, E=5, d=192, h=320, seed=4)
    for gather in (True, False):
        sc = []
        y, y_ref = run_ffn(w, idx, "gelu", dt, E=5, gather=gather, scale_out=sc)
        G.assert_close(y, y_ref, dt, f"y_sorted gather={gather}", scale=sc[0])


# first layers whose tiles fill whole rounds of one workgroup per CU plus a
# last round of at most half the CUs: that round's tiles run as f K parts and a
# small kernel adds the parts.  f = 2 (272 and 528 tiles), f = 3 (328 tiles:
# 72 in the last round), f = 4 (808 tiles: 40 in the last round); "skew"
# routes every token to experts 0 and 1, so the kernel finds too few tiles to
# split
TAIL_CASES = [(80, 16, 512, 2176, "swiglu", None), (100, 8, 512, 8448, "gelu", None),
              (100, 8, 768, 5248, "swiglu", None), (100, 8, 1024, 12928, "swiglu", None),
              (400, 16, 512, 2176, "swiglu", "skew")]


@pytest.mark.parametrize("T,E,d,h,act,mode", TAIL_CASES,
                         ids=[f"T{c[0]}-E{c[1]}-d{c[2]}-h{c[3]}-{c[4]}" + (f"-{c[5]}" if c[5] else "")
                              for c in TAIL_CASES])
def test_ffn_tail_split(T, E, d, h, act, mode):
    w, idx = small_ffn_case(act, gen.BF16, T=T, E=E, d=d, h=h, seed=T + E)
    if mode == "skew":
        idx[:, 0], idx[:, 1] = 0, 1
    for gather in (True, False):
        y, y_ref = run_ffn(w, idx, act, gen.BF16, E=E, gather=gather)
        G.assert_bf16_close(y, y_ref, f"tail split T={T} gather={gather}")


def test_ffn_tail_split_full_size():
    """8-expert SwiGLU layer at T = 512 (d = 2048, h = 5632): 352 first-layer tiles, of which the 96
    of the last round run as K halves; a seeded sample of rows of every expert against the oracle."""
    T, E, d, h, act = 512, 8, 2048, 5632, "swiglu"
    w, idx = small_ffn_case(act, gen.BF16, T=T, E=E, d=d, h=h, seed=11)
    ref = oracle.dispatch(idx, E)
    sh = moe.Shape(T, d, h, E, gen.BF16, moe.ACT_CODES[act])
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    y = G.empty((2 * T, d), G.tdtype(gen.BF16))
    moe.expert_ffn(sh, G.dev(w["x"]), G.dev(ref["sorted_assign"]), G.dev(ref["offsets"]), G.dev(w["w1"]),
                   G.dev(w["w2"]), y, ws, ws_bytes, w3=G.dev(w["w3"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    off = ref["offsets"]
    pos = np.unique(np.concatenate([[off[e], off[e + 1] - 1] for e in range(E) if off[e + 1] > off[e]] +
                                   [rng.choice(2 * T, size=32, replace=False)]))
    rows_t = ref["sorted_assign"][pos] // 2
    rows_e = idx.reshape(-1)[ref["sorted_assign"][pos]]
    y_ref = oracle.ffn_rows(w["x"], rows_t, rows_e, w["w1"], w["w2"], act, w3=w["w3"], mirror=True)
    G.assert_bf16_close(G.host(y)[pos], y_ref, "tail split, full size")


SHORT_K_CASES = [(256, 2, 64, 128, "swiglu"), (256, 2, 128, 64, "gelu"), (300, 2, 192, 320, "relu"),
                 (256, 3, 64, 64, "swiglu")]


@pytest.mark.parametrize("T,E,d,h,act", SHORT_K_CASES,
                         ids=[f"T{c[0]}-E{c[1]}-d{c[2]}-h{c[3]}-{c[4]}" for c in SHORT_K_CASES])
def test_ffn_big_tiles_short_k(T, E, d, h, act):
    """The large-tile GEMM with K of 1, 2, 3 or 5 k-tiles of 64: the copies of the k-tiles past
    the last one (which re-read it) and the first k-tiles' copies issued before the loop."""
    w, idx = small_ffn_case(act, gen.BF16, T=T, E=E, d=d, h=h, seed=T + d + h)
    for gather in (True, False):
        y, y_ref = run_ffn(w, idx, act, gen.BF16, E=E, gather=gather)
        G.assert_bf16_close(y, y_ref, f"short K d={d} h={h} gather={gather}")


def _random_ffn_cases(n=10, seed=2026):
    """Seeded random grouped-GEMM shapes (T > 64, so the tiled GEMM path runs):
    E in [2, 64], d and h multiples of 64, all three activations, uniform or
    Zipf-skewed routing; tile counts land anywhere relative to the CU rounds,
    so whole rounds, remainders and tail splits all occur.  The oracle's work
    (2T rows of the full FFN) stays below about 4e9 multiply-adds per case."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.integers(65, 2500))
        E = int(rng.integers(2, 65))
        d = 64 * int(rng.integers(1, 17))
        h = 64 * int(rng.integers(1, 25))
        act = ("relu", "gelu", "swiglu")[len(out) % 3]
        skew = bool(rng.integers(0, 2))
        if 2 * T * d * h * (3 if act == "swiglu" else 2) > 4e9:
            continue
        out.append((T, E, d, h, act, skew))
    return out


RANDOM_FFN_CASES = _random_ffn_cases()


@pytest.mark.parametrize("T,E,d,h,act,skew", RANDOM_FFN_CASES,
                         ids=[f"T{c[0]}-E{c[1]}-d{c[2]}-h{c[3]}-{c[4]}" + ("-zipf" if c[5] else "") for c in RANDOM_FFN_CASES])
def test_ffn_random_shapes(T, E, d, h, act, skew):
    """The grouped GEMM path on seeded random shapes against the oracle, every row."""
    p = None
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p = p / p.sum()
    w, idx = small_ffn_case(act, gen.BF16, T=T, E=E, d=d, h=h, skew=p, seed=T + E + d + h)
    for gather in (True, False):
        y, y_ref = run_ffn(w, idx, act, gen.BF16, E=E, gather=gather)
        G.assert_bf16_close(y, y_ref, f"random shape T={T} E={E} d={d} h={h} {act} gather={gather}")


DECODE_CASES = [(1, 8, 256, 384, "swiglu"), (1, 2, 128, 320, "gelu"), (5, 8, 192, 256, "relu"),
                (16, 4, 256, 320, "swiglu"), (33, 8, 128, 192, "gelu"), (64, 8, 256, 256, "swiglu"),
                (64, 64, 64, 128, "relu"), (2, 16, 1024, 512, "swiglu")]


@pytest.mark.parametrize("T,E,d,h,act", DECODE_CASES, ids=[f"T{c[0]}-E{c[1]}-d{c[2]}-h{c[3]}-{c[4]}" for c in DECODE_CASES])
def test_ffn_decode_sizes(T, E, d, h, act):
    """Decode-sized batches (weight-streaming kernel, split-K with ordered fixup)."""
    w, idx = small_ffn_case(act, gen.BF16, T=T, E=E, d=d, h=h, seed=T * 7 + E)
    for gather in (True, False):
        y, y_ref = run_ffn(w, idx, act, gen.BF16, E=E, gather=gather)
        G.assert_bf16_close(y, y_ref, f"decode T={T} gather={gather}")


def test_ffn_decode_expert_over_32_rows():
    """T = 64 with every token on experts 0 and 1: 64 rows per expert run as two 32-row chunks."""
    w, idx = small_ffn_case("swiglu", gen.BF16, T=64, E=8, d=256, h=256, seed=3)
    idx[:, 0], idx[:, 1] = 0, 1
    y, y_ref = run_ffn(w, idx, "swiglu", gen.BF16, E=8)
    G.assert_bf16_close(y, y_ref, "decode chunked rows")
    # a repeated call on the same workspace (which holds the first call's partials) gives the same bits
    y2, _ = run_ffn(w, idx, "swiglu", gen.BF16, E=8)
    assert np.array_equal(y, y2)


FUSED_H_CASES = [(5, 8, 192, 256, "relu", None), (3, 8, 512, 1024, "gelu", None), (4, 16, 512, 2048, "swiglu", None),
                 (24, 16, 512, 2048, "swiglu", "two")]


@pytest.mark.parametrize("T,E,d,h,act,skew", FUSED_H_CASES,
                         ids=[f"T{c[0]}-E{c[1]}-d{c[2]}-h{c[3]}-{c[4]}" + ("-skew" if c[5] else "") for c in FUSED_H_CASES])
def test_ffn_decode_h_from_partials(T, E, d, h, act, skew):
    """Decode shapes whose first layer is K-split: inside expert_ffn the second
    layer rebuilds H from the first layer's partials (no H store, no reduce
    launch).  It must equal the single-layer entry points chained through H
    (which reduce and store H) bit for bit.  "two": every token on experts 0
    and 1, so 24 rows per expert run as a 16-row chunk and a ragged 8-row one."""
    w, idx = small_ffn_case(act, gen.BF16, T=T, E=E, d=d, h=h, seed=T + E + d)
    if skew == "two":
        idx[:, 0], idx[:, 1] = 0, 1
    ref = oracle.dispatch(idx, E)
    sh = moe.Shape(T, d, h, E, gen.BF16, moe.ACT_CODES[act])
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    x, sa, off = G.dev(w["x"]), G.dev(ref["sorted_assign"]), G.dev(ref["offsets"])
    dw = {k: G.dev(w[k]) for k in ("w1", "w2", "w3", "b1", "b2")}
    y_full = G.empty((2 * T, d), torch.bfloat16)
    H = G.empty((2 * T, h), torch.bfloat16)
    y = G.empty((2 * T, d), torch.bfloat16)
    for _ in range(2):  # the second call reuses a scratch that holds the first call's partials
        moe.expert_ffn(sh, x, sa, off, dw["w1"], dw["w2"], y_full, ws, ws_bytes, w3=dw["w3"], b1=dw["b1"],
                       b2=dw["b2"])
        moe.expert_ffn_up(sh, x, sa, off, dw["w1"], H, ws, ws_bytes, w3=dw["w3"], b1=dw["b1"])
        moe.expert_ffn_down(sh, H, off, dw["w2"], y, ws, ws_bytes, b2=dw["b2"])
        torch.cuda.synchronize()
        assert torch.equal(y, y_full)
    y_ref = oracle.ffn_rows(w["x"], ref["sorted_assign"] // 2, idx.reshape(-1)[ref["sorted_assign"]], w["w1"],
                            w["w2"], act, w3=w["w3"], b1=w["b1"], b2=w["b2"], mirror=True)
    G.assert_bf16_close(G.host(y_full), y_ref, f"fused-H decode T={T}")


ROW_TILE_COUNTS = {
    # large tiles (up to 320 rows, 64-row pairs dealt out evenly): 641 -> 256 + 256 + 129,
    # 321 -> 192 + 129, 320 -> 320, 650 -> 256 + 256 + 138, 1030 -> 320 + 256 + 256 + 198, 33 -> 33
    # (subtiles 2 / 1 over the two wave rows), 1 and 10 -> one subtile, the other wave row empty
    "big": [641, 321, 320, 33, 1, 0, 650, 10, 1030],
    # mid-size tiles (128 rows, up to 192; no more than 160 rows per expert on average):
    # 129 -> 1 x 129, 160 -> 1 x 160, 192 -> 2 x 96, 193 -> 97 + 96, 255 -> 128 + 127
    "mid": [129, 160, 192, 193, 255, 1, 0, 70],
}


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("which", ["big", "mid"])
def test_ffn_row_tiles_split_evenly(act, which):
    """Per-expert counts around the grouped GEMM's row-tile boundaries: experts are
    cut into equal row tiles, a small tail is spread over the other tiles, and the
    tiles' 32-row subtiles split unevenly over the two wave rows."""
    counts = ROW_TILE_COUNTS[which]
    E = len(counts)
    rng = np.random.default_rng(21)
    slots = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), counts))
    T = len(slots) // 2
    w, _ = small_ffn_case(act, gen.BF16, T=T, E=E, d=128, h=256, seed=21)
    idx = slots.reshape(T, 2)
    for gather in (True, False):
        y, y_ref = run_ffn(w, idx, act, gen.BF16, E=E, gather=gather)
        G.assert_bf16_close(y, y_ref, f"row tiles {act} gather={gather}")


SPLIT_CASES = [(100, 8, 2048, 128, "swiglu"), (100, 8, 2048, 128, "gelu"), (300, 8, 128, 2048, "relu"),
               (300, 8, 128, 2048, "swiglu")]


@pytest.mark.parametrize("T,E,d,h,act", SPLIT_CASES, ids=[f"T{c[0]}-d{c[2]}-h{c[3]}-{c[4]}" for c in SPLIT_CASES])
def test_ffn_gemm_k_split(T, E, d, h, act):
    """Few tiles and a long K: the grouped GEMM splits K (d = 2048: the first
    layer, h = 2048: the second), writes fp32 partials and a reduce applies the
    epilogue; for the second layer the layer entry point instead lets the
    combine add the partials (covered by the composed-equality test)."""
    w, idx = small_ffn_case(act, gen.BF16, T=T, E=E, d=d, h=h, seed=T + d)
    for gather in (True, False):
        y, y_ref = run_ffn(w, idx, act, gen.BF16, E=E, gather=gather)
        G.assert_bf16_close(y, y_ref, f"k split {act} gather={gather}")


def test_ffn_degenerate_routings():
    E = 8
    for seed, skew in ((1, [0.93] + [0.01] * 7), (2, [0.5, 0.5, 0, 0, 0, 0, 0, 0])):
        w, idx = small_ffn_case("swiglu", gen.BF16, T=257, E=E, seed=seed, skew=skew)
        if seed == 2:
            idx[:, 1] = 1 - idx[:, 0]     # only experts 0 and 1 used; 6 empty experts
        y, y_ref = run_ffn(w, idx, "swiglu", gen.BF16, E=E)
        G.assert_bf16_close(y, y_ref, f"degenerate routing {seed}")


def test_ffn_small_integers_bit_exact():
    """bf16 ReLU path with small-integer operands: every MFMA product and fp32
    sum is exact, so y must equal the oracle bit for bit (tests tiling and
    indexing with no rounding noise)."""
    rng = np.random.default_rng(11)
    T, E, d, h = 200, 4, 256, 192
    ints = lambda s, lo, hi: gen.f32_to_bf16_bits(rng.integers(lo, hi + 1, size=s).astype(np.float32))
    w = {"x": ints((T, d), -3, 3), "w1": ints((E, d, h), -2, 2), "w2": ints((E, h, d), -2, 2), "w3": None,
         "b1": ints((E, h), -4, 4), "b2": ints((E, d), -4, 4)}
    idx = _pairs(rng, T, E)
    y, y_ref = run_ffn(w, idx, "relu", gen.BF16, E=E)
    assert np.array_equal(y.astype(np.float64), y_ref)


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("dt", [gen.F32, gen.BF16])
def test_combine_parity(dt):
    rng = np.random.default_rng(5)
    T, d = 333, 448
    ap = rng.permutation(2 * T).astype(np.int32)
    g0 = rng.uniform(0.5, 1.0, T).astype(np.float32)
    gate = np.stack([g0, np.float32(1) - g0], 1)
    yf = rng.standard_normal((2 * T, d)).astype(np.float32)
    y = yf if dt == gen.F32 else gen.f32_to_bf16_bits(yf)
    sh = moe.Shape(T, d, 64, 4, dt, moe.RELU)
    out = G.empty((T, d), G.tdtype(dt))
    moe.combine(sh, G.dev(y), G.dev(ap), G.dev(gate), out)
    torch.cuda.synchronize()
    y64 = yf.astype(np.float64) if dt == gen.F32 else gen.bf16_bits_to_f32(y).astype(np.float64)
    ref = oracle.combine(y64, ap, gate.astype(np.float64), dt)
    G.assert_close(G.host(out), ref, dt, "combine",
                   scale=G.combine_scale(gate, np.stack([y64[ap[0::2]], y64[ap[1::2]]], 1)))


# ------------------------------------------------------------------ whole layer
def run_layer(layer, stream=None):
    """The layer through colibri_moe_layer_forward; besides its outputs, the
    dispatch it computed internally (offsets and both permutations), read from
    the workspace at the offsets colibri_moe_workspace_layout reports."""
    sh = layer.shape
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    out = G.empty((sh.T, sh.d), G.tdtype(sh.dtype))
    idx = G.empty((sh.T, 2), torch.int32)
    gate = G.empty((sh.T, 2), torch.float32)
    counts = G.empty((sh.E,), torch.int32)
    dw = layer.dw
    moe.layer_forward(sh, G.dev(layer.x), dw["w_r"], dw["b_r"], dw["w1"], dw["w2"], out, ws, ws_bytes, w3=dw["w3"],
                      b1=dw["b1"], b2=dw["b2"], topk_idx=idx, topk_gate=gate, counts=counts, stream=stream)
    torch.cuda.synchronize()
    lay = moe.workspace_layout(sh)
    wsh = ws.cpu().numpy()
    i32 = lambda off, n: wsh[off:off + 4 * n].view(np.int32).copy()
    return {"out": out, "idx": idx.cpu().numpy(), "gate": gate.cpu().numpy(), "counts": counts.cpu().numpy(),
            "offsets": i32(lay["expert_offsets"], sh.E + 1), "sorted_assign": i32(lay["sorted_assign"], 2 * sh.T),
            "assign_pos": i32(lay["assign_pos"], 2 * sh.T)}


def row_tile_starts(R: int, big: bool):
    """First rows (relative to the expert's first row) of the grouped GEMM's row
    tiles of an expert of R rows.  Big tiles (up to 320 rows): the expert's
    ceil(R / 64) 64-row pairs dealt out evenly over ceil(R / 320) tiles; mid
    tiles (128 rows, up to 192): equal tiles, a tail of at most 32 rows spread
    over the others."""
    if big:
        P, mt = -(-R // 64), -(-R // 320)
        q, r = divmod(P, mt)
        return [64 * (m * q + min(m, r)) for m in range(mt)]
    mt = -(-R // 128)
    if mt > 1 and R % 128 != 0 and R % 128 <= 32 and R <= 192 * (mt - 1):
        mt -= 1
    rt = -(-R // mt)
    return list(range(0, R, rt))


def tile_edge_rows(offsets: np.ndarray) -> np.ndarray:
    """Expert-sorted rows at the edges of the grouped GEMM's tiles: the first
    and last row of every row tile of every expert, under both tilings the
    GEMM uses, and of every 32-row subtile inside each tile."""
    rows = set()
    for big in (True, False):
        for e in range(len(offsets) - 1):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi == lo:
                continue
            starts = [lo + s for s in row_tile_starts(hi - lo, big)] + [hi]
            for t0, t1 in zip(starts[:-1], starts[1:]):
                for s0 in range(t0, t1, 32):
                    rows.update((s0, min(s0 + 31, t1 - 1)))
    return np.array(sorted(rows), np.int64)


# token selection: every token, or the tokens owning the rows at the GEMM's tile edges
LAYER_CASES = [("tiny", 32, "all"), ("e8", 1, "all"), ("e8", 64, "all"), ("e8", 512, "all"),
               ("mixtral_decode", 1, "all"), ("mixtral_decode", 4, "all"), ("mixtral_decode", 16, "all"),
               ("mixtral_decode", 32, "all"), ("mixtral_prefill", 4096, "tiles"), ("skew16", 8192, "tiles")]


@pytest.mark.parametrize("key,T,which", LAYER_CASES, ids=[f"{k}-T{t}" for k, t, _ in LAYER_CASES])
def test_layer_parity(key, T, which):
    layer = G.seeded_layer(key, T)
    print(f"layer parity {key} T={T}", flush=True)
    r = run_layer(layer)
    w = layer.hw
    E = layer.cfg.E
    # routing over all tokens
    lg_ref = oracle.logits(layer.x, w["w_r"], w["b_r"])
    diff, ties = G.assert_selection(r["idx"], lg_ref, f"{key}/T={T}")
    # the layer's own dispatch (the fused route + dispatch kernel up to 16 tokens) is
    # exactly the oracle's dispatch of the indices it chose
    d_ref = oracle.dispatch(r["idx"], E)
    for k in ("counts", "offsets", "sorted_assign", "assign_pos"):
        assert np.array_equal(r[k], d_ref[k]), f"{key}/T={T}: layer dispatch {k} differs from the oracle's"
    assert r["counts"].sum() == 2 * T
    assert np.all(r["gate"].sum(1) == np.float32(1.0))
    out = G.host(r["out"])
    assert np.all(np.isfinite(out))
    if which == "all":
        toks = np.arange(T)
    else:
        edge = tile_edge_rows(r["offsets"])
        toks = np.unique(r["sorted_assign"][edge] >> 1)
    toks = np.union1d(toks, np.flatnonzero(diff))  # every token whose indices differ
    ref = layer.oracle_tokens(toks, idx_override=r["idx"][toks])
    assert np.array_equal(ref["idx"], r["idx"][toks])
    scale = None
    if layer.cfg.dtype == gen.F32:
        scale = G.layer_scale(layer.x, w["w_r"], w["b_r"], w["w1"], w["w2"], layer.cfg.act, toks, r["idx"][toks],
                              ref, w3=w["w3"], b1=w["b1"], b2=w["b2"])
    G.assert_close(out[toks], ref["out"], layer.cfg.dtype, f"{key}/T={T} out", scale=scale)
    G.report({"check": "layer", "case": f"{key}/T={T}", "tokens_compared": int(len(toks)), **ties,
              "counts": r["counts"].tolist()})


@pytest.mark.parametrize("key,T", [("e8", 64), ("e8", 1), ("mixtral_decode", 1), ("e8", 512)])
def test_layer_equals_composed_entry_points(key, T):
    """layer_forward equals route -> dispatch -> expert_ffn -> combine bit for bit
    (at T = 1 the layer call adds the second layer's K-split partials inside
    the combine instead of a separate reduce)."""
    layer = G.seeded_layer(key, T)
    r = run_layer(layer)
    sh = layer.shape
    idx, gate, _ = run_route(layer)
    d = run_dispatch(idx, sh.E)
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    y = G.empty((2 * sh.T, sh.d), torch.bfloat16)
    dw = layer.dw
    moe.expert_ffn(sh, G.dev(layer.x), G.dev(d["sorted_assign"]), G.dev(d["offsets"]), dw["w1"], dw["w2"], y, ws,
                   ws_bytes, w3=dw["w3"], b1=dw["b1"], b2=dw["b2"])
    out = G.empty((sh.T, sh.d), torch.bfloat16)
    moe.combine(sh, y, G.dev(d["assign_pos"]), G.dev(gate), out)
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])


@pytest.mark.parametrize("act,dt", [("swiglu", gen.BF16), ("gelu", gen.BF16), ("relu", gen.F32)])
def test_ffn_up_down_compose(act, dt):
    """The two single-layer entry points chained through H equal expert_ffn."""
    w, idx = small_ffn_case(act, dt, T=150, E=6, d=192, h=256, seed=21)
    T, d = w["x"].shape
    h = w["w1"].shape[2]
    ref = oracle.dispatch(idx, 6)
    sh = moe.Shape(T, d, h, 6, dt, moe.ACT_CODES[act])
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    x, sa, off = G.dev(w["x"]), G.dev(ref["sorted_assign"]), G.dev(ref["offsets"])
    dw = {k: G.dev(w[k]) for k in ("w1", "w2", "w3", "b1", "b2")}
    y_full = G.empty((2 * T, d), G.tdtype(dt))
    moe.expert_ffn(sh, x, sa, off, dw["w1"], dw["w2"], y_full, ws, ws_bytes, w3=dw["w3"], b1=dw["b1"], b2=dw["b2"])
    H = G.empty((2 * T, h), G.tdtype(dt))
    y = G.empty((2 * T, d), G.tdtype(dt))
    moe.expert_ffn_up(sh, x, sa, off, dw["w1"], H, ws, ws_bytes, w3=dw["w3"], b1=dw["b1"])
    moe.expert_ffn_down(sh, H, off, dw["w2"], y, ws, ws_bytes, b2=dw["b2"])
    torch.cuda.synchronize()
    assert torch.equal(y, y_full)
    rt, re = ref["sorted_assign"] // 2, idx.reshape(-1)[ref["sorted_assign"]]
    scale = G.ffn_scale(w["x"], rt, re, w["w1"], w["w2"], act, w3=w["w3"], b1=w["b1"], b2=w["b2"]) \
        if dt == gen.F32 else None
    G.assert_close(G.host(y), oracle.ffn_rows(w["x"], rt, re, w["w1"], w["w2"], act, w3=w["w3"], b1=w["b1"],
                                              b2=w["b2"]), dt, "y", scale=scale)


def test_layer_deterministic_and_stream():
    layer = G.seeded_layer("e8", 512)
    a = run_layer(layer)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_layer(layer, stream=s)
    assert torch.equal(a["out"], b["out"]) and np.array_equal(a["idx"], b["idx"])


@pytest.mark.parametrize("E,d,h,act,dt", [(2, 64, 64, "relu", gen.F32), (64, 128, 192, "swiglu", gen.BF16),
                                          (3, 64, 128, "gelu", gen.BF16), (64, 64, 64, "gelu", gen.F32)])
def test_layer_shape_edges(E, d, h, act, dt):
    """Smallest and largest expert counts and dims, T = 1 and ragged T."""
    rng = np.random.default_rng(E + d + h)
    cvt = (lambda a: a) if dt == gen.F32 else gen.f32_to_bf16_bits
    f = lambda s, sc: cvt((rng.standard_normal(s) * sc).astype(np.float32))
    for T in (1, 2, 97):
        x, w_r = f((T, d), 1.0), f((d, E), d ** -0.5)
        w = {"w1": f((E, d, h), d ** -0.5), "w2": f((E, h, d), h ** -0.5),
             "w3": f((E, d, h), d ** -0.5) if act == "swiglu" else None,
             "b1": f((E, h), 0.1) if act != "swiglu" else None, "b2": f((E, d), 0.1) if act != "swiglu" else None}
        sh = moe.Shape(T, d, h, E, dt, moe.ACT_CODES[act])
        ws_bytes = moe.workspace_size(sh)
        ws = G.empty((ws_bytes,), torch.uint8)
        out = G.empty((T, d), G.tdtype(dt))
        idx = G.empty((T, 2), torch.int32)
        moe.layer_forward(sh, G.dev(x), G.dev(w_r), None, G.dev(w["w1"]), G.dev(w["w2"]), out, ws, ws_bytes,
                          w3=G.dev(w["w3"]), b1=G.dev(w["b1"]), b2=G.dev(w["b2"]), topk_idx=idx)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
        ref = oracle.layer_tokens(x, w_r, w["w1"], w["w2"], act, np.arange(T), w3=w["w3"], b1=w["b1"], b2=w["b2"],
                                  idx_override=gi)
        lg = ref["logits"]
        G.assert_selection(gi, lg, f"E={E} d={d} h={h} T={T}")
        scale = G.layer_scale(x, w_r, None, w["w1"], w["w2"], act, np.arange(T), gi, ref, w3=w["w3"], b1=w["b1"],
                              b2=w["b2"]) if dt == gen.F32 else None
        G.assert_close(G.host(out), ref["out"], dt, f"E={E} d={d} h={h} T={T}", scale=scale)


ROUTER_SHAPES = [(24, 64, 1), (24, 320, 17), (40, 320, 33), (63, 192, 200), (48, 2048, 16), (9, 4096, 31),
                 (2, 128, 40), (64, 128, 5)]


@pytest.mark.parametrize("E,d,T", ROUTER_SHAPES, ids=[f"E{e}-d{d}-T{t}" for e, d, t in ROUTER_SHAPES])
def test_router_odd_shapes_and_fused_path(E, d, T):
    """The bf16 router at expert counts that leave part of a 16-expert column
    tile empty, k-step counts that do not fill the waves evenly, and token
    counts around the 16-token tiles; up to 16 tokens the layer routes with
    the fused route + dispatch kernel, which must choose exactly what the route
    entry point chooses."""
    rng = np.random.default_rng(E * 1000 + d + T)
    x = gen.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w_r = gen.f32_to_bf16_bits((rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32))
    b_r = (rng.standard_normal(E) * 0.1).astype(np.float32)
    sh = moe.Shape(T, d, 64, E, gen.BF16, moe.RELU)
    idx = G.empty((T, 2), torch.int32)
    gate = G.empty((T, 2), torch.float32)
    lg = G.empty((T, E), torch.float32)
    xd, wd, bd = G.dev(x), G.dev(w_r), G.dev(b_r)
    moe.route(sh, xd, wd, bd, idx, gate, lg)
    torch.cuda.synchronize()
    idx_h, gate_h, lg_h = idx.cpu().numpy(), gate.cpu().numpy(), lg.cpu().numpy()
    lg_ref = oracle.logits(x, w_r, b_r)
    S_lg = G.logits_scale(x, w_r, b_r)
    G.assert_fp32_close(lg_h, lg_ref, S_lg, "logits")
    assert np.array_equal(oracle.top2(lg_h.astype(np.float64)), idx_h)
    G.assert_selection(idx_h, lg_ref, "router odd shapes")
    g_ref = oracle.gates(lg_ref, idx_h)
    G.assert_fp32_close(gate_h, g_ref, G.gates_scale(S_lg, idx_h, g_ref, lg_ref), "gates")
    # the whole layer (fused routing at T <= 16) picks the same experts and gates
    w1 = G.dev(gen.f32_to_bf16_bits((rng.standard_normal((E, d, 64)) / np.sqrt(d)).astype(np.float32)))
    w2 = G.dev(gen.f32_to_bf16_bits((rng.standard_normal((E, 64, d)) / 8).astype(np.float32)))
    ws_bytes = moe.workspace_size(sh)
    ws = G.empty((ws_bytes,), torch.uint8)
    out = G.empty((T, d), torch.bfloat16)
    idx2 = G.empty((T, 2), torch.int32)
    gate2 = G.empty((T, 2), torch.float32)
    counts = G.empty((E,), torch.int32)
    moe.layer_forward(sh, xd, wd, bd, w1, w2, out, ws, ws_bytes, topk_idx=idx2, topk_gate=gate2, counts=counts)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), idx_h)
    assert np.array_equal(gate2.cpu().numpy(), gate_h)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(idx_h.reshape(-1), minlength=E))
