#!/usr/bin/env python3
"""Benchmark of the MoE layer forward pass on one MI355X.

Default workload (the prefill metric's configuration): the Mixtral-shaped
layer -- E=8 experts, top-2, d=4096, h=14336, SwiGLU experts, bf16 storage
with fp32 accumulation -- on a T=4096-token batch; one step = one
colibri_moe_layer_forward (route, dispatch, grouped expert FFN, combine) over
the batch.  Inputs are seeded synthetic tensors already resident in HBM;
expert weights rotate over enough identical copies (>= 2 GB) that the 256 MB
last-level cache cannot serve them.

Timing is GPU time from HIP events on the stream the kernels run on.  Before
each timed region a spin kernel keeps the GPU busy while the host enqueues
the work, so host launch latency does not show up as GPU idle time inside the
region.  The K timed steps are bracketed by one pair of events (value,
ms_per_step) and each step also by its own pair (median, min, p90).

Prints one JSON line: the layer's tokens/s, the roofline of the dominant
kernel (the first-layer grouped GEMM: bf16 MFMA bound), every entry point's
time, and -- as extra keys -- the Mixtral-shaped decode batches (T = 1, 4,
16, 32; bf16, int8 and 4-bit weights), the 16-expert Zipf-skewed prefill
(T = 8192), the 8-expert 1.3B-class layer (T = 1, 64, 512), the layer
variants, the multi-layer decode step, the chip's achieved streaming-read
and MFMA ceilings, and the fp64 CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
SLEEP_CYCLES = 3_000_000     # spin kernel in front of a timed region (~1.5 ms)
METRIC = "MoE-layer tokens/s (prefill) + µs/step (decode); % of MFMA / HBM peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_prefill", help="workload key in gen.CONFIGS")
    ap.add_argument("--T", type=int, default=None, help="tokens per step (default: the config's largest T)")
    ap.add_argument("--rotate-gb", type=float, default=2.0, help="total bytes of rotated weight copies")
    ap.add_argument("--decode-iters", type=int, default=200)
    ap.add_argument("--headline-only", action="store_true", help="only the headline workload (no extra keys)")
    ap.add_argument("--no-quantized", action="store_true", help="skip the int8- and 4-bit-weight decode lines")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the shared-expert / softmax-gating / residual layer lines")
    ap.add_argument("--step-layers", type=int, default=8,
                    help="layers of the multi-layer decode step timed eagerly and as a HIP graph (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time for the headline workload")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (calibrates PMC byte counters)")
    return ap.parse_args()


# ---------------------------------------------------------------------------- helpers
class Gpu:
    """Device, stream, event timing and host -> device copies."""

    def __init__(self, torch, np):
        self.torch, self.np = torch, np
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.stream = torch.cuda.current_stream()
        self.can_sleep = hasattr(torch.cuda, "_sleep")

    def prefill_queue(self):
        if self.can_sleep:
            self.torch.cuda._sleep(SLEEP_CYCLES)

    def to_dev(self, a):
        if a is None:
            return None
        a = self.np.ascontiguousarray(a)
        if a.dtype == self.np.uint16:
            return self.torch.from_numpy(a.view(self.np.int16)).to(self.dev).view(self.torch.bfloat16)
        if a.dtype == self.np.uint32:
            return self.torch.from_numpy(a.view(self.np.int32)).to(self.dev)
        return self.torch.from_numpy(a).to(self.dev)

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def per_step_us(self, fn, iters, warmup, sync_every=10):
        """GPU time of each call (us), the queue pre-filled every sync_every calls."""
        torch = self.torch
        times = []
        for it in range(warmup + iters):
            e0, e1 = self.event(), self.event()
            if it % sync_every == 0:
                self.prefill_queue()
            e0.record(self.stream)
            fn(it)
            e1.record(self.stream)
            if it % sync_every == sync_every - 1:
                torch.cuda.synchronize()
            if it >= warmup:
                times.append((e0, e1))
        torch.cuda.synchronize()
        return self.np.array([a.elapsed_time(b) * 1e3 for a, b in times])


def stats(us, np):
    return {"median": round(float(np.median(us)), 2), "min": round(float(us.min()), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "mean": round(float(us.mean()), 2)}


def weight_key(gen, key):
    """Workloads that draw identical expert weights share one set (the Mixtral
    decode and prefill layers do)."""
    c = gen.CONFIGS[key]
    for k, o in gen.CONFIGS.items():
        if (o.E, o.d, o.h, o.act, o.dtype, o.biases, o.seed) == (c.E, c.d, c.h, c.act, c.dtype, c.biases, c.seed):
            return k
    return key


class Weights:
    """R identical device copies of a workload's expert weights (R * bytes >= rotate_gb)."""

    def __init__(self, g, gen, cfg, rotate_gb):
        t0 = time.time()
        hw = gen.make_experts(cfg)
        w0 = {k: g.to_dev(v) for k, v in hw.items()}
        del hw
        self.el = 4 if cfg.dtype == gen.F32 else 2
        self.per_expert = {k: (v[0].numel() * self.el if v is not None else 0) for k, v in w0.items()}
        self.up_e = self.per_expert["w1"] + self.per_expert["w3"] + self.per_expert["b1"]
        self.down_e = self.per_expert["w2"] + self.per_expert["b2"]
        self.layer_bytes = sum(v.numel() * self.el for v in w0.values() if v is not None)
        self.R = max(1, math.ceil(rotate_gb * 1e9 / self.layer_bytes))
        self.copies = [w0] + [{k: (v.clone() if v is not None else None) for k, v in w0.items()}
                              for _ in range(self.R - 1)]
        log(f"{cfg.key}: {self.R} weight copies x {self.layer_bytes / 1e6:.1f} MB ({time.time() - t0:.1f}s)")

    def __getitem__(self, i):
        return self.copies[i % self.R]


class Layer:
    """One workload: router, inputs up to Tmax tokens, a workspace for Tmax."""

    def __init__(self, g, gen, moe, cfg, W, Tmax):
        torch = g.torch
        self.g, self.cfg, self.W, self.moe = g, cfg, W, moe
        self.x_np = gen.make_x(cfg, Tmax)
        self.w_r_np = gen.make_router(cfg)
        self.b_r_np = gen.router_bias(cfg)
        self.x, self.w_r, self.b_r = g.to_dev(self.x_np), g.to_dev(self.w_r_np), g.to_dev(self.b_r_np)
        self.act = gen.ACT_CODE[cfg.act]
        self.m = 2 if cfg.act == "swiglu" else 1
        self.shape = moe.Shape(Tmax, cfg.d, cfg.h, cfg.E, cfg.dtype, self.act)
        self.ws_bytes = moe.workspace_size(self.shape)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=g.dev)
        self.tdt = torch.float32 if cfg.dtype == gen.F32 else torch.bfloat16
        self.out = torch.empty((Tmax, cfg.d), dtype=self.tdt, device=g.dev)
        self.counts = torch.empty(cfg.E, dtype=torch.int32, device=g.dev)

    def step(self, i, T):
        w = self.W[i]
        s = self.shape.with_T(T)
        self.moe.layer_forward(s, self.x[:T], self.w_r, self.b_r, w["w1"], w["w2"], self.out[:T], self.ws,
                               self.ws_bytes, w3=w["w3"], b1=w["b1"], b2=w["b2"], counts=self.counts)

    def hit(self):
        return int((self.counts.cpu().numpy() > 0).sum())

    def weight_bytes(self, hit):
        return hit * (self.W.up_e + self.W.down_e)

    def flops(self, T):
        c = self.cfg
        return 2.0 * T * c.d * c.E + 2.0 * (2 * T) * c.d * c.h * (self.m + 1)

    def bytes(self, T, hit):
        """Algorithmic bytes of a step: X, W_r (+ b_r), the hit experts' weights,
        out, and the index and gate arrays."""
        c, el = self.cfg, self.W.el
        return (T * c.d * el + c.d * c.E * el + (c.E * 4 if self.b_r is not None else 0) + self.weight_bytes(hit)
                + T * c.d * el + T * 16)

    def entry_points(self, T, iters, warmup):
        """Average GPU time of each of the five single-step entry points (us)."""
        g, moe, torch, np = self.g, self.moe, self.g.torch, self.g.np
        c = self.cfg
        s = self.shape.with_T(T)
        A = 2 * T
        dev = g.dev
        idx = torch.empty((T, 2), dtype=torch.int32, device=dev)
        gate = torch.empty((T, 2), dtype=torch.float32, device=dev)
        offs = torch.empty(c.E + 1, dtype=torch.int32, device=dev)
        sa = torch.empty(A, dtype=torch.int32, device=dev)
        ap_ = torch.empty(A, dtype=torch.int32, device=dev)
        H = torch.empty((A, c.h), dtype=self.tdt, device=dev)
        y = torch.empty((A, c.d), dtype=self.tdt, device=dev)
        names = ("route", "dispatch", "ffn_up", "ffn_down", "combine")
        acc = np.zeros(len(names))
        for it in range(warmup + iters):
            w = self.W[it]
            evs = [g.event() for _ in range(len(names) + 1)]
            g.prefill_queue()
            evs[0].record(g.stream)
            moe.route(s, self.x[:T], self.w_r, self.b_r, idx, gate)
            evs[1].record(g.stream)
            moe.dispatch(s, idx, self.counts, offs, sa, ap_, ws=self.ws, ws_bytes=self.ws_bytes)
            evs[2].record(g.stream)
            moe.expert_ffn_up(s, self.x[:T], sa, offs, w["w1"], H, self.ws, self.ws_bytes, w3=w["w3"], b1=w["b1"])
            evs[3].record(g.stream)
            moe.expert_ffn_down(s, H, offs, w["w2"], y, self.ws, self.ws_bytes, b2=w["b2"])
            evs[4].record(g.stream)
            moe.combine(s, y, ap_, gate, self.out[:T])
            evs[5].record(g.stream)
            torch.cuda.synchronize()
            if it >= warmup:
                acc += np.array([evs[j].elapsed_time(evs[j + 1]) * 1e3 for j in range(len(names))])
        acc /= iters
        hit = self.hit()
        el = self.W.el
        # algorithmic work of each entry point: its inputs read once (weights of the
        # experts hit), its outputs written once; the H and Y round trips between
        # the entry points are implementation traffic and are not counted
        work = {
            "route": (T * c.d * el + c.d * c.E * el + T * 16, 2.0 * T * c.d * c.E),
            "dispatch": (A * 4 + (c.E * 2 + 1) * 4 + A * 8, 0.0),
            "ffn_up": (hit * self.W.up_e + T * c.d * el, 2.0 * A * c.d * c.h * self.m),
            "ffn_down": (hit * self.W.down_e, 2.0 * A * c.h * c.d),
            "combine": (T * c.d * el + A * 8, 3.0 * T * c.d),
        }
        out = {}
        for nme, us in zip(names, acc):
            byt, flp = work[nme]
            sec = us * 1e-6
            out[nme] = {"us": round(float(us), 2), "GB_s": round(byt / sec / 1e9, 1),
                        "TFLOP_s": round(flp / sec / 1e12, 2), "hbm_frac": round(byt / sec / 1e9 / HBM_PEAK_GBS, 4),
                        "mfma_frac": round(flp / sec / 1e12 / MFMA_BF16_PEAK_TFS, 4), "bytes": int(byt),
                        "flops": flp}
        return out


# ---------------------------------------------------------------------------- roofline of the dominant kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gemm_up_mixtral_prefill_T4096_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_12_amd", "csrc", "ffn_gemm.hip")


def measured_traffic(entry):
    """HBM bytes per launch of the roofline kernel from the committed PMC summary,
    or None when there is none or the kernel source changed since it was taken."""
    try:
        text = open(TRAFFIC_FILE).read()
        src_sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != src_sha or fields.get("entry") != entry:
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def roofline(kern, key, T):
    """The first-layer grouped GEMM (entry point colibri_moe_expert_ffn_up; at the
    Mixtral prefill it launches ffn_gemm_kernel alone): algorithmic flops per
    launch over its average event time, against the bf16 MFMA peak when its
    intensity is above the ridge, else bytes against the HBM peak."""
    k = kern["ffn_up"]
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    sec = k["us"] * 1e-6
    if k["flops"] / k["bytes"] >= ridge:
        roof = {"bound": "mfma", "achieved": round(k["flops"] / sec / 1e12, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(k["bytes"] / sec / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    traffic = measured_traffic("ffn_up") if (key == "mixtral_prefill" and T == 4096) else None
    roof.update({"traffic": traffic, "kernel": "ffn_gemm_kernel (first layer: X W1 | X W3, SwiGLU epilogue)",
                 "entry": "ffn_up", "avg_launch_us": k["us"], "algorithmic_flops_per_launch": k["flops"],
                 "algorithmic_bytes_per_launch": k["bytes"]})
    return roof


# ---------------------------------------------------------------------------- extra workloads
def layer_record(L, T, us, np):
    hit = L.hit()
    med = float(np.median(us))
    return {"us_per_step": stats(us, np), "tokens_per_s": round(T / (med * 1e-6), 1), "experts_hit": hit,
            "hbm_frac": round(L.bytes(T, hit) / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(L.flops(T) / (med * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4)}


def decode_batches(g, gen, moe, cfg, W, Ts, iters):
    np = g.np
    L = Layer(g, gen, moe, cfg, W, max(Ts))
    rec = {}
    for T in Ts:
        us = g.per_step_us(lambda i: L.step(i, T), iters, 20)
        rec[f"T={T}"] = layer_record(L, T, us, np)
        log(f"{cfg.key} T={T}: {rec[f'T={T}']}")
    return rec, L


def quantized_decode(g, gen, moe, L, Ts, iters, rotate_gb, kind):
    """The decode batches with int8 (per-column) or 4-bit (group-128, zero point)
    expert weights, quantized on the GPU by the library's own quantizers and
    rotated like the bf16 weights; HBM fraction over the quantized bytes."""
    torch, np = g.torch, g.np
    cfg, W = L.cfg, L.W
    w0 = W[0]
    q0 = {"b1": w0["b1"], "b2": w0["b2"]}
    nbytes = lambda v: 0 if v is None else (sum(a.numel() * a.element_size() for a in v) if isinstance(v, tuple)
                                            else v.numel() * v.element_size())
    per_e = lambda v: 0 if v is None else (sum(a[0].numel() * a.element_size() for a in v) if isinstance(v, tuple)
                                           else v[0].numel() * v.element_size())
    for name in ("w1", "w3", "w2"):
        wt = w0[name]
        if wt is None:
            q0[name] = None
            continue
        E_, K_, N_ = wt.shape
        if kind == "int8":
            t = (torch.empty((E_, K_, N_), dtype=torch.int8, device=g.dev),
                 torch.empty((E_, N_), dtype=torch.float32, device=g.dev))
            moe.quantize_q8(wt, gen.BF16, E_, K_, N_, *t)
        else:
            t = (torch.empty((E_, K_ // 8, N_), dtype=torch.int32, device=g.dev),
                 torch.empty((E_, K_ // 128, N_), dtype=torch.float32, device=g.dev),
                 torch.empty((E_, K_ // 128, N_), dtype=torch.uint8, device=g.dev))
            moe.quantize_q4(wt, gen.BF16, E_, K_, N_, *t)
        q0[name] = t
    torch.cuda.synchronize()
    up_e = per_e(q0["w1"]) + per_e(q0["w3"]) + per_e(q0["b1"])
    down_e = per_e(q0["w2"]) + per_e(q0["b2"])
    layer_bytes = sum(nbytes(v) for v in q0.values())
    R = max(1, math.ceil(rotate_gb * 1e9 / layer_bytes))
    cl = lambda v: None if v is None else (tuple(a.clone() for a in v) if isinstance(v, tuple) else v.clone())
    copies = [q0] + [{k: cl(v) for k, v in q0.items()} for _ in range(R - 1)]
    log(f"{kind} weights: {R} copies x {layer_bytes / 1e6:.1f} MB")

    def step(i, T):
        w = copies[i % R]
        s = L.shape.with_T(T)
        if kind == "int8":
            (q1, s1), (q2, s2) = w["w1"], w["w2"]
            q3, s3 = w["w3"] if w["w3"] is not None else (None, None)
            moe.layer_forward_q8(s, L.x[:T], L.w_r, L.b_r, q1, s1, q2, s2, L.out[:T], L.ws, L.ws_bytes, q3=q3, s3=s3,
                                 b1=w["b1"], b2=w["b2"], counts=L.counts)
        else:
            moe.layer_forward_q4(s, L.x[:T], L.w_r, L.b_r, w["w1"], w["w2"], L.out[:T], L.ws, L.ws_bytes,
                                 w3q=w["w3"], b1=w["b1"], b2=w["b2"], counts=L.counts)

    rec = {}
    for T in Ts:
        us = g.per_step_us(lambda i: step(i, T), iters, 20)
        hit = L.hit()
        med = float(np.median(us))
        byt = hit * (up_e + down_e) + 2 * T * cfg.d * 2 + cfg.d * cfg.E * 2
        rec[f"T={T}"] = {"us_per_step": stats(us, np), "experts_hit": hit,
                         "hbm_frac": round(byt / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"{cfg.key} {kind} T={T}: {rec[f'T={T}']}")
    return rec


def ceilings(g, moe_pkg):
    """Achieved streaming-read bandwidth and bf16 MFMA rate of this chip."""
    torch, np = g.torch, g.np
    lib = ctypes.CDLL(os.path.join(os.path.dirname(moe_pkg.__file__), "libcolibri_ceilings.so"))
    lib.colibri_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                                ctypes.c_void_p]
    lib.colibri_ceiling_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.colibri_ceiling_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.colibri_ceiling_mfma_flops.restype = ctypes.c_double
    st = g.stream.cuda_stream
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=g.dev)
    blocks = 256 * 8
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=g.dev)
    us = g.per_step_us(lambda i: lib.colibri_ceiling_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, st),
                       10, 2, sync_every=5)
    read_gbs = nbytes / (float(np.median(us)) * 1e-6) / 1e9
    del buf
    mblocks, iters = 256 * 2, 4000  # two workgroups of 4 waves per CU: 2 waves per SIMD
    msink = torch.empty(mblocks * 256, dtype=torch.float32, device=g.dev)
    us = g.per_step_us(lambda i: lib.colibri_ceiling_mfma_loop(iters, msink.data_ptr(), mblocks, st), 10, 2,
                       sync_every=5)
    tfs = lib.colibri_ceiling_mfma_flops(iters, mblocks) / (float(np.median(us)) * 1e-6) / 1e12
    rec = {"stream_read_GB_s": round(read_gbs, 1), "stream_read_frac_of_spec": round(read_gbs / HBM_PEAK_GBS, 4),
           "stream_read_bytes": nbytes, "mfma_bf16_TFLOP_s": round(tfs, 1),
           "mfma_frac_of_spec": round(tfs / MFMA_BF16_PEAK_TFS, 4),
           "mfma_loop": f"{mblocks} workgroups x 4 waves x {iters} x 8 v_mfma_f32_32x32x16_bf16, register operands"}
    log(f"ceilings: {rec}")
    return rec


# ---------------------------------------------------------------------------- CPU oracle
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class HostLayer:
    """A workload's host tensors for the oracle (weights shared between the
    workloads that draw the same ones)."""
    _experts = {}

    def __init__(self, gen, key, T):
        self.cfg = gen.CONFIGS[key]
        self.x = gen.make_x(self.cfg, T)
        self.w_r, self.b_r = gen.make_router(self.cfg), gen.router_bias(self.cfg)
        wk = weight_key(gen, key)
        if wk not in HostLayer._experts:
            HostLayer._experts.clear()
            HostLayer._experts[wk] = gen.make_experts(self.cfg)
        self.w = HostLayer._experts[wk]


def time_oracle(np, hl, T, threads, seconds, chunk):
    """Tokens/s of the fp64 oracle over the whole layer (logits, top-2, gates,
    both expert rows, combine) for consecutive chunks of the T-token batch,
    repeated until about `seconds` have passed."""
    import oracle
    oracle.set_threads(threads)
    w = hl.w
    done, t0, start = 0, time.perf_counter(), 0
    while True:
        toks = np.arange(start, min(start + chunk, T))
        oracle.layer_tokens(hl.x, hl.w_r, w["w1"], w["w2"], hl.cfg.act, toks, b_r=hl.b_r, w3=w["w3"], b1=w["b1"],
                            b2=w["b2"], mirror=True)
        done += len(toks)
        start = (start + chunk) % T
        el = time.perf_counter() - t0
        if el >= seconds:
            return done, el


def cpu_baselines(gen, np, key, T, seconds, per_workload):
    """The oracle on the host cores: the headline workload on every core, and
    (per_workload) each workload once, one thread up to 64 tokens, every core
    beyond."""
    import oracle
    ncores = oracle.max_threads()
    model = cpu_model()
    done, el = time_oracle(np, HostLayer(gen, key, T), T, ncores, seconds, 32)
    head = {"value": round(done / el, 2), "unit": "tokens/s", "cores": ncores, "kind": "oracle",
            "sample": f"{done} of the {T} tokens of the timed batch (consecutive chunks of 32), whole layer in fp64; "
                      f"{el:.1f} s on {ncores} threads of {model}", "cpu_model": model, "nproc": os.cpu_count()}
    log(f"cpu oracle {key} T={T}: {head}")
    if not per_workload:
        return head, None
    per = {}
    for k, Ts in (("mixtral_decode", (1, 4, 16, 32)), ("tiny", (32,)), ("e8", (1, 64, 512)), ("skew16", (8192,))):
        for t in Ts:
            thr = 1 if t <= 64 else ncores
            d, e = time_oracle(np, HostLayer(gen, k, t), t, thr, 2.0, min(t, 32))
            per[f"{k} T={t}"] = {"tokens_per_s": round(d / e, 2), "us_per_token": round(e / d * 1e6, 1),
                                 "threads": thr, "tokens_timed": d}
    per["cpu_model"] = model
    per["nproc"] = os.cpu_count()
    HostLayer._experts.clear()
    oracle.set_threads(ncores)
    log(f"cpu oracle per workload: {per}")
    return head, per


# ---------------------------------------------------------------------------- layer variants, multi-layer step
def time_variants(g, gen, moe, rotate_gb):
    """GPU time per step of the 15 routed + 1 shared expert layer through
    colibri_moe_layer_forward_ex (softmax gating, shared expert, residual) and of
    the same routed layer through colibri_moe_layer_forward, at T = 1, 64, 512."""
    torch, np = g.torch, g.np
    cfg = gen.CONFIGS["shared15"]
    w0 = {k: g.to_dev(v) for k, v in gen.make_experts(cfg).items()}
    s0 = {k: g.to_dev(v) for k, v in gen.make_shared_expert(cfg).items()}
    Tmax = max(cfg.Ts)
    x = g.to_dev(gen.make_x(cfg, Tmax))
    res = g.to_dev(gen.make_residual(cfg, Tmax))
    w_r = g.to_dev(gen.make_router(cfg))
    el = 2
    routed_bytes = sum(v.numel() * el for v in w0.values() if v is not None)
    shared_bytes = sum(v.numel() * el for v in s0.values() if v is not None)
    R = max(1, math.ceil(rotate_gb * 1e9 / (routed_bytes + shared_bytes)))
    copies = [(w0, s0)] + [({k: (v.clone() if v is not None else None) for k, v in w0.items()},
                            {k: (v.clone() if v is not None else None) for k, v in s0.items()}) for _ in range(R - 1)]
    act = gen.ACT_CODE[cfg.act]
    up_e, down_e = 2 * cfg.d * cfg.h * el, cfg.h * cfg.d * el
    out = torch.empty((Tmax, cfg.d), dtype=torch.bfloat16, device=g.dev)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=g.dev)
    rec = {}
    for T in cfg.Ts:
        sh = moe.Shape(T, cfg.d, cfg.h, cfg.E, cfg.dtype, act)
        ws_ex = moe.workspace_size_ex(sh, gate="softmax", shared=s0, shared_h=cfg.shared_h, residual=res[:T])
        ws = torch.empty(max(ws_ex, moe.workspace_size(sh)), dtype=torch.uint8, device=g.dev)

        def step_ex(i):
            w, sw = copies[i % R]
            moe.layer_forward_ex(sh, x[:T], w_r, None, w["w1"], w["w2"], out[:T], ws, w3=w["w3"], gate="softmax",
                                 shared=sw, shared_h=cfg.shared_h, residual=res[:T], counts=counts)

        def step_plain(i):
            w, _ = copies[i % R]
            moe.layer_forward(sh, x[:T], w_r, None, w["w1"], w["w2"], out[:T], ws, w3=w["w3"], counts=counts)

        for name, fn, extra in (("softmax+shared+residual", step_ex, shared_bytes + T * cfg.d * el),
                                ("plain", step_plain, 0)):
            us = g.per_step_us(fn, 200 if T <= 64 else 60, 10)
            med = float(np.median(us))
            hit = int((counts.cpu().numpy() > 0).sum())
            byt = hit * (up_e + down_e) + extra + 2 * T * cfg.d * el
            rec[f"{name} T={T}"] = {"us_per_step": stats(us, np), "tokens_per_s": round(T / (med * 1e-6), 1),
                                    "experts_hit": hit, "hbm_frac": round(byt / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"variant {name} T={T}: {rec[f'{name} T={T}']}")
    rec["workload"] = (f"{cfg.title}: E={cfg.E} routed + 1 shared (h_shared={cfg.shared_h}), top-2, d={cfg.d}, "
                       f"h={cfg.h}, {cfg.act}, bf16")
    return rec


def time_steps(g, gen, moe, L):
    """A decode step through L layers (x <- layer_l(x) + x, each layer with its
    own weights), launched eagerly (colibri_moe_step_forward) and replayed as one
    HIP graph (colibri_moe_graph_*): GPU time per step (median) and the
    host-inclusive time of back-to-back steps."""
    torch, np = g.torch, g.np
    rec = {}
    for key, Ts, shared in (("e8", (1, 64), False), ("shared15", (1, 64), True)):
        cfg = gen.CONFIGS[key]
        layers, wbytes = [], []
        for l in range(L):
            c = gen.layer_of(cfg, l)
            d = {k: g.to_dev(v) for k, v in gen.make_experts(c).items()}
            d["w_r"] = g.to_dev(gen.make_router(c))
            d["gate"] = "softmax" if shared else "pair"
            eb = sum(v[0].numel() * v.element_size() for k, v in d.items()
                     if k in ("w1", "w3", "w2", "b1", "b2") and v is not None)
            sb = 0
            if shared:
                d["shared"] = {k: g.to_dev(v) for k, v in gen.make_shared_expert(c).items()}
                d["shared_h"] = cfg.shared_h
                sb = sum(v.numel() * v.element_size() for v in d["shared"].values() if v is not None)
            layers.append(d)
            wbytes.append((eb, sb))
        act = gen.ACT_CODE[cfg.act]
        for T in Ts:
            sh = moe.Shape(T, cfg.d, cfg.h, cfg.E, cfg.dtype, act)
            ws = torch.empty(moe.step_workspace_size(sh, layers), dtype=torch.uint8, device=g.dev)
            x0 = g.to_dev(gen.make_x(cfg, T))
            x = x0.clone()
            gr = moe.Graph(sh, layers, x, ws, residual=True)
            out = {}
            for name, fn in (("eager", lambda: moe.step_forward(sh, layers, x, ws, residual=True)),
                             ("graph", lambda: gr.launch())):
                def one(i):
                    x.copy_(x0)
                    fn()
                us = g.per_step_us(one, 100, 10)
                h0 = time.perf_counter()
                for _ in range(100):
                    fn()
                torch.cuda.synchronize()
                host_us = (time.perf_counter() - h0) / 100 * 1e6
                med = float(np.median(us))
                out[name] = {"us_per_step_median": round(med, 1), "us_per_layer": round(med / L, 2),
                             "us_per_step_host_inclusive": round(host_us, 1)}
            gr.destroy()
            routed_e = min(cfg.E, 2 * T)
            byt = sum(routed_e * eb + sb for eb, sb in wbytes)
            for v in out.values():
                v["hbm_frac_weights"] = round(byt / (v["us_per_step_median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            rec[f"{key} L={L} T={T}"] = out
            log(f"step {key} L={L} T={T}: {out}")
    rec["workload"] = (f"{L} layers in place with residual, each with its own weights: the 8-expert 1.3B-class "
                       f"layer (pair gating), and the 15 routed + 1 shared expert layer (softmax gating; in the "
                       f"graph each layer's shared expert runs on a parallel branch)")
    return rec


# ---------------------------------------------------------------------------- main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the layer on one GPU only; this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import mixture_experts_layer_12_amd as moe

    moe.load(build_if_missing=True)
    g = Gpu(torch, np)
    key = args.config
    cfg = gen.CONFIGS[key]
    T = args.T or max(cfg.Ts)
    rings = {}

    def ring(k):
        wk = weight_key(gen, k)
        if wk not in rings:
            rings[wk] = Weights(g, gen, gen.CONFIGS[k], args.rotate_gb)
        return rings[wk]

    # ------------------------------------------------------------ the timed region: K steps of the headline layer
    L = Layer(g, gen, moe, cfg, ring(key), T)
    for i in range(args.warmup):
        L.step(i, T)
    torch.cuda.synchronize()
    ev0, ev1 = g.event(), g.event()
    step_ev = [(g.event(), g.event()) for _ in range(args.steps)]
    g.prefill_queue()
    ev0.record(g.stream)
    for i in range(args.steps):
        step_ev[i][0].record(g.stream)
        L.step(i, T)
        step_ev[i][1].record(g.stream)
    ev1.record(g.stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tok_s = T / (ms_per_step * 1e-3)
    step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in step_ev])
    hit = L.hit()
    log(f"layer: {ms_per_step * 1e3:.1f} us/step, {tok_s / 1e6:.3f} M tokens/s, experts hit {hit}/{cfg.E}")

    kern = L.entry_points(T, max(args.steps, 20), 3)
    log(f"entry points: {json.dumps(kern)}")
    roof = roofline(kern, key, T)

    if args.copy_mb:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=g.dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_mb} MiB")
        del src, dst

    rec = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == gen.BF16 else "f32",
        "data": "synthetic (seeded Philox normals; random-init weights of the layer's shape)",
        "config": {"workload": f"{cfg.title}: E={cfg.E}, top-2, d={cfg.d}, h={cfg.h}, {cfg.act}, T={T}",
                   "T": T, "E": cfg.E, "d": cfg.d, "h": cfg.h, "act": cfg.act, "weight_copies": L.W.R,
                   "experts_hit": hit},
        "us_per_step": stats(step_us, np),
        "layer_mfma_frac": round(L.flops(T) / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        "layer_tflop_s": round(L.flops(T) / (ms_per_step * 1e-3) / 1e12, 1),
        "roofline": roof, "cpu_baseline": None, "kernels": kern,
    }

    if not args.headline_only:
        # Mixtral-shaped decode (the same expert weights as the prefill workload)
        dcfg = gen.CONFIGS["mixtral_decode"]
        rec["decode"], DL = decode_batches(g, gen, moe, dcfg, ring("mixtral_decode"), (1, 4, 16, 32),
                                           args.decode_iters)
        rec["decode"]["workload"] = f"{dcfg.title}: E={dcfg.E}, d={dcfg.d}, h={dcfg.h}, {dcfg.act}, bf16"
        if not args.no_quantized:
            rec["decode_int8_weights"] = quantized_decode(g, gen, moe, DL, (1, 4, 16, 32), args.decode_iters,
                                                          args.rotate_gb, "int8")
            rec["decode_int4_weights"] = quantized_decode(g, gen, moe, DL, (1, 4, 16, 32), args.decode_iters,
                                                          args.rotate_gb, "int4")
        del DL
        rings.clear()
        del L
        torch.cuda.empty_cache()
        # 16-expert Zipf-skewed prefill
        scfg = gen.CONFIGS["skew16"]
        SL = Layer(g, gen, moe, scfg, ring("skew16"), 8192)
        us = g.per_step_us(lambda i: SL.step(i, 8192), args.steps, args.warmup)
        rec["skew16"] = layer_record(SL, 8192, us, np)
        rec["skew16"]["kernels"] = SL.entry_points(8192, 20, 3)
        rec["skew16"]["counts"] = SL.counts.cpu().numpy().tolist()
        rec["skew16"]["workload"] = f"{scfg.title}: E={scfg.E}, d={scfg.d}, h={scfg.h}, {scfg.act}, T=8192"
        log(f"skew16: {rec['skew16']}")
        del SL
        rings.clear()
        torch.cuda.empty_cache()
        # 8-expert 1.3B-class layer
        ecfg = gen.CONFIGS["e8"]
        rec["e8"], EL = decode_batches(g, gen, moe, ecfg, ring("e8"), (1, 64, 512), args.decode_iters)
        rec["e8"]["T=512"]["kernels"] = EL.entry_points(512, 50, 3)
        rec["e8"]["workload"] = f"{ecfg.title}: E={ecfg.E}, d={ecfg.d}, h={ecfg.h}, {ecfg.act} + biases, bf16"
        del EL
        rings.clear()
        torch.cuda.empty_cache()
        # tiny fp32 layer: launch-latency bound (its 0.27 MB of weights stay in cache), so one weight copy
        tcfg = gen.CONFIGS["tiny"]
        rec["tiny"], TL = decode_batches(g, gen, moe, tcfg, Weights(g, gen, tcfg, 0.0), (32,), args.decode_iters)
        rec["tiny"]["T=32"].pop("mfma_frac", None)
        rec["tiny"]["T=32"].pop("hbm_frac", None)
        rec["tiny"]["workload"] = (f"{tcfg.title}: E={tcfg.E}, d={tcfg.d}, h={tcfg.h}, {tcfg.act} + biases, fp32 "
                                   "(launch-latency bound; one weight copy)")
        del TL
        torch.cuda.empty_cache()
        if not args.no_variants:
            rec["variants"] = time_variants(g, gen, moe, args.rotate_gb)
            torch.cuda.empty_cache()
        if args.step_layers > 0:
            rec["multi_layer_step"] = time_steps(g, gen, moe, args.step_layers)
            torch.cuda.empty_cache()
        rec["ceilings"] = ceilings(g, moe)

    if not args.no_cpu_baseline:
        head, per = cpu_baselines(gen, np, key, T, args.cpu_seconds, not args.headline_only)
        rec["cpu_baseline"] = head
        if per is not None:
            rec["cpu_oracle_per_workload"] = per
    rec["timing"] = ("GPU time (HIP events on the library's stream, queue pre-filled by a spin kernel)"
                     if g.can_sleep else "GPU time (HIP events)")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
