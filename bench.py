#!/usr/bin/env python3
"""Benchmark of the MoE layer forward pass on one MI355X.

Default workload: the 8-expert 1.3B-class layer (E=8, d=2048, h=5632, GELU
experts with biases, bf16 storage, fp32 accumulation) on a T=512-token batch;
one step = one colibri_moe_layer_forward (route, dispatch, grouped expert FFN,
combine) over the batch.  Inputs are seeded synthetic tensors already resident
in HBM; expert weights rotate over enough identical copies (>= 2 GB) that the
256 MB MALL cannot serve them from cache.

Timing is GPU time from HIP events on the stream the kernels run on.  Before
each timed region a spin kernel keeps the GPU busy while the host enqueues
the work, so host launch latency does not show up as GPU idle time inside the
region (decode steps are also reported host-inclusive, back to back).

Prints one JSON line: whole-layer tokens/s, the roofline fraction of the
dominant kernel, every kernel's time and fraction, decode microseconds per
step at T=1 and T=64 with bf16 expert weights, with per-column int8 expert
weights (colibri_moe_layer_forward_q8) and with 4-bit group-128 weights
(colibri_moe_layer_forward_q4), both quantized on the GPU by the library's
own quantizers, and the fp64 CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="e8", help="workload key in gen.CONFIGS")
    ap.add_argument("--T", type=int, default=None, help="tokens per step (default: the config's largest T)")
    ap.add_argument("--rotate-gb", type=float, default=2.0, help="total bytes of rotated weight copies")
    ap.add_argument("--decode-T", default="1,64", help="decode batch sizes also timed (comma list, '' = none)")
    ap.add_argument("--decode-iters", type=int, default=200)
    ap.add_argument("--no-q8", action="store_true", help="skip the int8- and 4-bit-weight decode lines")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the shared-expert / softmax-gating / residual layer lines")
    ap.add_argument("--step-layers", type=int, default=8,
                    help="layers of the multi-layer decode step timed eagerly and as a HIP graph (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens in the oracle's timed sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="repeat the oracle sample for about this long")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (calibrates PMC byte counters)")
    return ap.parse_args()


# Kernel that each timed entry point launches for the default workload (8-expert
# layer, T=512: the first layer's K is not split, so one GEMM launch).
ENTRY_KERNEL = {"route": "route_kernel", "dispatch": "dispatch_kernel",
                "ffn_up": "ffn_gemm_kernel (first layer: X W1, GELU epilogue)",
                "ffn_down": "ffn_gemm_kernel (second layer, K split) + split_reduce_kernel",
                "combine": "combine_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gemm_up_e8_T512_traffic.md")
TRAFFIC_SOURCE = os.path.join(ROOT, "mixture_experts_layer_12_amd", "csrc", "ffn_gemm.hip")


def measured_traffic(kernel_key):
    """HBM bytes per launch of the roofline kernel from the committed PMC summary,
    or None when there is none or the kernel source changed since it was taken."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        src_sha = hashlib.sha256(open(TRAFFIC_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != src_sha or fields.get("entry") != kernel_key:
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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
    cfg = gen.CONFIGS[args.config]
    T = args.T or max(cfg.Ts)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    can_sleep = hasattr(torch.cuda, "_sleep")

    def prefill_queue():
        if can_sleep:
            torch.cuda._sleep(SLEEP_CYCLES)

    def to_dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    t0 = time.time()
    hw = gen.make_experts(cfg)
    x_np = gen.make_x(cfg, T)
    w_r_np = gen.make_router(cfg)
    b_r_np = gen.router_bias(cfg)
    log(f"generated inputs in {time.time() - t0:.1f}s")
    dw0 = {k: to_dev(v) for k, v in hw.items()}
    del hw
    x = to_dev(x_np)
    w_r = to_dev(w_r_np)
    b_r = to_dev(b_r_np)
    el = 4 if cfg.dtype == gen.F32 else 2
    per_expert = {k: (v[0].numel() * el if v is not None else 0) for k, v in dw0.items()}
    up_bytes_e = per_expert["w1"] + per_expert["w3"] + per_expert["b1"]
    down_bytes_e = per_expert["w2"] + per_expert["b2"]
    layer_w_bytes = sum(v.numel() * el for v in dw0.values() if v is not None)
    R = max(1, math.ceil(args.rotate_gb * 1e9 / layer_w_bytes))
    copies = [dw0] + [{k: (v.clone() if v is not None else None) for k, v in dw0.items()} for _ in range(R - 1)]
    log(f"{R} weight copies x {layer_w_bytes / 1e6:.1f} MB")

    act = gen.ACT_CODE[cfg.act]
    m = 2 if cfg.act == "swiglu" else 1
    sh = moe.Shape(T, cfg.d, cfg.h, cfg.E, cfg.dtype, act)
    ws_bytes = moe.workspace_size(sh)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    tdt = torch.float32 if cfg.dtype == gen.F32 else torch.bfloat16
    out = torch.empty((T, cfg.d), dtype=tdt, device=dev)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)

    def step(i, xx=x, s=sh, o=out):
        w = copies[i % R]
        moe.layer_forward(s, xx, w_r, b_r, w["w1"], w["w2"], o, ws, ws_bytes, w3=w["w3"], b1=w["b1"], b2=w["b2"],
                          counts=counts)

    # ---------------------------------------------------------------- whole layer (the timed region)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    prefill_queue()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tok_s = T / (ms_per_step * 1e-3)
    cnt = counts.cpu().numpy()
    hit = int((cnt > 0).sum())
    log(f"layer: {ms_per_step * 1e3:.1f} us/step, {tok_s / 1e6:.3f} M tokens/s, experts hit {hit}/{cfg.E}")

    # ---------------------------------------------------------------- per-kernel durations (same workload)
    A = 2 * T
    idx = torch.empty((T, 2), dtype=torch.int32, device=dev)
    gate = torch.empty((T, 2), dtype=torch.float32, device=dev)
    offs = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    sa = torch.empty(A, dtype=torch.int32, device=dev)
    ap_ = torch.empty(A, dtype=torch.int32, device=dev)
    H = torch.empty((A, cfg.h), dtype=tdt, device=dev)
    y = torch.empty((A, cfg.d), dtype=tdt, device=dev)
    names = ("route", "dispatch", "ffn_up", "ffn_down", "combine")
    kern_ms = np.zeros(len(names))
    iters = max(args.steps, 20)
    for it in range(args.warmup + iters):
        w = copies[it % R]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        prefill_queue()
        evs[0].record(stream)
        moe.route(sh, x, w_r, b_r, idx, gate)
        evs[1].record(stream)
        moe.dispatch(sh, idx, counts, offs, sa, ap_, ws=ws, ws_bytes=ws_bytes)
        evs[2].record(stream)
        moe.expert_ffn_up(sh, x, sa, offs, w["w1"], H, ws, ws_bytes, w3=w["w3"], b1=w["b1"])
        evs[3].record(stream)
        moe.expert_ffn_down(sh, H, offs, w["w2"], y, ws, ws_bytes, b2=w["b2"])
        evs[4].record(stream)
        moe.combine(sh, y, ap_, gate, out)
        evs[5].record(stream)
        torch.cuda.synchronize()
        if it >= args.warmup:
            kern_ms += np.array([evs[j].elapsed_time(evs[j + 1]) for j in range(len(names))])
    kern_ms /= iters

    # algorithmic work per launch: weights of the experts hit, read once; each
    # kernel's own inputs read once and outputs written once
    s_ = el
    work = {
        "route": (T * cfg.d * s_ + cfg.d * cfg.E * s_ + T * 16, 2.0 * T * cfg.d * cfg.E),
        "dispatch": (A * 4 + (cfg.E * 2 + 1) * 4 + A * 8, 0.0),
        "ffn_up": (hit * up_bytes_e + T * cfg.d * s_ + A * cfg.h * s_, 2.0 * A * cfg.d * cfg.h * m),
        "ffn_down": (hit * down_bytes_e + A * cfg.h * s_ + A * cfg.d * s_, 2.0 * A * cfg.h * cfg.d),
        "combine": (A * cfg.d * s_ + T * cfg.d * s_ + A * 4 + A * 4, 3.0 * T * cfg.d),
    }
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    kernels = {}
    for nme, ms_ in zip(names, kern_ms):
        byt, flp = work[nme]
        sec = ms_ * 1e-3
        kernels[nme] = {"us": round(ms_ * 1e3, 2), "GB_s": round(byt / sec / 1e9, 1),
                        "TFLOP_s": round(flp / sec / 1e12, 2), "hbm_frac": round(byt / sec / 1e9 / HBM_PEAK_GBS, 4),
                        "mfma_frac": round(flp / sec / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                        "bytes": int(byt), "flops": flp}
    log(f"kernels: {json.dumps(kernels)}")
    # roofline of the dominant single-kernel entry point
    single = [k for k in kernels if "+" not in ENTRY_KERNEL[k]]
    dom = max(single, key=lambda k: kernels[k]["us"])
    byt, flp = work[dom]
    sec = kernels[dom]["us"] * 1e-6
    if flp / byt < ridge:
        roof = {"bound": "hbm", "achieved": round(byt / sec / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flp / sec / 1e12, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    traffic = measured_traffic(dom) if (args.config == "e8" and T == 512) else None
    roof.update({"traffic": traffic, "kernel": ENTRY_KERNEL[dom], "entry": dom, "avg_launch_us": kernels[dom]["us"],
                 "algorithmic_bytes_per_launch": int(byt), "algorithmic_flops_per_launch": flp})

    if args.copy_mb:
        src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_mb} MiB")

    # ---------------------------------------------------------------- decode sizes
    def time_decode(step_fn, tok):
        """GPU-time median/min/p90 (spin kernel in front every 10 steps) and the
        host-inclusive time of back-to-back steps, in us."""
        s2 = sh.with_T(tok)
        xd, od = x[:tok], out[:tok]
        times = []
        for it in range(20 + args.decode_iters):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            if it % 10 == 0:
                prefill_queue()
            e0.record(stream)
            step_fn(it, xx=xd, s=s2, o=od)
            e1.record(stream)
            if it % 10 == 9:
                torch.cuda.synchronize()
            if it >= 20:
                times.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in times])
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for it in range(args.decode_iters):
            step_fn(it, xx=xd, s=s2, o=od)
        torch.cuda.synchronize()
        host_us = (time.perf_counter() - h0) / args.decode_iters * 1e6
        return float(np.median(us)), float(us.min()), float(np.percentile(us, 90)), host_us

    def decode_record(tok, med, umin, p90, host_us, up_e, down_e):
        hit2 = int((counts.cpu().numpy() > 0).sum())
        byt2 = hit2 * (up_e + down_e) + tok * cfg.d * s_ * 2 + cfg.d * cfg.E * s_
        return {"us_per_step_median": round(med, 2), "us_min": round(umin, 2), "us_p90": round(p90, 2),
                "us_per_step_host_inclusive": round(host_us, 2), "experts_hit": hit2,
                "hbm_frac": round(byt2 / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    decode_ts = [int(v) for v in args.decode_T.split(",") if v.strip() and int(v) <= T]
    decode = {}
    for tok in decode_ts:
        decode[f"T={tok}"] = decode_record(tok, *time_decode(step, tok), up_bytes_e, down_bytes_e)
        log(f"decode T={tok}: {decode[f'T={tok}']}")

    # int8 expert weights (per-column scales), decode sizes only: quantized on the
    # GPU by the library's own quantizer, rotated like the bf16 weights
    decode_q8 = {}
    q8_ts = [t for t in decode_ts if t <= 64]
    if q8_ts and cfg.dtype == gen.BF16 and not args.no_q8:
        q0 = {"b1": dw0["b1"], "b2": dw0["b2"]}
        for name, qn, sn in (("w1", "q1", "s1"), ("w3", "q3", "s3"), ("w2", "q2", "s2")):
            wt = dw0[name]
            if wt is None:
                q0[qn] = q0[sn] = None
                continue
            E_, K_, N_ = wt.shape
            q0[qn] = torch.empty((E_, K_, N_), dtype=torch.int8, device=dev)
            q0[sn] = torch.empty((E_, N_), dtype=torch.float32, device=dev)
            moe.quantize_q8(wt, gen.BF16, E_, K_, N_, q0[qn], q0[sn])
        torch.cuda.synchronize()
        qb = {k: (v[0].numel() * v.element_size() if v is not None else 0) for k, v in q0.items()}
        up_q8_e = qb["q1"] + qb["q3"] + qb["s1"] + qb["s3"] + qb["b1"]
        down_q8_e = qb["q2"] + qb["s2"] + qb["b2"]
        q8_layer_bytes = sum(v.numel() * v.element_size() for v in q0.values() if v is not None)
        R8 = max(1, math.ceil(args.rotate_gb * 1e9 / q8_layer_bytes))
        qcopies = [q0] + [{k: (v.clone() if v is not None else None) for k, v in q0.items()} for _ in range(R8 - 1)]
        log(f"int8 weights: {R8} copies x {q8_layer_bytes / 1e6:.1f} MB")

        def step_q8(i, xx=x, s=sh, o=out):
            w = qcopies[i % R8]
            moe.layer_forward_q8(s, xx, w_r, b_r, w["q1"], w["s1"], w["q2"], w["s2"], o, ws, ws_bytes, q3=w["q3"],
                                 s3=w["s3"], b1=w["b1"], b2=w["b2"], counts=counts)

        for tok in q8_ts:
            decode_q8[f"T={tok}"] = decode_record(tok, *time_decode(step_q8, tok), up_q8_e, down_q8_e)
            log(f"decode int8 weights T={tok}: {decode_q8[f'T={tok}']}")
        del qcopies, q0

    # 4-bit expert weights (zero point, groups of 128 input channels), decode
    # sizes only: quantized on the GPU by the library's own quantizer, rotated
    # like the bf16 weights
    decode_q4 = {}
    if q8_ts and cfg.dtype == gen.BF16 and not args.no_q8 and cfg.d % 128 == 0 and cfg.h % 128 == 0:
        q0 = {"b1": dw0["b1"], "b2": dw0["b2"]}
        for name in ("w1", "w3", "w2"):
            wt = dw0[name]
            if wt is None:
                q0[name + "q"] = None
                continue
            E_, K_, N_ = wt.shape
            t = (torch.empty((E_, K_ // 8, N_), dtype=torch.int32, device=dev),
                 torch.empty((E_, K_ // 128, N_), dtype=torch.float32, device=dev),
                 torch.empty((E_, K_ // 128, N_), dtype=torch.uint8, device=dev))
            moe.quantize_q4(wt, gen.BF16, E_, K_, N_, *t)
            q0[name + "q"] = t
        torch.cuda.synchronize()
        nb = lambda v: 0 if v is None else (sum(a[0].numel() * a.element_size() for a in v) if isinstance(v, tuple)
                                            else v[0].numel() * v.element_size())
        up_q4_e = nb(q0["w1q"]) + nb(q0["w3q"]) + nb(q0["b1"])
        down_q4_e = nb(q0["w2q"]) + nb(q0["b2"])
        tb = lambda v: 0 if v is None else (sum(a.numel() * a.element_size() for a in v) if isinstance(v, tuple)
                                            else v.numel() * v.element_size())
        q4_layer_bytes = sum(tb(v) for v in q0.values())
        R4 = max(1, math.ceil(args.rotate_gb * 1e9 / q4_layer_bytes))
        cl = lambda v: None if v is None else (tuple(a.clone() for a in v) if isinstance(v, tuple) else v.clone())
        q4copies = [q0] + [{k: cl(v) for k, v in q0.items()} for _ in range(R4 - 1)]
        log(f"4-bit weights: {R4} copies x {q4_layer_bytes / 1e6:.1f} MB")

        def step_q4(i, xx=x, s=sh, o=out):
            w = q4copies[i % R4]
            moe.layer_forward_q4(s, xx, w_r, b_r, w["w1q"], w["w2q"], o, ws, ws_bytes, w3q=w["w3q"], b1=w["b1"],
                                 b2=w["b2"], counts=counts)

        for tok in q8_ts:
            decode_q4[f"T={tok}"] = decode_record(tok, *time_decode(step_q4, tok), up_q4_e, down_q4_e)
            log(f"decode 4-bit weights T={tok}: {decode_q4[f'T={tok}']}")
        del q4copies, q0

    # ---------------------------------------------------------------- layer variants
    # 15 routed + 1 shared expert, softmax over all experts (unnormalised pair),
    # residual added in the combine; beside it the same routed layer without the
    # shared expert and residual, pair gating, to show what the options cost
    variants = {}
    if not args.no_variants:
        variants = time_variants(args, moe, gen, torch, np, to_dev, stream, prefill_queue)

    # ---------------------------------------------------------------- multi-layer decode step
    steps = {}
    if args.step_layers > 0:
        steps = time_steps(args, moe, gen, torch, np, to_dev, stream, prefill_queue)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = args.cpu_sample or T
        toks = np.arange(min(n, T))
        w_host = gen.make_experts(cfg)
        reps = 0
        c0 = time.perf_counter()
        while True:
            oracle.layer_tokens(x_np, w_r_np, w_host["w1"], w_host["w2"], cfg.act, toks, b_r=b_r_np, w3=w_host["w3"],
                                b1=w_host["b1"], b2=w_host["b2"], mirror=True)
            reps += 1
            el_s = time.perf_counter() - c0
            if el_s >= args.cpu_seconds or el_s * (reps + 1) / reps > 30.0:
                break
        cpu = {"value": round(reps * len(toks) / el_s, 2), "unit": "tokens/s", "cores": oracle.max_threads(),
               "kind": "oracle", "seconds": round(el_s, 2),
               "sample": f"{reps} x {len(toks)} of the {T} tokens of the timed batch, whole layer (fp64 logits, "
                         f"top-2, gates, two expert FFN rows per token, combine)"}
        log(f"cpu oracle: {cpu}")

    rec = {
        "metric": "MoE-layer tokens/s (prefill) + \u00b5s/step (decode); % of MFMA / HBM peak",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == gen.BF16 else "f32", "data": "synthetic (seeded Philox normals)",
        "config": {"workload": f"{cfg.title}: E={cfg.E}, top-2, d={cfg.d}, h={cfg.h}, {cfg.act}, T={T}",
                   "T": T, "E": cfg.E, "d": cfg.d, "h": cfg.h, "act": cfg.act, "weight_copies": R,
                   "experts_hit": hit},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels, "decode": decode, "decode_int8_weights": decode_q8,
        "decode_int4_weights": decode_q4,
        "variants": variants, "multi_layer_step": steps,
        "timing": "GPU time (HIP events, queue pre-filled by a spin kernel)" if can_sleep else "GPU time (HIP events)",
    }
    print(json.dumps(rec), flush=True)


def time_variants(args, moe, gen, torch, np, to_dev, stream, prefill_queue):
    """GPU time per step of the 15 + 1 shared-expert layer through
    colibri_moe_layer_forward_ex (softmax gating, shared expert, residual) and of
    the same routed layer through colibri_moe_layer_forward, at T = 1, 64, 512.
    Weights rotate over copies (as in the main measurement) so that no step
    finds them in the last-level cache."""
    cfg = gen.CONFIGS["shared15"]
    dev = torch.device("cuda:0")
    t0 = time.time()
    w0 = {k: to_dev(v) for k, v in gen.make_experts(cfg).items()}
    s0 = {k: to_dev(v) for k, v in gen.make_shared_expert(cfg).items()}
    Tmax = max(cfg.Ts)
    x = to_dev(gen.make_x(cfg, Tmax))
    res = to_dev(gen.make_residual(cfg, Tmax))
    w_r = to_dev(gen.make_router(cfg))
    el = 2
    routed_bytes = sum(v.numel() * el for v in w0.values() if v is not None)
    shared_bytes = sum(v.numel() * el for v in s0.values() if v is not None)
    R = max(1, math.ceil(args.rotate_gb * 1e9 / (routed_bytes + shared_bytes)))
    copies = [(w0, s0)] + [({k: (v.clone() if v is not None else None) for k, v in w0.items()},
                            {k: (v.clone() if v is not None else None) for k, v in s0.items()}) for _ in range(R - 1)]
    log(f"variants: shared15 inputs in {time.time() - t0:.1f}s, {R} weight copies")
    act = gen.ACT_CODE[cfg.act]
    up_e = 2 * cfg.d * cfg.h * el
    down_e = cfg.h * cfg.d * el
    out = torch.empty((Tmax, cfg.d), dtype=torch.bfloat16, device=dev)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    rec = {}
    for T in cfg.Ts:
        sh = moe.Shape(T, cfg.d, cfg.h, cfg.E, cfg.dtype, act)
        ws_ex = moe.workspace_size_ex(sh, gate="softmax", shared=s0, shared_h=cfg.shared_h, residual=res)
        ws_pl = moe.workspace_size(sh)
        ws = torch.empty(max(ws_ex, ws_pl), dtype=torch.uint8, device=dev)

        def step_ex(i):
            w, sw = copies[i % R]
            moe.layer_forward_ex(sh, x[:T], w_r, None, w["w1"], w["w2"], out[:T], ws, ws_ex, w3=w["w3"], gate="softmax",
                                 shared=sw, shared_h=cfg.shared_h, residual=res[:T], counts=counts)

        def step_plain(i):
            w, _ = copies[i % R]
            moe.layer_forward(sh, x[:T], w_r, None, w["w1"], w["w2"], out[:T], ws, ws_pl, w3=w["w3"], counts=counts)

        for name, fn, extra in (("softmax+shared+residual", step_ex, shared_bytes + T * cfg.d * el),
                                ("plain", step_plain, 0)):
            iters = 200 if T <= 64 else 60
            times = []
            for it in range(10 + iters):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                if it % 10 == 0:
                    prefill_queue()
                e0.record(stream)
                fn(it)
                e1.record(stream)
                if it % 10 == 9:
                    torch.cuda.synchronize()
                if it >= 10:
                    times.append((e0, e1))
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in times]))
            hit = int((counts.cpu().numpy() > 0).sum())
            byt = hit * (up_e + down_e) + extra + 2 * T * cfg.d * el
            rec[f"{name} T={T}"] = {"us_per_step_median": round(us, 2), "tokens_per_s": round(T / (us * 1e-6), 1),
                                    "experts_hit": hit, "hbm_frac": round(byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"variant {name} T={T}: {rec[f'{name} T={T}']}")
    rec["workload"] = (f"{cfg.title}: E={cfg.E} routed + 1 shared (h_shared={cfg.shared_h}), top-2, d={cfg.d}, "
                       f"h={cfg.h}, {cfg.act}, bf16")
    del copies
    return rec


def time_steps(args, moe, gen, torch, np, to_dev, stream, prefill_queue):
    """A decode step through L layers (x <- layer_l(x) + x, each layer with its
    own weights), launched eagerly (colibri_moe_step_forward) and replayed as
    one HIP graph (colibri_moe_graph_*): GPU time per step (median) and the
    host-inclusive time of back-to-back steps.  L layers of distinct weights
    (several GB) keep every step's weights out of the last-level cache."""
    L = args.step_layers
    rec = {}
    for key, Ts, shared in (("e8", (1, 64), False), ("shared15", (1, 64), True)):
        cfg = gen.CONFIGS[key]
        layers, wbytes = [], []
        for l in range(L):
            c = gen.layer_of(cfg, l)
            d = {k: to_dev(v) for k, v in gen.make_experts(c).items()}
            d["w_r"] = to_dev(gen.make_router(c))
            d["gate"] = "softmax" if shared else "pair"
            eb = {k: (v[0].numel() * v.element_size() if v is not None else 0) for k, v in d.items()
                  if k in ("w1", "w3", "w2", "b1", "b2")}
            sb = 0
            if shared:
                d["shared"] = {k: to_dev(v) for k, v in gen.make_shared_expert(c).items()}
                d["shared_h"] = cfg.shared_h
                sb = sum(v.numel() * v.element_size() for v in d["shared"].values() if v is not None)
            layers.append(d)
            wbytes.append((sum(eb.values()), sb))
        act = gen.ACT_CODE[cfg.act]
        for T in Ts:
            sh = moe.Shape(T, cfg.d, cfg.h, cfg.E, cfg.dtype, act)
            ws_bytes = moe.step_workspace_size(sh, layers)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
            x0 = to_dev(gen.make_x(cfg, T))
            x = x0.clone()
            g = moe.Graph(sh, layers, x, ws, ws_bytes, residual=True)
            out = {}
            for name, fn in (("eager", lambda: moe.step_forward(sh, layers, x, ws, ws_bytes, residual=True)),
                             ("graph", lambda: g.launch())):
                times = []
                iters = 100
                for it in range(10 + iters):
                    x.copy_(x0)
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    if it % 10 == 0:
                        prefill_queue()
                    e0.record(stream)
                    fn()
                    e1.record(stream)
                    if it % 10 == 9:
                        torch.cuda.synchronize()
                    if it >= 10:
                        times.append((e0, e1))
                torch.cuda.synchronize()
                us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in times]))
                h0 = time.perf_counter()
                for it in range(iters):
                    fn()
                torch.cuda.synchronize()
                host_us = (time.perf_counter() - h0) / iters * 1e6
                out[name] = {"us_per_step_median": round(us, 1), "us_per_layer": round(us / L, 2),
                             "us_per_step_host_inclusive": round(host_us, 1)}
            g.destroy()
            # weights of the experts a step reads: at T = 1 two per layer, at 64 every one (seeded routing)
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


if __name__ == "__main__":
    main()
