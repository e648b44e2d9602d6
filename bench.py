#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer forward on one MI355X.

A step is one forward of one layer (router -> top-k -> grouping by expert ->
gate/up + SwiGLU -> down -> combine) for one batch of seeded synthetic tokens.
Steps walk through a stack of distinct seeded layers, so that the experts a step
reads were last read hundreds of MB earlier and are not served from the 256 MB
Infinity Cache; every input is resident (in HBM, or for offloaded experts in
pinned host memory) before timing starts.

The printed line (one JSON object) carries the headline workload, the
DeepSeek-style layer (H7168 I2048 E384 k6, int4 G128, Zipf alpha 1.0) on its 70/30
plan (the 115 coldest experts read in place from host memory) at batch 1, with
--steps timed steps after --warmup untimed ones, 4 layers rotated. Nested under
"configs", each with its own roofline and CPU-oracle baseline:
  deepseek  the same layers on the 70/30, all-HBM and all-host plans at batches 1, 4, 16
            (residency switched by moe_cache_update with want_resident)
  qwen3     the Qwen3-30B-A3B-shaped layer (H2048 I768 E128 k8, alpha 0.8), all in HBM,
            batches 1 and 4, 24 layers rotated
  prefill   the Qwen3 layer shape at 2048 and 1024 tokens, bias-free routing, 4 layers
  cache     48 stacked Qwen3-shaped layers, 90 HBM slots per layer, 256 single-token steps
            from a cold start with a pipelined cache update after every step, beside the
            static coldest-on-host plan (value: full-stack tokens/s)
plus the measured link ceilings (streaming reads of HBM and of host-mapped memory,
DMA host -> device) and where the host pool sits (NUMA).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tokens/s + achieved HBM/host-link GB/s vs peak; prefill tok/s"
HBM_PEAK_GBS = 8000.0
HOST_LINK_PEAK_GBS = 63.0
MFMA_BF16_PEAK_TFLOPS = 2516.6

DIMS = {
    "deepseek": dict(H=7168, I=2048, E=384, k=6, G=128, alpha=1.0, seed=2),
    "qwen3": dict(H=2048, I=768, E=128, k=8, G=128, alpha=0.8, seed=1),
    "prefill": dict(H=2048, I=768, E=128, k=8, G=128, alpha=0.0, seed=4),
    "cache": dict(H=2048, I=768, E=128, k=8, G=128, alpha=0.8, seed=3),
    "tiny": dict(H=256, I=128, E=8, k=2, G=32, alpha=0.0, seed=0),
}
NAMES = {"deepseek": "DeepSeek-style layer", "qwen3": "Qwen3-30B-A3B-shaped layer",
         "prefill": "Qwen3-30B-A3B-shaped prefill", "cache": "expert-cache run", "tiny": "tiny layer (fp32 activations)"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps per decode/prefill measurement")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="deepseek,qwen3,prefill,cache,tiny",
                    help="comma list of the workloads to run (the first one run gives the top-level line)")
    ap.add_argument("--deepseek-layers", type=int, default=4)
    ap.add_argument("--deepseek-runs", default="mixed:1,mixed:4,mixed:16,hbm:1,hbm:4,hbm:16,host:1,host:4,host:16",
                    help="plan:batch runs of the DeepSeek-style layer, in order (plans mixed, hbm, host)")
    ap.add_argument("--lowbit", default="3,2", help="code widths below 4 bits also run on the DeepSeek-style layers")
    ap.add_argument("--host-runs", default="misses:1,misses:4,misses:16,layer:1,layer:4",
                    help="DeepSeek-style runs with host computation: misses:B = the 70/30 plan with the host cores "
                         "computing the offloaded experts; layer:B = one layer in four computed entirely by the "
                         "host cores, the rest all in HBM (layer-granular placement)")
    ap.add_argument("--lowbit-runs", default="mixed:1,mixed:4,hbm:1,host:1",
                    help="plan:batch runs of the DeepSeek-style layers at each lower code width")
    ap.add_argument("--qwen3-layers", type=int, default=24)
    ap.add_argument("--qwen3-batches", default="1,4", help="batch sizes of the Qwen3-shaped decode runs")
    ap.add_argument("--prefill-tokens", default="2048,1024", help="micro-batch sizes of the prefill runs")
    ap.add_argument("--prefill-layers", type=int, default=4)
    ap.add_argument("--cache-steps", type=int, default=256)
    ap.add_argument("--max-promotions", type=int, default=8, help="cache run: promotions per layer per update")
    ap.add_argument("--decay", type=float, default=0.9, help="cache run: score decay per update")
    ap.add_argument("--prefetch-slots", type=int, default=8, help="cache run: prefetch slots per layer")
    ap.add_argument("--graph", action="store_true",
                    help="cache run: replay each step's 48 layers as one captured HIP graph instead of enqueueing them")
    ap.add_argument("--cpu-seconds", type=float, default=3.0, help="CPU oracle time budget per configuration")
    ap.add_argument("--head-cpu-seconds", type=float, default=10.0,
                    help="CPU oracle time budget of the DeepSeek-style batch-1 configurations (the head line)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--copy-mb", type=float, default=None,
                    help="only run 10 device-to-device copies of this many MiB (a plain copy kernel of known "
                         "size, for scaling the memory counters of a profiler run), then exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------- inputs


def gen_layers(wl, n_layers):
    import synth
    d = DIMS[wl]
    out, t0 = [], time.time()
    for l in range(n_layers):
        out.append(dict(Wr=synth.router_weight(d["seed"], l, d["E"], d["H"], "bf16"),
                         b=synth.router_bias(d["seed"], l, d["E"], d["alpha"]),
                         blobs=synth.expert_blobs(d["seed"], l, 0, d["E"], d["H"], d["I"], d["G"])))
        log("%s: layer %d/%d generated (%.1fs)" % (wl, l + 1, n_layers, time.time() - t0))
    return out


def device_inputs(wl, B, n):
    """n seeded activation batches [B, H] (bf16) on the device, and their host bits."""
    import numpy as np
    import torch
    import synth
    d = DIMS[wl]
    bits = [synth.activations(d["seed"], 1000 + 97 * B + i, B, d["H"], "bf16") for i in range(n)]
    dev = [torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).cuda() for b in bits]
    return dev, bits


# ----------------------------------------------------------------------------- rooflines


def measured_traffic(kernels, key):
    """DRAM-side bytes per step of `kernels` (kernel classes, summed) from committed
    counter summaries (profiles/*_traffic.md `traffic:` lines for the configuration
    `key`), or None when one is missing or a kernel's sources have changed since the
    counters were taken."""
    csrc = os.path.join(ROOT, "expert_offloaded_ffn_moe_amd", "csrc")
    total = 0
    for kern in kernels:
        found = None
        for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
            for line in open(f, encoding="utf-8"):
                if not line.startswith("traffic:"):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if (kv.get("kernel"), kv.get("config")) != (kern, key):
                    continue
                h = hashlib.sha256()
                for src in kv["sources"].split(","):
                    with open(os.path.join(csrc, src), "rb") as fh:
                        h.update(fh.read())
                if h.hexdigest()[:16] == kv["sha256_16"]:
                    found = int(kv["bytes_per_launch"])
        if found is None:
            return None
        total += found
    return total


def link_peak(hb, sb):
    """(bound, peak GB/s) for hb HBM bytes and sb host-link bytes moved by one launch: the
    rate at which those bytes would move with each link at its own peak."""
    if sb == 0:
        return "hbm", HBM_PEAK_GBS
    if hb == 0:
        return "host-link", HOST_LINK_PEAK_GBS
    return "hbm+host-link", (hb + sb) / (hb / HBM_PEAK_GBS + sb / HOST_LINK_PEAK_GBS)


def roofline(per_kernel, bytes_hbm, bytes_host, A, H, I, key, staged=False):
    """Roofline of the expert FFN of one step: gate/up + down summed (the GEMV pair on the
    decode path, the grouped GEMM pair on the MFMA path). Algorithmic work per step: the
    canonical bytes of every unique expert the step touches (split by the link it is read
    over) and, for the GEMMs, 2*A*3*H*I flops (A = T*k routed rows). The GEMM pair reports
    the bound it comes closer to (flops at prefill sizes, weight bytes for small batches),
    the other under "other". Routing (router logits, top-k, grouping) is reported beside
    it under "route_us", and the whole step under "step_us"."""
    gemm = "gemm_gateup" in per_kernel
    pair = ["gemm_gateup", "gemm_down"] if gemm else ["gateup", "down"]
    names = {"gateup": "k_gateup", "down": "k_down_comb16/k_down_comb/k_down", "gemm_gateup": "k_gemm<gate/up>",
             "gemm_down": "k_gemm<down>"}
    t_us = sum(per_kernel[n]["avg_us"] for n in pair if n in per_kernel)
    t = t_us * 1e-6
    hb, sb = (float(bytes_hbm + bytes_host), 0.0) if staged else (float(bytes_hbm), float(bytes_host))
    bound, peak = link_peak(hb, sb)
    achieved = (hb + sb) / t / 1e9
    by_bytes = dict(bound=bound, kernel=" + ".join(names[n] for n in pair), achieved=round(achieved, 1),
                    peak=round(peak, 1), unit="GB/s", frac=round(achieved / peak, 4), traffic=None,
                    alg_bytes_per_launch=int(hb + sb), alg_bytes_hbm=int(hb), alg_bytes_host=int(sb),
                    avg_launch_us=round(t_us, 3))
    route_us = sum(per_kernel[n]["avg_us"] for n in ("router", "route", "stage") if n in per_kernel)
    step_us = sum(v["avg_us"] * v["launches"] for v in per_kernel.values()) / max(
        1, per_kernel[pair[0]]["launches"])
    extra = dict(route_us=round(route_us, 3), step_us=round(step_us, 3),
                 kernels_us={n: round(v["avg_us"], 3) for n, v in per_kernel.items()})
    traffic = measured_traffic(pair, key)
    by_bytes["traffic"] = traffic
    if not gemm:
        by_bytes.update(extra)
        return by_bytes
    flops = 2.0 * A * 3 * H * I
    tf = flops / t / 1e12
    by_flops = dict(bound="mfma", kernel=by_bytes["kernel"], achieved=round(tf, 1), peak=MFMA_BF16_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), traffic=traffic,
                    alg_flops_per_launch=int(flops), avg_launch_us=round(t_us, 3))
    main, other = (by_flops, by_bytes) if by_flops["frac"] >= by_bytes["frac"] else (by_bytes, by_flops)
    main["other"] = {k: other[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    main.update(extra)
    return main


# ----------------------------------------------------------------------------- measurement


def time_steps(plan, n_layers, xs, y, steps, warmup):
    """Warm-up, then exactly `steps` timed forwards (layer i mod n_layers, input i mod
    len(xs)) between two device synchronisations; then a second pass of the same steps
    with the dispatch's own HIP events for the per-kernel times. Returns (seconds,
    stats of the timed pass, {kernel: launches, avg_us})."""
    import torch
    stream = torch.cuda.current_stream()

    def step(i):
        plan.forward(i % n_layers, xs[i % len(xs)], y, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    plan.reset_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = plan.stats(-1)
    plan.profile(True)
    for i in range(steps):
        step(warmup + i)
    kt = plan.kernel_times()
    plan.profile(False)
    per_kernel = {n: dict(launches=v[0], avg_us=v[1] * 1e3 / v[0]) for n, v in kt.items() if v[0]}
    return elapsed, st, per_kernel


def layer_result(wl, key, B, plan_kind, n_layers, steps, warmup, elapsed, st, per_kernel, slots, bits=4):
    d = DIMS[wl]
    import synth
    eb = synth.expert_bytes(d["H"], d["I"], d["G"], bits)
    fwd = max(st["forwards"], 1)
    bh, bs = st["bytes_hbm"] / fwd, st["bytes_host"] / fwd
    ms = elapsed * 1e3 / steps
    # experts the host cores compute are not read by the GPU kernels: their bytes leave
    # the kernels' algorithmic bytes (first the host-read ones, which they are in the
    # misses mode; a host-computed layer's experts may sit in HBM)
    hc = st.get("host_computed", 0) / fwd * eb
    gs = max(0.0, bs - hc)
    gh = bh - max(0.0, hc - bs)
    roof = roofline(per_kernel, gh, gs, B * d["k"], d["H"], d["I"], key)
    return {
        "value": round(B * steps / elapsed, 2), "unit": "layer-tokens/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "workload": "%s H%d I%d E%d k%d %d-bit codes G%d, batch %d, plan %s (%d of %d experts in HBM), %d layers "
                    "rotated" % (NAMES[wl], d["H"], d["I"], d["E"], d["k"], bits, d["G"], B, plan_kind, slots, d["E"],
                                 n_layers),
        "roofline": roof,
        "layer": {"expert_bytes_per_step_hbm": int(bh), "expert_bytes_per_step_host": int(bs),
                  "unique_experts_per_step": round((bh + bs) / eb, 3),
                  "layer_GBps_wall": round((bh + bs) / (ms * 1e-3) / 1e9, 1),
                  "host_link_GBps_wall": round(bs / (ms * 1e-3) / 1e9, 2),
                  "hit_rate": round(st["hits"] / max(st["hits"] + st["misses"], 1), 5),
                  "host_computed_bytes_per_step": int(hc)},
    }


# ----------------------------------------------------------------------------- CPU oracle


def cpu_cores():
    return len(os.sched_getaffinity(0))


def cpu_baseline(wl, layers, batches_bits, seconds, tokens=None, per_step_forwards=1, label=None, threads=None,
                 bits=4, act="bf16"):
    """The CPU oracle (float64 NumPy, unmodified) on a bounded sample of the same
    workload: forwards of the given batches through the first two layers, until
    `seconds` have passed (at least one). tokens: evaluate y only for these token rows of
    each batch (routing still covers all), with the rate scaled to those rows. BLAS
    threads are pinned to the cores this process may run on (or to `threads`)."""
    import numpy as np
    import threadpoolctl
    from oracle import moe_oracle as O
    d = DIMS[wl]
    cores = threads or cpu_cores()
    n_l = min(2, len(layers))
    done_tokens, n, t0 = 0, 0, time.perf_counter()
    with threadpoolctl.threadpool_limits(limits=cores):
        while n == 0 or time.perf_counter() - t0 < seconds:
            ly = layers[n % n_l]
            xb = batches_bits[n % len(batches_bits)]
            widen = O.bf16_bits_to_f64 if act == "bf16" else (lambda v: v.astype(np.float64))
            O.layer_forward(widen(xb), widen(ly["Wr"]), ly["b"], ly["blobs"], d["H"], d["I"], d["E"], d["k"], d["G"],
                            act, tokens=tokens, bits=bits)
            done_tokens += len(tokens) if tokens is not None else xb.shape[0]
            n += 1
    el = time.perf_counter() - t0
    rate = done_tokens / el
    sample = "%d forwards%s over %d of the layers, %.1fs (float64 NumPy oracle, %d BLAS threads)" % (
        n, "" if tokens is None else " (y of %d token rows each)" % len(tokens), n_l, el, cores)
    unit = "layer-tokens/s"
    if per_step_forwards > 1:
        rate /= per_step_forwards
        unit = "tokens/s"
        sample += "; scaled to full %d-layer steps" % per_step_forwards
    if label:
        sample += "; " + label
    return {"value": round(rate, 5), "unit": unit, "cores": cores, "kind": "oracle", "sample": sample}


# ----------------------------------------------------------------------------- workloads


def run_deepseek(args, out):
    """The DeepSeek-style layers, one plan with an HBM slot for every expert; the 70/30,
    all-HBM and all-host residency sets are switched by moe_cache_update(want_resident)."""
    import numpy as np
    import torch
    import expert_offloaded_ffn_moe_amd as moe
    import synth
    d = DIMS["deepseek"]
    L = args.deepseek_layers
    cfg = moe.make_config(d["H"], d["I"], d["E"], d["k"], d["G"], "bf16", num_layers=L, max_tokens=16,
                          hbm_slots=d["E"])
    plan = moe.Plan(cfg)
    mixed = np.stack([synth.coldest_host_plan(d["seed"], l, d["E"], 0.7) for l in range(L)])
    kept = None
    widths = [int(b) for b in args.lowbit.split(",") if b.strip()]
    low = {b: [] for b in widths}
    for l, ly in enumerate(gen_layers("deepseek", L)):
        plan.load_layer(l, ly["Wr"], ly["b"], ly["blobs"], mixed[l])
        for b in widths:  # the same layers with their codes cut to b bits (seeded synthetic b-bit experts)
            low[b].append(dict(Wr=ly["Wr"], b=ly["b"], blobs=synth.cut_codes(ly["blobs"], d["H"], d["I"], d["G"], b)))
        if l == 0:
            kept = [ly]
    info = plan.info()
    xs = {B: device_inputs("deepseek", B, min(args.warmup + args.steps, 64)) for B in (1, 4, 16)}
    y = torch.empty((16, d["H"]), device="cuda")
    res = {}
    wants = {"mixed": mixed, "hbm": np.ones_like(mixed), "host": np.zeros_like(mixed)}
    current = "mixed"
    for item in args.deepseek_runs.split(","):
        kind, B = item.split(":")
        B = int(B)
        if kind != current:
            plan.cache_update(-1, want_resident=wants[kind])
            current = kind
        slots = int(wants[kind][0].sum())
        steps = args.steps if kind != "host" else max(4, min(args.steps, 20))  # ~20 ms per all-host step at 16
        el, st, pk = time_steps(plan, L, xs[B][0], y[:B], steps, args.warmup)
        key = "deepseek_%s_b%d" % (kind, B)
        r = layer_result("deepseek", key, B, kind, L, steps, args.warmup, el, st, pk, slots)
        log("deepseek %s B%d: %.1f layer-tokens/s, %s" % (kind, B, r["value"], r["roofline"]["frac"]))
        res[key] = r
    for item in [it for it in args.host_runs.split(",") if it.strip()]:
        kind, B = item.split(":")
        B = int(B)
        if kind == "misses":  # 70/30 residency, offloaded experts computed by the host cores
            plan.cache_update(-1, want_resident=wants["mixed"])
            plan.set_host_compute(-1, moe.HOST_COMPUTE_MISSES)
            current, slots, label = "mixed", int(wants["mixed"][0].sum()), "mixed, offloaded experts on host cores"
        else:  # layer-granular: layer 0 entirely on the host cores, layers 1.. all in HBM
            plan.cache_update(-1, want_resident=wants["hbm"])
            plan.set_host_compute(-1, moe.HOST_COMPUTE_NONE)
            plan.set_host_compute(0, moe.HOST_COMPUTE_LAYER)
            current, slots, label = "hbm", d["E"], "all in HBM, 1 of %d layers on host cores" % L
        el, st, pk = time_steps(plan, L, xs[B][0], y[:B], args.steps, args.warmup)
        key = "deepseek_host%s_b%d" % (kind, B)
        r = layer_result("deepseek", key, B, label, L, args.steps, args.warmup, el, st, pk, slots)
        r["layer"]["host_computed_experts_per_step"] = round(st["host_computed"] / max(st["forwards"], 1), 4)
        log("deepseek host %s B%d: %.1f layer-tokens/s" % (kind, B, r["value"]))
        res[key] = r
        plan.set_host_compute(-1, moe.HOST_COMPUTE_NONE)
    plan.destroy()
    for b in widths:
        cfgb = moe.make_config(d["H"], d["I"], d["E"], d["k"], d["G"], "bf16", num_layers=L, max_tokens=16,
                               hbm_slots=d["E"], weight_bits=b)
        plan = moe.Plan(cfgb, layers=[(ly["Wr"], ly["b"], ly["blobs"]) for ly in low[b]], initial_hbm=mixed)
        current = "mixed"
        for item in args.lowbit_runs.split(","):
            kind, B = item.split(":")
            B = int(B)
            if kind != current:
                plan.cache_update(-1, want_resident=wants[kind])
                current = kind
            steps = args.steps if kind != "host" else max(4, min(args.steps, 20))
            el, st, pk = time_steps(plan, L, xs[B][0], y[:B], steps, args.warmup)
            key = "deepseek%dbit_%s_b%d" % (b, kind, B)
            r = layer_result("deepseek", key, B, kind, L, steps, args.warmup, el, st, pk, int(wants[kind][0].sum()),
                             bits=b)
            log("deepseek %d-bit %s B%d: %.1f layer-tokens/s, %s" % (b, kind, B, r["value"], r["roofline"]["frac"]))
            res[key] = r
        plan.destroy()
        if not args.no_cpu:
            cb = cpu_baseline("deepseek", low[b][:1], xs[1][1][:4], args.cpu_seconds, bits=b)
            for key in [kk for kk in res if kk.startswith("deepseek%dbit_" % b) and kk.endswith("_b1")]:
                res[key]["cpu_baseline"] = cb
        low[b] = None
    if not args.no_cpu:
        for B in (1, 4, 16):
            keys = [key for key in res if key.endswith("_b%d" % B) and "bit_" not in key]
            if not keys:
                continue
            toks = [0, 1] if B == 16 else None
            # the head configuration's baseline gets the longer sample (10 s at least)
            secs = max(args.cpu_seconds, args.head_cpu_seconds) if B == 1 else args.cpu_seconds
            cb = cpu_baseline("deepseek", kept, xs[B][1][:4], secs, tokens=toks,
                              label="the oracle evaluates only the routed experts, so residency does not change it")
            for key in keys:
                res[key]["cpu_baseline"] = cb
    out.update(res)
    return {"plan_info": info}


def run_tiny(args, out):
    """The tiny layer (H256 I128 E8 k2 G32, fp32 activations, 16 tokens, all resident):
    a correctness-sized case, timed with the CPU oracle on all of its tokens beside it."""
    import torch
    import expert_offloaded_ffn_moe_amd as moe
    import synth
    d = DIMS["tiny"]
    T = 16
    ly = dict(Wr=synth.router_weight(d["seed"], 0, d["E"], d["H"], "f32"),
              b=synth.router_bias(d["seed"], 0, d["E"], d["alpha"]),
              blobs=synth.expert_blobs(d["seed"], 0, 0, d["E"], d["H"], d["I"], d["G"]))
    cfg = moe.make_config(d["H"], d["I"], d["E"], d["k"], d["G"], "f32", max_tokens=T, hbm_slots=d["E"])
    plan = moe.Plan(cfg, layers=[(ly["Wr"], ly["b"], ly["blobs"])])
    bits = [synth.activations(d["seed"], 1000 + i, T, d["H"], "f32") for i in range(8)]
    xs = [torch.from_numpy(b.copy()).cuda() for b in bits]
    y = torch.empty((T, d["H"]), device="cuda")
    el, st, pk = time_steps(plan, 1, xs, y, args.steps, args.warmup)
    plan.destroy()
    r = layer_result("tiny", "tiny_t16", T, "hbm", 1, args.steps, args.warmup, el, st, pk, d["E"])
    log("tiny T16: %.0f layer-tokens/s" % r["value"])
    if not args.no_cpu:
        r["cpu_baseline"] = cpu_baseline("tiny", [ly], bits[:4], args.cpu_seconds, act="f32",
                                         label="every token of each 16-token batch")
    out["tiny_t16"] = r


def run_qwen3(args, out):
    import torch
    import expert_offloaded_ffn_moe_amd as moe
    d = DIMS["qwen3"]
    L = args.qwen3_layers
    layers = gen_layers("qwen3", L)
    batches = [int(v) for v in args.qwen3_batches.split(",") if v]
    cfg = moe.make_config(d["H"], d["I"], d["E"], d["k"], d["G"], "bf16", num_layers=L, max_tokens=max(batches),
                          hbm_slots=d["E"])
    plan = moe.Plan(cfg, layers=[(ly["Wr"], ly["b"], ly["blobs"]) for ly in layers])
    y = torch.empty((max(batches), d["H"]), device="cuda")
    res = {}
    for B in batches:
        xs, bits = device_inputs("qwen3", B, min(args.warmup + args.steps, 64))
        el, st, pk = time_steps(plan, L, xs, y[:B], args.steps, args.warmup)
        r = layer_result("qwen3", "qwen3_hbm_b%d" % B, B, "hbm", L, args.steps, args.warmup, el, st, pk, d["E"])
        log("qwen3 B%d: %.1f layer-tokens/s, %s" % (B, r["value"], r["roofline"]["frac"]))
        if not args.no_cpu:
            r["cpu_baseline"] = cpu_baseline("qwen3", layers, bits[:4], args.cpu_seconds)
            if B == 1:
                r["cpu_baseline"]["value_one_thread"] = cpu_baseline("qwen3", layers, bits[:4], args.cpu_seconds,
                                                                     threads=1)["value"]
        res["qwen3_hbm_b%d" % B] = r
    plan.destroy()
    out.update(res)


def run_prefill(args, out):
    import torch
    import expert_offloaded_ffn_moe_amd as moe
    d = DIMS["prefill"]
    L = args.prefill_layers
    layers = gen_layers("prefill", L)
    cfg = moe.make_config(d["H"], d["I"], d["E"], d["k"], d["G"], "bf16", num_layers=L, max_tokens=2048,
                          hbm_slots=d["E"])
    plan = moe.Plan(cfg, layers=[(ly["Wr"], ly["b"], ly["blobs"]) for ly in layers])
    y = torch.empty((2048, d["H"]), device="cuda")
    res = {}
    steps = max(4, min(args.steps, 40))
    for T in [int(v) for v in args.prefill_tokens.split(",") if v]:
        xs, bits = device_inputs("prefill", T, 4)
        el, st, pk = time_steps(plan, L, xs, y[:T], steps, min(args.warmup, 5))
        r = layer_result("prefill", "prefill_t%d" % T, T, "hbm", L, steps, min(args.warmup, 5), el, st, pk, d["E"])
        r["unit"] = "layer-tokens/s"
        log("prefill T%d: %.0f layer-tokens/s, %s" % (T, r["value"], r["roofline"]["frac"]))
        if not args.no_cpu:
            r["cpu_baseline"] = cpu_baseline("prefill", layers, bits[:1], args.cpu_seconds, tokens=list(range(8)))
        res["prefill_t%d" % T] = r
    plan.destroy()
    out.update(res)


def run_cache(args, out):
    """Expert-cache decode run over the stacked layers. One step = one token through
    every layer along a residual stream: x_0 is the step's seeded token activation,
    x_{l+1} = bf16(x_l + y_l). Plans, each on the same inputs:
      static   - the coldest-on-host residency (warm-up steps first), no updates;
      cache    - cold start (slots hold experts 0..S-1), pipelined update after every step;
      prefetch - as cache, plus P prefetch slots per layer: before the forward of layer l,
                 the experts of layer l+1 that its router picks for x_l are copied in;
      cache_more_slots - as cache with S+P slots (the same HBM as the prefetch plan);
    and, for comparison with runs that fed every (step, layer) its own activations,
      cache_independent_inputs - as cache on such inputs."""
    import numpy as np
    import torch
    import expert_offloaded_ffn_moe_amd as moe
    import synth
    d = DIMS["cache"]
    H, I, E, k, G = d["H"], d["I"], d["E"], d["k"], d["G"]
    L, B, steps, warmup = 48, 1, args.cache_steps, args.warmup
    S, P = int(round(0.7 * E)), args.prefetch_slots
    layers = gen_layers("cache", L)
    x0b = synth.activations(d["seed"], 7100, (warmup + steps) * B, H, "bf16")
    x0 = torch.from_numpy(x0b.view(np.int16).copy()).view(torch.bfloat16).cuda().view(warmup + steps, B, H)
    n_x = (warmup + steps) * L
    xib = synth.activations(d["seed"], 7000, n_x * B, H, "bf16")
    xind = torch.from_numpy(xib.view(np.int16).copy()).view(torch.bfloat16).cuda().view(n_x, B, H)
    xl = torch.empty((L + 1, B, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((B, H), device="cuda")
    stream = torch.cuda.current_stream()
    modes = {}
    runs = [("static", S, 0, False, True), ("cache", S, 0, True, True), ("prefetch", S, P, True, True),
            ("cache_more_slots", S + P, 0, True, True), ("cache_independent_inputs", S, 0, True, False)]
    for mode, slots, pf, update, chained in runs:
        cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=B, hbm_slots=slots, prefetch_slots=pf)
        init = (np.stack([synth.coldest_host_plan(d["seed"], l, E, slots / E) for l in range(L)]) if not update
                else None)
        plan = moe.Plan(cfg, layers=[(ly["Wr"], ly["b"], ly["blobs"]) for ly in layers], initial_hbm=init)
        torch.cuda.synchronize()

        def layers_pass(i, st):
            for l in range(L):
                x = xl[l] if chained else xind[i * L + l]
                if pf and l + 1 < L:
                    plan.prefetch(l + 1, x=x, stream=st)
                if chained:  # y and x_l+1 = bf16(x_l + y) from the same kernel
                    plan.forward_residual(l, x, y, xl[l + 1], stream=st)
                else:
                    plan.forward(l, x, y, stream=st)

        graph = None
        if chained and args.graph:  # the 48 layers of a step as one HIP graph
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                layers_pass(0, torch.cuda.current_stream())
            torch.cuda.synchronize()

        def one_step(i, eager=False):
            if chained:
                xl[0].copy_(x0[i])
            if graph is not None and not eager:
                graph.replay()
            else:
                layers_pass(i, stream)
            if update:
                plan.cache_update(-1, decay=args.decay, max_promotions=args.max_promotions, overlap=True,
                                  stream=stream)

        first = 0
        if not update:
            for i in range(warmup):
                one_step(i)
            torch.cuda.synchronize()
            plan.reset_stats()
            first = warmup
        times = []
        t_all = time.perf_counter()
        for i in range(first, first + steps):
            t0 = time.perf_counter()
            one_step(i)
            if not update:
                torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_all
        st = plan.stats(-1)
        log("cache run, %s: %d steps x %d layers in %.3fs, hit rate %.4f, prefetched %d" % (
            mode, steps, L, elapsed, st["hits"] / max(st["hits"] + st["misses"], 1), st["prefetched"]))
        plan.profile(True)  # per-kernel times over a further 16 steps in the same mode, enqueued eagerly
        for i in range(first, first + min(16, steps)):
            one_step(i, eager=True)
        kt = plan.kernel_times()
        plan.profile(False)
        launch = "one HIP graph per step" if graph is not None else "eager"
        del graph
        plan.destroy()
        t = np.sort(np.array(times))
        fwd = max(st["forwards"], 1)
        pk = {n: dict(launches=v[0], avg_us=v[1] * 1e3 / v[0]) for n, v in kt.items() if v[0]}
        modes[mode] = dict(
            tokens_per_s=round(B * steps / elapsed, 2), step_ms_median=round(float(np.median(t)) * 1e3, 4),
            step_ms_p95=round(float(np.percentile(t, 95)) * 1e3, 4),
            hbm_slots=slots, prefetch_slots=pf, inputs="residual stream" if chained else "independent per layer",
            launch=launch,
            hit_rate=round(st["hits"] / max(st["hits"] + st["misses"], 1), 5), hits=st["hits"], misses=st["misses"],
            prefetched=st["prefetched"],
            bytes_hbm_per_layer_step=int(st["bytes_hbm"] / fwd), bytes_host_per_layer_step=int(st["bytes_host"] / fwd),
            bytes_copied=st["bytes_copied"], promotions=st["promotions"], evictions=st["evictions"],
            roofline=roofline(pk, st["bytes_hbm"] / fwd, st["bytes_host"] / fwd, B * k, H, I, "cache_48_layers"))
    c = modes["cache"]
    r = {"value": c["tokens_per_s"], "unit": "tokens/s", "steps": steps, "warmup": 0,
         "ms_per_step": round(1e3 * B / c["tokens_per_s"], 5),
         "workload": "%s: %d stacked Qwen3-30B-A3B-shaped layers H%d I%d E%d k%d int4 G%d on a residual stream "
                     "(x_l+1 = bf16(x_l + y_l), fused into each layer's combine), %d HBM slots per layer (rest "
                     "host-mapped), batch %d, %d steps, cold start, pipelined cache update after every step (max %d "
                     "promotions per layer, score decay %g)" % (
                         NAMES["cache"], L, H, I, E, k, G, S, B, steps, args.max_promotions, args.decay),
         "roofline": c.pop("roofline"), "cache_run": c,
         "other_plans": {m: v for m, v in modes.items() if m != "cache"}}
    if not args.no_cpu:
        # 2 steps x 48 layers of the same inputs, extrapolated to full steps
        cb = cpu_baseline("cache", layers[:2], [xib[(i * L) * B:(i * L + 1) * B] for i in range(4)], args.cpu_seconds,
                          per_step_forwards=L, label="extrapolated from forwards of single layers")
        r["cpu_baseline"] = cb
    out["cache_48_layers"] = r


# ----------------------------------------------------------------------------- main


def topology():
    try:
        txt = subprocess.run(["rocm-smi", "--showtopo"], capture_output=True, text=True, timeout=30).stdout
        numa = [ln.strip() for ln in txt.splitlines() if "Numa" in ln or "NUMA" in ln]
    except Exception as e:  # rocm-smi is only informative here
        numa = ["rocm-smi --showtopo unavailable: %s" % e]
    try:
        txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30).stdout
        clocks = [ln.strip() for ln in txt.splitlines() if "clk" in ln.lower()]
    except Exception as e:  # informative only
        clocks = ["rocm-smi --showclocks unavailable: %s" % e]
    nodes = sorted(glob.glob("/sys/devices/system/node/node[0-9]*"))
    return {"host_numa_nodes": len(nodes), "rocm_smi_numa": numa[:8], "rocm_smi_clocks_at_start": clocks[:8],
            "cpu_cores_available": cpu_cores()}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (expert-parallel sharding "
              "is a design note, not code); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_mb:
        n = int(args.copy_mb * (1 << 20)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 4 * n, "launches": 10}), flush=True)
        return
    import expert_offloaded_ffn_moe_amd as moe

    extra = {"topology": topology()}
    log("topology:", extra["topology"])
    if not args.no_ceilings:
        ceil = {}
        for label, hbm, host in (("1GiB", 1 << 30, 256 << 20), ("136MB", 136 << 20, 64 << 20),
                                 ("13MB", 13 << 20, 16 << 20)):
            c = moe.measure_link_ceilings(hbm, host, 5)
            ceil["hbm_read_%s_GBps" % label] = round(c["hbm_read_gbps"], 1)
            if label == "1GiB":
                ceil["host_mapped_read_256MiB_GBps"] = round(c["host_read_gbps"], 2)
                ceil["h2d_copy_256MiB_GBps"] = round(c["h2d_copy_gbps"], 2)
        extra["measured_ceilings"] = ceil
        log("ceilings:", ceil)
    configs = {}
    order = [w.strip() for w in args.only.split(",") if w.strip()]
    for wl in order:
        r = {"deepseek": run_deepseek, "qwen3": run_qwen3, "prefill": run_prefill, "cache": run_cache,
             "tiny": run_tiny}[wl](
            args, configs)
        if r:
            extra.update(r)
    head_key = {"deepseek": "deepseek_mixed_b1", "qwen3": "qwen3_hbm_b1", "prefill": "prefill_t2048",
                "cache": "cache_48_layers", "tiny": "tiny_t16"}[order[0]]
    if head_key not in configs:  # a subset of runs: the first one measured heads the line
        head_key = next(iter(configs))
    head = configs[head_key]
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init int4 experts of the named shapes)",
        "config": {"workload": head["workload"], "key": head_key,
                   "arithmetic": "int4 weight codes (exact in the bf16 dot products and MFMA), fp16 group scales, "
                                 "bf16 activations, fp32 accumulation, fp32 y"},
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "layer": head.get("layer"),
        "configs": {k: v for k, v in configs.items() if k != head_key},
    }
    for key, v in head.items():  # the head workload's own extra fields (comparison runs and the like)
        if key not in line and key not in ("workload", "unit", "value", "steps", "warmup", "ms_per_step"):
            line[key] = v
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
