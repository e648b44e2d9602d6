#!/usr/bin/env python3
"""Benchmark of the routed MoE FFN layer forward on one MI355X.

A step is one forward of one layer (router -> top-k -> grouping by expert ->
gate/up + SwiGLU -> down -> combine) for a batch of tokens. Steps walk through
a stack of seeded layers (default 24), so that the experts a step reads were
last read many steps (hundreds of MB) earlier and are not served from the
256 MB Infinity Cache; every input is resident in HBM (or, for offloaded
experts, in pinned host memory) before timing starts.

Workloads (--workload):
  decode    Qwen3-30B-A3B-shaped layer (H2048 I768 E128 k8 G128 bf16, Zipf bias
            alpha 0.8), all experts in HBM; --batch 1 (default) or 4.
  deepseek  H7168 I2048 E384 k6 G128 bf16, Zipf alpha 1.0, 70% of experts in HBM
            and the coldest 30% read from host memory (--plan mixed | hbm | host).
  prefill   the Qwen3 layer shape with 2048 (or --batch) tokens, bias-free routing.
  cache     expert-cache decode run: 48 stacked Qwen3-shaped layers (Zipf alpha 0.8,
            seeded per layer), HBM slots for 70% of each layer's experts, the rest read
            from host memory; 256 single-token steps, a pipelined cache update after every step
            from a cold start (slots hold experts 0..89), beside the static coldest-on-host
            plan without updates. value = full-stack tokens/s.

Prints one JSON line. value = layer-tokens/s over exactly --steps timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tokens/s + achieved HBM/host-link GB/s vs peak; prefill tok/s"
HBM_PEAK_GBS = 8000.0
HOST_LINK_PEAK_GBS = 63.0
MFMA_BF16_PEAK_TFLOPS = 2516.6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_dims(args):
    if args.workload in ("decode", "prefill", "cache"):
        return dict(H=2048, I=768, E=128, k=8, G=128, act="bf16", alpha=0.0 if args.workload == "prefill" else 0.8,
                    seed={"decode": 1, "prefill": 4, "cache": 3}[args.workload])
    if args.workload == "deepseek":
        return dict(H=7168, I=2048, E=384, k=6, G=128, act="bf16", alpha=1.0, seed=2)
    raise SystemExit("unknown workload")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (decode 200, prefill 40, cache 256)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=["decode", "deepseek", "prefill", "cache"])
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--plan", default="mixed", choices=["mixed", "hbm", "host"])
    ap.add_argument("--sweep", default=None,
                    help="comma list of plan:batch runs on the same generated layers, one JSON line each")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--max-promotions", type=int, default=8, help="cache workload: promotions per layer per update")
    ap.add_argument("--decay", type=float, default=0.9, help="cache workload: score decay per update")
    ap.add_argument("--copy-mb", type=float, default=None,
                    help="only run 10 device-to-device copies of this many MiB (a plain copy kernel of known "
                         "size, for scaling the memory counters of a profiler run), then exit")
    ap.add_argument("--gemm-min-tokens", type=int, default=0,
                    help="batches of at least this many tokens take the grouped MFMA GEMM (0: the library default)")
    ap.add_argument("--stage-slots", type=int, default=0,
                    help="prefill: HBM staging slots for the offloaded experts a batch touches (0 = read in place)")
    ap.add_argument("--no-cpu", action="store_true")
    return ap.parse_args()


def make_layers(d, L, keep_blobs):
    import synth
    H, I, E, G, act, alpha, seed = (d[n] for n in ("H", "I", "E", "G", "act", "alpha", "seed"))
    layers, t0 = [], time.time()
    for l in range(L):
        blobs = synth.expert_blobs(seed, l, 0, E, H, I, G)
        Wr = synth.router_weight(seed, l, E, H, act)
        b = synth.router_bias(seed, l, E, alpha)
        layers.append(dict(Wr=Wr, b=b, blobs=blobs))
        log("layer %d/%d generated (%.1fs)" % (l + 1, L, time.time() - t0))
    return layers


def measured_traffic(kernel, workload, plan, batch):
    """DRAM-side bytes per launch of `kernel` from a committed counter summary
    (profiles/*_traffic.md, a `traffic:` line), or None when there is none for this
    workload or the kernel's sources have changed since the counters were taken."""
    import glob
    import hashlib

    csrc = os.path.join(ROOT, "expert_offloaded_ffn_moe_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        for line in open(f, encoding="utf-8"):
            if not line.startswith("traffic:"):
                continue
            kv = dict(t.split("=", 1) for t in line.split()[1:])
            if (kv.get("kernel"), kv.get("workload"), kv.get("plan"), kv.get("batch")) != (
                    kernel, workload, plan, str(batch)):
                continue
            h = hashlib.sha256()
            for src in kv["sources"].split(","):
                with open(os.path.join(csrc, src), "rb") as fh:
                    h.update(fh.read())
            if h.hexdigest()[:16] == kv["sha256_16"]:
                return int(kv["bytes_per_launch"])
    return None


def roofline(per_kernel, bytes_hbm, bytes_host, assignments, H, I):
    """Roofline of the dominant expert kernel (largest total time over the profiled pass).

    Expert kernels move weight bytes: gate/up reads 2/3 of each touched expert's bytes,
    down 1/3. With every touched expert in HBM the peak is HBM's; with every one on the
    host it is the host link's; with both, the peak is the rate at which those bytes would
    move with each link at its own peak (time = hbm bytes / HBM + host bytes / link).
    GEMM kernels are also priced in flops against bf16 MFMA: 2*A*H*2I for gate/up, 2*A*I*H
    for down, with A = T*k routed token rows. A GEMM launch reports the bound it comes
    closer to (flops for large batches, weight bytes for small ones), the other under
    "other".
    """
    ffn = [n for n in ("gateup", "down", "gemm_gateup", "gemm_down", "stage") if n in per_kernel]
    dom = max(ffn, key=lambda n: per_kernel[n]["avg_us"] * per_kernel[n]["launches"])
    t = per_kernel[dom]["avg_us"] * 1e-6
    staged = "stage" in per_kernel
    if dom == "stage":  # the staging copy moves the touched offloaded experts over the host link once
        hb, sb = 0.0, bytes_host
    elif staged:  # the GEMMs then read every touched expert from HBM
        share = 2.0 / 3.0 if dom == "gemm_gateup" else 1.0 / 3.0
        hb, sb = share * (bytes_hbm + bytes_host), 0.0
    else:
        share = 2.0 / 3.0 if dom in ("gateup", "gemm_gateup") else 1.0 / 3.0
        hb, sb = share * bytes_hbm, share * bytes_host
    if sb == 0:
        bound, peak = "hbm", HBM_PEAK_GBS
    elif hb == 0:
        bound, peak = "host-link", HOST_LINK_PEAK_GBS
    else:
        bound = "hbm+host-link"
        peak = (hb + sb) / (hb / HBM_PEAK_GBS + sb / HOST_LINK_PEAK_GBS)
    achieved = (hb + sb) / t / 1e9
    by_bytes = dict(bound=bound, kernel=dom, achieved=round(achieved, 1), peak=round(peak, 1), unit="GB/s",
                    frac=round(achieved / peak, 4), traffic=None, alg_bytes_per_launch=int(hb + sb),
                    alg_bytes_hbm=int(hb), alg_bytes_host=int(sb), avg_launch_us=round(per_kernel[dom]["avg_us"], 3))
    if not dom.startswith("gemm"):
        return by_bytes
    flops = 2.0 * assignments * H * I * (2 if dom == "gemm_gateup" else 1)
    tf = flops / t / 1e12
    by_flops = dict(bound="mfma", kernel=dom, achieved=round(tf, 1), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), traffic=None, alg_flops_per_launch=int(flops),
                    avg_launch_us=round(per_kernel[dom]["avg_us"], 3))
    main, other = (by_flops, by_bytes) if by_flops["frac"] >= by_bytes["frac"] else (by_bytes, by_flops)
    main["other"] = {k: other[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    return main


def run_one(args, d, layers, B, plan_kind, steps, warmup):
    """Time `steps` forwards (layer i mod L) at batch B under one residency plan."""
    import numpy as np
    import torch

    import expert_offloaded_ffn_moe_amd as moe
    import synth

    H, I, E, k, G, act, alpha, seed = (d[n] for n in ("H", "I", "E", "k", "G", "act", "alpha", "seed"))
    L = len(layers)
    eb = synth.expert_bytes(H, I, G)
    slots = {"mixed": int(round(0.7 * E)), "hbm": E, "host": 0}[plan_kind]
    cfg = moe.make_config(H, I, E, k, G, act, num_layers=L, max_tokens=B, hbm_slots=slots,
                          gemm_min_tokens=args.gemm_min_tokens, prefill_stage_slots=args.stage_slots)
    plan = moe.Plan(cfg)
    for l, ly in enumerate(layers):
        res = synth.coldest_host_plan(seed, l, E, slots / E) if plan_kind == "mixed" else None
        plan.load_layer(l, ly["Wr"], ly["b"], ly["blobs"], res)
    n_in = min(warmup + steps, 64)
    xs_bits = [synth.activations(seed, 1000 + i, B, H, act) for i in range(n_in)]
    xs = [torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).cuda() for xb in xs_bits]
    y = torch.empty((B, H), device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        plan.forward(i % L, xs[i % len(xs)], y, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    plan.reset_stats()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    st = plan.stats(-1)
    log("timed %d steps in %.4fs (plan %s, batch %d)" % (steps, elapsed, plan_kind, B))

    # profiled pass: per-kernel times from events stamped by each dispatch
    plan.profile(True)
    for i in range(steps):
        step(warmup + i)
    kt = plan.kernel_times()
    plan.profile(False)
    plan.destroy()

    ms_per_step = elapsed * 1e3 / steps
    fwd = max(st["forwards"], 1)
    bytes_hbm, bytes_host = st["bytes_hbm"] / fwd, st["bytes_host"] / fwd
    per_kernel = {n: dict(launches=v[0], avg_us=(v[1] * 1e3 / v[0])) for n, v in kt.items() if v[0]}
    roof = roofline(per_kernel, bytes_hbm, bytes_host, B * k, H, I)
    roof["traffic"] = measured_traffic(roof["kernel"], args.workload, plan_kind, B)
    name = {"decode": "Qwen3-30B-A3B-shaped decode", "deepseek": "DeepSeek-style decode",
            "prefill": "Qwen3-30B-A3B-shaped prefill"}[args.workload]
    return {
        "metric": METRIC,
        "value": round(B * steps / elapsed, 2),
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s layer H%d I%d E%d k%d int4 G%d, batch %d, %d-layer rotation, plan %s" % (
            name, H, I, E, k, G, B, L, plan_kind), "hbm_slots": slots, "prefill_stage_slots": args.stage_slots,
            "alpha": alpha, "seed": seed},
        "roofline": roof,
        "layer": {"expert_bytes_per_step_hbm": int(bytes_hbm), "expert_bytes_per_step_host": int(bytes_host),
                  "unique_experts_per_step": round((bytes_hbm + bytes_host) / eb, 3),
                  "layer_GBps_wall": round((bytes_hbm + bytes_host) / (ms_per_step * 1e-3) / 1e9, 1),
                  "host_link_GBps_wall": round(bytes_host / (ms_per_step * 1e-3) / 1e9, 2),
                  "hit_rate": round(st["hits"] / max(st["hits"] + st["misses"], 1), 5),
                  "kernels_us": {n: round(v["avg_us"], 3) for n, v in per_kernel.items()}},
        "_xs_bits": xs_bits,
    }


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
    d = workload_dims(args)
    if args.steps is None:
        args.steps = {"decode": 200, "deepseek": 200, "prefill": 40, "cache": 256}[args.workload]
    L = args.layers or {"decode": 24, "deepseek": 3, "prefill": 4, "cache": 48}[args.workload]
    layers = make_layers(d, L, keep_blobs=True)
    if args.workload == "cache":
        out, xs_bits = run_cache(args, d, layers)
        if not args.no_cpu:
            cb = cpu_baseline(args, d, args.batch or 1, L, layers, xs_bits)
            cb["value"] = round(cb["value"] / L, 6)
            cb["unit"] = "tokens/s"
            cb["sample"] += "; value scaled to full %d-layer steps" % L
            out["cpu_baseline"] = cb
        print(json.dumps(out), flush=True)
        return
    default_plan = args.plan if args.workload == "deepseek" else "hbm"
    if args.sweep:
        runs = []
        for item in args.sweep.split(","):
            pk, bs = item.split(":")
            runs.append((pk, int(bs)))
    else:
        runs = [(default_plan, args.batch or (2048 if args.workload == "prefill" else 1))]
    for i, (pk, B) in enumerate(runs):
        out = run_one(args, d, layers, B, pk, args.steps, args.warmup)
        xs_bits = out.pop("_xs_bits")
        if not args.no_cpu and i == 0:
            out["cpu_baseline"] = cpu_baseline(args, d, B, L, layers, xs_bits)
        print(json.dumps(out), flush=True)


def run_cache(args, d, layers):
    """Expert-cache decode run over the stacked layers: the static plan first (warm-up
    steps, then the timed steps, no updates), then the cached plan from its cold start
    with a pipelined cache update after every step. One step = one token batch through every layer;
    each (step, layer) takes its own seeded activations."""
    import numpy as np
    import torch

    import expert_offloaded_ffn_moe_amd as moe
    import synth

    H, I, E, k, G, act, alpha, seed = (d[n] for n in ("H", "I", "E", "k", "G", "act", "alpha", "seed"))
    L, B, steps, warmup = len(layers), args.batch or 1, args.steps, args.warmup
    S = int(round(0.7 * E))
    eb = synth.expert_bytes(H, I, G)
    n_x = (warmup + steps) * L
    xb = synth.activations(seed, 7000, n_x * B, H, act)
    xs = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).cuda().view(n_x, B, H)
    y = torch.empty((B, H), device="cuda")
    out = {}
    for mode in ("static", "cache"):
        cfg = moe.make_config(H, I, E, k, G, act, num_layers=L, max_tokens=B, hbm_slots=S)
        plan = moe.Plan(cfg)
        for l, ly in enumerate(layers):
            res = synth.coldest_host_plan(seed, l, E, S / E) if mode == "static" else None
            plan.load_layer(l, ly["Wr"], ly["b"], ly["blobs"], res)
        torch.cuda.synchronize()
        first = 0
        if mode == "static":
            for i in range(warmup):
                for l in range(L):
                    plan.forward(l, xs[i * L + l], y)
            torch.cuda.synchronize()
            plan.reset_stats()
            first = warmup
        times = []
        t_all = time.perf_counter()
        for i in range(first, first + steps):
            t0 = time.perf_counter()
            for l in range(L):
                plan.forward(l, xs[i * L + l], y)
            if mode == "cache":
                plan.cache_update(-1, decay=args.decay, max_promotions=args.max_promotions, overlap=True)  # pipelined
            else:
                torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_all
        st = plan.stats(-1)
        log("%s plan: %d steps x %d layers in %.3fs, hit rate %.4f" % (
            mode, steps, L, elapsed, st["hits"] / max(st["hits"] + st["misses"], 1)))
        # profiled pass over a further 16 steps (same mode)
        plan.profile(True)
        n_prof = min(16, steps)
        for i in range(first, first + n_prof):
            for l in range(L):
                plan.forward(l, xs[i * L + l], y)
            if mode == "cache":
                plan.cache_update(-1, decay=args.decay, max_promotions=args.max_promotions, overlap=True)
        kt = plan.kernel_times()
        plan.profile(False)
        plan.destroy()
        t = np.sort(np.array(times))
        fwd = max(st["forwards"], 1)
        per_kernel = {n: dict(launches=v[0], avg_us=(v[1] * 1e3 / v[0])) for n, v in kt.items() if v[0]}
        out[mode] = dict(
            tokens_per_s=round(B * steps / elapsed, 2),
            step_ms_median=round(float(np.median(t)) * 1e3, 4),
            step_ms_p95=round(float(np.percentile(t, 95)) * 1e3, 4),
            tokens_per_s_median=round(B / float(np.median(t)), 2),
            tokens_per_s_p5=round(B / float(np.percentile(t, 95)), 2),
            hit_rate=round(st["hits"] / max(st["hits"] + st["misses"], 1), 5),
            hits=st["hits"], misses=st["misses"],
            bytes_hbm_per_layer_step=int(st["bytes_hbm"] / fwd), bytes_host_per_layer_step=int(st["bytes_host"] / fwd),
            bytes_copied=st["bytes_copied"], promotions=st["promotions"], evictions=st["evictions"],
            kernels_us={n: round(v["avg_us"], 3) for n, v in per_kernel.items()},
            roofline=roofline(per_kernel, st["bytes_hbm"] / fwd, st["bytes_host"] / fwd, B * k, H, I))
    c = out["cache"]
    res = {
        "metric": METRIC,
        "value": c["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 0,
        "ms_per_step": round(1e3 * B / c["tokens_per_s"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "expert-cache decode run: %d stacked Qwen3-30B-A3B-shaped layers H%d I%d E%d k%d "
                               "int4 G%d, %d HBM slots per layer (rest host-mapped), batch %d, %d steps, cold start, "
                               "pipelined cache update after every step (max %d promotions per layer, score decay %g)" % (
                                   L, H, I, E, k, G, S, B, steps, args.max_promotions, args.decay),
                   "alpha": alpha, "seed": seed},
        "roofline": c["roofline"],
        "cache_run": {n: v for n, v in c.items() if n != "roofline"},
        "static_plan": out["static"],
    }
    xs_bits = [xb[(i * L) * B:(i * L + 1) * B] for i in range(min(8, warmup + steps))]
    return res, xs_bits


def cpu_baseline(args, d, B, L, layers_host, xs_bits):
    """The CPU oracle (float64, unmodified) on a bounded sample of the same steps."""
    import numpy as np

    from oracle import moe_oracle as O

    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
    except Exception:
        threads = 1
    H, I, E, k, G, act = (d[n] for n in ("H", "I", "E", "k", "G", "act"))
    n_layers = min(2, len(layers_host))
    tokens, t0, i = 0, time.perf_counter(), 0
    while time.perf_counter() - t0 < args.cpu_seconds:
        l = i % n_layers
        Wr, b, blobs = layers_host[l]["Wr"], layers_host[l]["b"], layers_host[l]["blobs"]
        x = O.bf16_bits_to_f64(xs_bits[i % len(xs_bits)])
        O.layer_forward(x, O.bf16_bits_to_f64(Wr), b, blobs, H, I, E, k, G, act)
        tokens += B
        i += 1
    el = time.perf_counter() - t0
    log("cpu oracle: %d forwards in %.1fs" % (i, el))
    out = {"value": round(tokens / el, 4), "unit": "layer-tokens/s", "cores": threads, "kind": "oracle",
           "sample": "%d forwards of batch %d over %d of the %d layers (float64 NumPy oracle, %.1fs)" % (
               i, B, n_layers, L, el)}
    # the same oracle pinned to one thread, on a shorter sample
    try:
        import threadpoolctl
        with threadpoolctl.threadpool_limits(limits=1):
            tok1, t1, j = 0, time.perf_counter(), 0
            while time.perf_counter() - t1 < args.cpu_seconds / 3:
                l = j % n_layers
                Wr, b, blobs = layers_host[l]["Wr"], layers_host[l]["b"], layers_host[l]["blobs"]
                x = O.bf16_bits_to_f64(xs_bits[j % len(xs_bits)])
                O.layer_forward(x, O.bf16_bits_to_f64(Wr), b, blobs, H, I, E, k, G, act)
                tok1 += B
                j += 1
            out["value_one_thread"] = round(tok1 / (time.perf_counter() - t1), 4)
    except Exception as e:  # the one-thread figure is extra; the baseline above stands without it
        log("cpu oracle, one thread: skipped (%s)" % e)
    return out


if __name__ == "__main__":
    main()
