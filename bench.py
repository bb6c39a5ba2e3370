#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
route (histogram, scan, stable permutation) -> expert forward (gather, W13
grouped GEMM + SwiGLU, W2 grouped GEMM into route slots) -> combine, and for
training workloads the backward (combine backward, W2 DGRAD + SwiGLU
backward, W2/W13 WGRAD, W13 DGRAD, input-gradient reduction).

Default workload: T = 2,048 tokens, D = 7,168, F = 2,048, E = 384 experts,
top-6, balanced routing, BF16 operands with fp32 accumulation, forward +
backward.  Inputs are resident in HBM before timing starts.  Useful work is
6*R*D*F FLOPs forward and twice that backward (R = valid routes; padding and
replay excluded), the Dist-MoE explainer's count (section 07).

Prints ONE JSON line.  Also reports the dominant kernel against its roofline
(per-kernel HIP-event timing over a second pass of the timed steps) and the
CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3

WORKLOADS = {
    # name: (config key, training)
    "bf16_train_balanced": ("bf16_fwd_balanced", True),
    "bf16_fwd_balanced": ("bf16_fwd_balanced", False),
    "bf16_train_zipf": ("bf16_train_zipf", True),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bf16_train_balanced", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-experts", type=int, default=24,
                    help="experts in the CPU-oracle sample (all their routes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a reference kernel "
                         "for scaling hardware byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert "
              "parallelism over xGMI is a design note only). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_routed_03_amd import binding as B
    from mixture_experts_routed_03_amd import workloads as wl

    cfg_key, training = WORKLOADS[args.workload]
    cfg = wl.CONFIGS[cfg_key]
    if args.workload == "bf16_train_zipf":
        training = True
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lay = wl.make_layer(cfg, 0, device=dev, grads=training)
    T, D, F, E, K = cfg.T, cfg.D, cfg.F, cfg.E, cfg.K
    layer = B.MoeLayer(T, D, F, E, K, cfg.prec, training=training, device=dev)
    act = layer.act_dtype
    y = torch.empty((T, D), dtype=act, device=dev)
    if training:
        dx = torch.empty((T, D), dtype=act, device=dev)
        dw13 = torch.empty((E, 2 * F, D), dtype=layer.dw_dtype, device=dev)
        dw2 = torch.empty((E, D, F), dtype=layer.dw_dtype, device=dev)
        dsc = torch.empty((T, K), dtype=torch.float32, device=dev)

    def step():
        layer.route(lay["ids"])
        layer.forward(lay["x"], lay["w13"], lay["w2"])
        layer.combine(lay["scores"], y)
        if training:
            layer.backward(lay["x"], lay["scores"], lay["dy"], lay["w13"], lay["w2"], dx, dw13,
                           dw2, dsc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rb = layer.readback(T)
    counts = rb["counts"].astype(np.int64)
    R = int(rb["R"])
    nonempty = int((counts > 0).sum())

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads and writes copy_probe_mb MiB each
        torch.cuda.synchronize()
        del src, dst

    # ---- timed region: K steps, bracketed by synchronize on both sides
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps

    # ---- second pass with per-kernel events (on the library's launch stream)
    B.moe_timing_enable(layer.plan, True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = B.moe_timing_read(layer.plan)
    B.moe_timing_enable(layer.plan, False)

    es = 2 if cfg.prec != "f32" else 4
    fwd_flops = 6 * R * D * F
    flops = fwd_flops * (3 if training else 1)
    value = flops / (ms_step * 1e-3) / 1e12

    # Algorithmic bytes per launch (what each kernel must move at minimum).
    w13_b = nonempty * 2 * F * D * es
    w2_b = nonempty * D * F * es
    alg = {
        "route": T * K * 4 * 2 + R * 4 * 2,
        "gather": T * D * es + R * D * es,
        "w13_swiglu": w13_b + R * D * es + R * 2 * F * es + R * F * es,
        "w2_scatter": w2_b + R * F * es + R * D * es,
        "combine": T * K * D * es + T * D * es + T * K * 8,
        "combine_bwd": T * D * es + T * K * D * es + R * D * es + T * K * 8,
        "w2_dgrad_swiglu": w2_b + R * D * es + R * 2 * F * es * 2,
        "w2_wgrad": w2_b // es * (4 if layer.dw_dtype == torch.float32 else 2) + R * D * es
        + R * 2 * F * es,
        "w13_dgrad": w13_b + R * 2 * F * es + R * D * 4,
        "w13_wgrad": w13_b // es * (4 if layer.dw_dtype == torch.float32 else 2)
        + R * 2 * F * es + R * D * es,
        "dx_reduce": R * D * 4 + T * D * es,
    }
    kflops = {"w13_swiglu": 2 * R * 2 * F * D, "w2_scatter": 2 * R * D * F,
              "w2_dgrad_swiglu": 2 * R * D * F, "w2_wgrad": 2 * R * D * F,
              "w13_dgrad": 2 * R * 2 * F * D, "w13_wgrad": 2 * R * 2 * F * D}
    kernels = {}
    for name, (tot, n) in ktimes.items():
        if n == 0:
            continue
        avg = tot / n
        ent = {"avg_ms": round(avg, 4), "launches": n}
        if name in alg:
            ent["GB/s"] = round(alg[name] / (avg * 1e-3) / 1e9, 1)
            ent["alg_bytes"] = int(alg[name])
        if name in kflops:
            ent["TFLOP/s"] = round(kflops[name] / (avg * 1e-3) / 1e12, 2)
        kernels[name] = ent
    dom = max((k for k in kernels if k in alg), key=lambda k: kernels[k]["avg_ms"] *
              kernels[k]["launches"])
    ach = alg[dom] / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                "alg_bytes_per_launch": int(alg[dom])}
    route_gbs = kernels.get("route", {}).get("GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lay, cfg, training, args.cpu_experts)

    out = {
        "metric": "useful TFLOP/s/GPU MoE expert fwd+bwd (BF16, MXFP8); % MFMA peak; route GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.prec == "bf16" else cfg.prec,
        "data": "synthetic (seeded; N(0,1) tokens, N(0,1/fan_in) weights, top-6 uniform routing)",
        "config": {"workload": f"{args.workload}: T={T} D={D} F={F} E={E} K={K} "
                               f"{'fwd+bwd' if training else 'fwd'}",
                   "routes": R, "nonempty_experts": nonempty, "max_rows": int(counts.max()),
                   "dw_dtype": "bf16" if layer.dw_dtype == torch.bfloat16 else "f32"},
        "mfma_peak_frac": round(value / PEAK_BF16_TFLOPS, 4),
        "route_GBps": route_gbs,
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(lay, cfg, training, n_exp):
    """The fp64 oracle, as it stands, on the routes of the first n_exp experts
    (all their tokens): forward (+ backward), wall time on the host cores."""
    import numpy as np
    import torch

    from oracle import moe as om

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    ids = lay["ids"].cpu().numpy()
    ids_s = np.where((ids >= 0) & (ids < n_exp), ids, -1).astype(np.int32)
    R_s = int((ids_s >= 0).sum())
    x = lay["x"].cpu()
    sc = lay["scores"].cpu()
    w13 = lay["w13"][:n_exp].cpu()
    w2 = lay["w2"][:n_exp].cpu()
    t0 = time.perf_counter()
    y, cache = om.forward(x, ids_s, sc, w13, w2, keep=True)
    if training:
        om.backward(lay["dy"].cpu(), x, ids_s, sc, w13, w2, cache)
    dt = time.perf_counter() - t0
    flops = 6 * R_s * cfg.D * cfg.F * (3 if training else 1)
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"routes of experts 0..{n_exp - 1} ({R_s} of {int((ids >= 0).sum())} routes), "
                      f"{'forward+backward' if training else 'forward'}, fp64 NumPy"}


if __name__ == "__main__":
    main()
