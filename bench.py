#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
route (histogram, scan, stable permutation) -> expert forward (W13 grouped
GEMM reading x rows through the permutation + SwiGLU, W2 grouped GEMM into
route slots) -> combine, and for
training workloads the backward (combine backward, W2 DGRAD + SwiGLU
backward, W2/W13 WGRAD, W13 DGRAD, input-gradient reduction).  MXFP8
workloads add the row quantizers and column bundles.

Workloads (all at T = 2,048 tokens, D = 7,168, F = 2,048, E = 384, top-6):
  bf16_train_zipf      BF16, Zipf(1.2) routing, forward + backward (default:
                       the stated BF16 forward + backward configuration)
  bf16_train_balanced  BF16, balanced routing, forward + backward
  bf16_fwd_balanced    BF16, balanced routing, forward only
  bf16_fwd_fused       the same with the combine fused into the W2 epilogue
                       (fp32 atomics; inference form)
  mxfp8_train_shared   MXFP8 routed layer + one shared BF16 SwiGLU expert,
                       forward + backward
  mxfp8_ten_layer      ten MXFP8 layers (Zipf 0, 0.6, 1.0, 1.4 cycled), ten
                       forwards then ten backwards in one byte-budgeted arena
  ep8_share, ep64_share  the same 12,288 routed rows as one GPU's share under
                       expert parallelism: 48 experts x ~256 rows, 6 x 2,048
                       (BF16 forward + backward; compute-bound probes)

Inputs are resident in HBM before timing starts.  Useful work is 6*R*D*F
FLOPs forward and twice that backward per routed layer (R = valid routes;
padding, replay and shared experts excluded), the Dist-MoE explainer's count
(section 07); the rate with the shared expert's 18*T*D*F counted is reported
beside it.

Prints ONE JSON line.  Also reports the dominant kernel against its roofline
(per-kernel HIP-event timing over a second pass of the timed steps, on the
library's launch stream; beside it the average duration of the same kernel in
the committed rocprofv3 summary of this workload), the bandwidth-bound row
kernels timed cold (a third pass in which the library writes a 1 GiB buffer
before each kernel, outside its events, evicting the 256 MiB Infinity Cache),
and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "f32": 157.3}
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "mixture_experts_routed_03_amd", "csrc")

WORKLOADS = {
    # name: (config key, training)
    "bf16_train_balanced": ("bf16_fwd_balanced", True),
    "bf16_fwd_balanced": ("bf16_fwd_balanced", False),
    "bf16_fwd_fused": ("bf16_fwd_balanced", False),
    "bf16_train_zipf": ("bf16_train_zipf", True),
    "mxfp8_train_shared": ("mxfp8_train_shared", True),
    "mxfp8_ten_layer": ("mxfp8_ten_layer", True),
    "bf16_train_clamped": ("bf16_train_clamped", True),
    "mxfp8_fwd_balanced": ("mxfp8_fwd_balanced", False),
    "mxfp8_fwd_1x32": ("mxfp8_fwd_1x32", False),
    "mxfp4_fwd_balanced": ("mxfp4_fwd_balanced", False),
    "bf16_decode_t1": ("bf16_decode_t1", False),
    "bf16_decode_t8": ("bf16_decode_t8", False),
    "bf16_decode_t64": ("bf16_decode_t64", False),
    "ep8_share": ("ep8_share", True),
    "ep64_share": ("ep64_share", True),
}
CPU_EXPERTS = {"bf16": 96, "mxfp8": 3, "mxfp4": 3}

# Library timing name -> (kernel symbols in rocprofv3 traces, per precision;
# source files that define them).  A timing slot may cover several launches
# (the BF16 forward GEMMs: streaming tiles, then the hot experts' tiles).
SYMBOLS = {
    "bf16": {
        "w13_swiglu": (["moe::k_gemm_fwd<unsigned short, 0, false>", "moe::k_gemm_hot<0>",
                        "moe::k_gemm_fwd<unsigned short, 0, true>",
                        "moe::k_fwd_splitk_finish<unsigned short, 0>"],
                       ["gemm_fwd.hip", "gemm_hot.hip"]),
        "w2_scatter": (["moe::k_gemm_fwd<unsigned short, 1, false>", "moe::k_gemm_hot<1>",
                        "moe::k_gemm_fwd<unsigned short, 1, true>",
                        "moe::k_fwd_splitk_finish<unsigned short, 1>"],
                       ["gemm_fwd.hip", "gemm_hot.hip"]),
        "mega_fwd": ("moe::k_gemm_mega<unsigned short>", ["gemm_fwd.hip"]),
        "w2_bwd_mega": ("moe::k_bwd_mega<0, unsigned short, 0>", ["gemm_bwd.hip"]),
        "w13_bwd_mega": ("moe::k_bwd_mega<1, unsigned short, 0>", ["gemm_bwd.hip"]),
        "w2_dgrad_swiglu": ("moe::k_gemm_dgrad<0>", ["gemm_bwd.hip"]),
        "w13_dgrad": ("moe::k_gemm_dgrad<1>", ["gemm_bwd.hip"]),
        "w2_wgrad": (["moe::k_gemm_wgrad<unsigned short, 2, 0>", "moe::k_wgrad_hot<2>"],
                     ["gemm_bwd.hip"]),
        "w13_wgrad": (["moe::k_gemm_wgrad<unsigned short, 13, 0>", "moe::k_wgrad_hot<13>"],
                      ["gemm_bwd.hip"]),
    },
    "mxfp8": {
        "w13_swiglu": ("moe::k_mx_fwd<0, 0, 0>", ["gemm_mx.hip", "mxq.h"]),
        "mega_fwd": ("moe::k_mx_fwd<2, 0, 0>", ["gemm_mx.hip", "mxq.h"]),
        "w2_bwd_mega": ("moe::k_mx_bwd_mega<0, unsigned short, 0>", ["gemm_mx.hip", "mxq.h"]),
        "w13_bwd_mega": ("moe::k_mx_bwd_mega<1, unsigned short, 0>", ["gemm_mx.hip", "mxq.h"]),
        "w2_scatter": ("moe::k_mx_fwd<1, 0, 0>", ["gemm_mx.hip", "mxq.h"]),
        "w2_dgrad_swiglu": ("moe::k_mx_dgrad<0>", ["gemm_mx.hip", "mxq.h"]),
        "w13_dgrad": ("moe::k_mx_dgrad<1>", ["gemm_mx.hip", "mxq.h"]),
        "w2_wgrad": (["moe::k_mx_wgrad<unsigned short, 2, 0>", "moe::k_mx_wgrad_hot<2>"],
                     ["gemm_mx.hip", "mxq.h"]),
        "w13_wgrad": (["moe::k_mx_wgrad<unsigned short, 13, 0>", "moe::k_mx_wgrad_hot<13>"],
                      ["gemm_mx.hip", "mxq.h"]),
    },
    "mxfp8_1x32": {
        "w13_swiglu": ("moe::k_mx_fwd<0, 1, 0>", ["gemm_mx.hip", "mxq.h"]),
        "w2_scatter": ("moe::k_mx_fwd<1, 1, 0>", ["gemm_mx.hip", "mxq.h"]),
    },
    "mxfp4": {
        "w13_swiglu": ("moe::k_mx_fwd<0, 1, 1>", ["gemm_mx.hip", "mxq.h"]),
        "w2_scatter": ("moe::k_mx_fwd<1, 1, 1>", ["gemm_mx.hip", "mxq.h"]),
    },
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bf16_train_zipf", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-experts", type=int, default=0,
                    help="experts in the CPU-oracle sample (all their routes); 0 = default "
                         "for the precision")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pipeline", choices=("staged", "mega"), default="staged",
                    help="expert forward: two launches (W13, W2) or one fused (Mega) launch; "
                         "BF16 training: also the fused backward (one launch per projection)")
    ap.add_argument("--width", type=int, default=0,
                    help="expert width F for a width sweep (default: the workload's F; "
                         "a multiple of 128)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a reference kernel "
                         "for scaling hardware byte counters)")
    ap.add_argument("--cold-steps", type=int, default=3,
                    help="steps of the cold-cache pass (row kernels timed after an Infinity "
                         "Cache flush); 0 = skip")
    return ap.parse_args()


# ---------------------------------------------------------------- algorithmic bytes

def alg_bytes(name, m):
    """Minimum HBM bytes of one launch of kernel ``name`` for a layer with
    metadata ``m`` (R valid routes, Rp rows padded to 32 per expert, ne
    experts with rows, shapes, precision); None if not modelled.  Replay
    kernels count only for a layer that replays, the forward's column
    bundles only for a layer that saves."""
    R, Rp, ne, T, K, D, F = m["R"], m["Rp"], m["ne"], m["T"], m["K"], m["D"], m["F"]
    es, dwb, mx, rep = m["es"], m["dwb"], m["mx"], m["replay"]
    ab, wb = m["ab"], m["wb"]     # bytes per quantized activation / weight value
    replay = name.startswith("replay_")
    if replay:
        if not rep:
            return 0
        name = name[len("replay_"):]
    elif name in ("bundle_x", "bundle_h2") and rep:
        return 0

    def q(n):  # E4M3 (or packed E2M1) codes plus one E8M0 byte per 32 values
        return int(n * ab) + n // 32

    if replay and mx and name == "w13_swiglu":   # rebuilds h1 and bf16 h2 only
        return int(ne * 2 * F * D * wb) + q(R * D) + R * 2 * F * 2 + R * F * 2

    w13 = int(ne * 2 * F * D * wb)
    w2 = int(ne * D * F * wb)
    common = {
        "route": T * K * 4 * 2 + R * 4 * 2,
        "zero_y32": T * D * 4,
        "fused_finish": T * D * 4 + T * D * es + T * K * 8,
        "gather": T * D * es + R * D * es,
        "combine": T * K * D * es + T * D * es + T * K * 8,
        "combine_bwd": T * D * es + T * K * D * es + R * D * es + T * K * 8,
        "dx_reduce": R * D * 4 + T * D * es,
    }
    if name in common:
        return common[name]
    if not mx:
        return {
            "w13_swiglu": w13 + T * D * es + R * 2 * F * es + R * F * es,
            "w2_scatter": w2 + R * F * es + R * D * es,
            # fused: x rows, h1 and h2 written, h3 slots; h2 is read back from L2
            "mega_fwd": w13 + w2 + T * D * es + R * 2 * F * es + R * F * es + R * D * es,
            "w2_fused": w2 + R * F * es + T * D * 4 + R * 4,
            "w2_dgrad_swiglu": w2 + R * D * es + 2 * R * 2 * F * es + R * F * es,
            "w2_wgrad": ne * D * F * dwb + R * D * es + R * F * es,
            "w13_dgrad": w13 + R * 2 * F * es + R * D * 4,
            "w13_wgrad": ne * 2 * F * D * dwb + R * 2 * F * es + R * D * es,
            # fused backward: the h2 rows W2 DGRAD rebuilds are read back from
            # L2; dH1 and the x rows are counted once
            "w2_bwd_mega": (w2 + R * D * es + 2 * R * 2 * F * es + R * F * es
                            + ne * D * F * dwb),
            "w13_bwd_mega": w13 + R * 2 * F * es + R * D * 4 + ne * 2 * F * D * dwb + R * D * es,
        }.get(name)
    return {
        "quant_x": T * D * 2 + q(R * D),
        "bundle_x": T * D * 2 + q(Rp * D),
        # h1, the h2 row blocks (quantized in the epilogue) and, in training,
        # bf16 h2 for its column bundle
        "w13_swiglu": w13 + q(R * D) + R * 2 * F * 2 + q(R * F) + (R * F * 2 if m["train"] else 0),
        # fused (Mega) forward: both GEMMs' operands and outputs, h2 handed over in L2
        "mega_fwd": (w13 + w2 + q(R * D) + R * 2 * F * 2 + q(R * F)
                     + (R * F * 2 if m["train"] else 0) + R * D * 2),
        "bundle_h2": R * F * 2 + q(Rp * F),
        "quant_h2": R * F * 2 + q(R * F),
        "w2_scatter": w2 + q(R * F) + R * D * 2,
        "w2_fused": w2 + q(R * F) + T * D * 4 + R * 4,
        "quant_dh3": R * D * 2 + q(R * D),
        "bundle_dh3": R * D * 2 + q(Rp * D),
        "w2_dgrad_swiglu": w2 + q(R * D) + 2 * R * 2 * F * 2,
        "w2_wgrad": ne * D * F * dwb + q(Rp * D) + q(Rp * F),
        "quant_dh1": R * 2 * F * 2 + q(R * 2 * F),
        "bundle_dh1": R * 2 * F * 2 + q(Rp * 2 * F),
        "w13_dgrad": w13 + q(R * 2 * F) + R * D * 4,
        "w13_wgrad": ne * 2 * F * D * dwb + q(Rp * 2 * F) + q(Rp * D),
        "w2_bwd_mega": w2 + q(R * D) + 2 * R * 2 * F * 2 + ne * D * F * dwb + q(Rp * D) + q(Rp * F),
        "w13_bwd_mega": w13 + q(R * 2 * F) + R * D * 4 + ne * 2 * F * D * dwb + q(Rp * 2 * F)
                        + q(Rp * D),
    }.get(name)


def kernel_flops(name, m):
    R, D, F = m["R"], m["D"], m["F"]
    if name.startswith("replay_"):
        if not m["replay"]:
            return 0
        name = name[len("replay_"):]
    if name in ("w13_swiglu", "w13_dgrad", "w13_wgrad"):
        return 2 * R * 2 * F * D
    if name == "mega_fwd":
        return 6 * R * D * F
    if name == "w2_bwd_mega":
        return 4 * R * D * F
    if name == "w13_bwd_mega":
        return 8 * R * D * F
    if name in ("w2_scatter", "w2_fused", "w2_dgrad_swiglu", "w2_wgrad"):
        return 2 * R * D * F
    return None


def measured_profile(workload, prec, kname):
    """(HBM bytes per launch, average launch microseconds) of timing slot
    ``kname`` from the committed rocprofv3 summary of this workload, summed
    over the slot's kernels, if the summary exists and the code of those
    kernels (comments ignored) is unchanged since it was taken; else
    (None, None)."""
    from mixture_experts_routed_03_amd.profsum import source_hashes
    syms, files = SYMBOLS.get(prec, {}).get(kname, (None, None))
    if syms is None:
        return None, None
    if isinstance(syms, str):
        syms = [syms]
    prof_dir = os.path.join(HERE, "profiles")
    if not os.path.isdir(prof_dir):
        return None, None
    for fn in sorted(os.listdir(prof_dir)):
        if not fn.startswith(workload + "_") or not fn.endswith(".md"):
            continue
        with open(os.path.join(prof_dir, fn)) as fh:
            text = fh.read()
        mt = re.search(r"```json\n(.*?)\n```", text, re.S)
        if not mt:
            continue
        blob = json.loads(mt.group(1))
        shas = blob.get("src_code_sha256_16", {})
        now = source_hashes(files + ["common.h"])
        if any(shas.get(f) != h for f, h in now.items()):
            return None, None
        traffic = [blob.get("traffic_bytes", {}).get(s) for s in syms]
        avg = [blob.get("avg_us_working", {}).get(s) for s in syms]
        if not any(avg):   # a summary of another pipeline of this workload
            continue
        tb = (int(sum(sum(t) / len(t) for t in traffic if t))
              if any(traffic) else None)
        us = round(sum(a for a in avg if a), 2)
        return tb, us
    return None, None


# ---------------------------------------------------------------- workloads

def layer_meta(layer, rb, replay, T):
    import numpy as np
    counts = rb["counts"].astype(np.int64)
    return {"R": int(rb["R"]), "Rp": int(rb["poffsets"][-1]), "ne": int((counts > 0).sum()),
            "train": bool(layer.training),
            "T": T, "K": layer.K, "D": layer.D, "F": layer.F,
            "es": 4 if layer.prec == "f32" else 2,
            "dwb": 4 if layer.dw_dtype.itemsize == 4 else 2,
            "mx": layer.prec in ("mxfp8", "mxfp4"), "replay": bool(replay),
            # bytes per value of quantized activations and of weights (codes +
            # exponents: 32x32 blocks one per 1024 values, 1x32 one per 32)
            "ab": 0.5 if layer.prec == "mxfp4" else 1.0,
            "wb": (0.5 + 1 / 32 if layer.prec == "mxfp4" else
                   1 + 1 / 32 if layer.mx_w1x32 else 1 + 1 / 1024)
                  if layer.prec in ("mxfp8", "mxfp4") else (4 if layer.prec == "f32" else 2),
            "max_rows": int(counts.max()) if counts.size else 0}


def setup(args, dev):
    """Build the workload; returns (step, plans, meta_fn, useful_flops_fn,
    cpu_fn, info) where plans maps a label to a MoeLayer whose per-kernel
    timings are read, meta_fn() lists (label, per-layer metadata)."""
    import torch

    from mixture_experts_routed_03_amd import binding as B
    from mixture_experts_routed_03_amd import workloads as wl

    cfg_key, training = WORKLOADS[args.workload]
    cfg = wl.CONFIGS[cfg_key]
    if args.width:
        if args.width % 128:
            raise SystemExit("--width must be a multiple of 128")
        cfg = wl.scaled(cfg, F=args.width)
    T, D, F, E, K = cfg.T, cfg.D, cfg.F, cfg.E, cfg.K
    bf = torch.bfloat16

    if args.workload == "mxfp8_ten_layer":
        L = cfg.layers
        budget = wl.ten_layer_budget(cfg)
        st = B.MoeStack(L, T, D, F, E, K, "mxfp8", arena_budget=budget, device=dev)
        mega = args.pipeline == "mega"
        lays, preps = [], []
        for l in range(L):
            lay = wl.make_layer(cfg, l, device=dev)
            preps.append(st.layer.prepare(lay["w13"], lay["w2"]))
            if l == 0:   # the CPU-oracle sample's experts, in bf16 on the host
                n_cpu = args.cpu_experts or CPU_EXPERTS["mxfp8"]
                keep0 = {k: lay[k][:n_cpu].cpu() for k in ("w13", "w2")}
            del lay["w13"], lay["w2"]
            lays.append(lay)
            torch.cuda.synchronize()
        ys = [torch.empty((T, D), dtype=bf, device=dev) for _ in range(L)]
        # one set of weight-gradient buffers, handed over after each layer's backward
        dx = torch.empty((T, D), dtype=bf, device=dev)
        dw13 = torch.empty((E, 2 * F, D), dtype=bf, device=dev)
        dw2 = torch.empty((E, D, F), dtype=bf, device=dev)
        ds = torch.empty((T, K), dtype=torch.float32, device=dev)

        def step():
            for l in range(L):
                st.route(l, lays[l]["ids"])
                st.forward(l, lays[l]["x"], None, None, lays[l]["scores"], ys[l],
                           prepared=preps[l], mega=mega)
            for l in reversed(range(L)):
                st.backward(l, lays[l]["x"], lays[l]["scores"], lays[l]["dy"], None, None, dx,
                            dw13, dw2, ds, prepared=preps[l], flags=B.BWD_MEGA if mega else 0)

        def meta():
            out = []
            for l in range(L):
                rb = st.readback(l, T)
                out.append(("", layer_meta(st.layer, rb, st.status(l)[1], T)))
            return out

        def cpu():
            lay0 = dict(lays[0], **keep0)
            return cpu_baseline(lay0, cfg, True, n_cpu, "layer 0 of 10, ")

        info = {"layers": L, "arena_budget_bytes": budget}
        return step, {"": st.layer}, meta, cpu, info, cfg, training

    lay = wl.make_layer(cfg, 0, device=dev, grads=training)
    layer = B.MoeLayer(T, D, F, E, K, cfg.prec, training=training, device=dev,
                       swiglu_limit=cfg.swiglu_limit, mx_w1x32=cfg.mx_w1x32)
    if cfg.prec in ("mxfp8", "mxfp4"):
        layer.prepare(lay["w13"], lay["w2"])
    act = layer.act_dtype
    y = torch.empty((T, D), dtype=act, device=dev)
    plans = {"": layer}
    if training:
        dx = torch.empty((T, D), dtype=act, device=dev)
        dw13 = torch.empty((E, 2 * F, D), dtype=layer.dw_dtype, device=dev)
        dw2 = torch.empty((E, D, F), dtype=layer.dw_dtype, device=dev)
        dsc = torch.empty((T, K), dtype=torch.float32, device=dev)
    shared = None
    if cfg.shared_expert:
        shared = B.MoeLayer(T, D, F, 1, 1, "bf16", training=training, device=dev)
        plans["shared:"] = shared
        sh_ids = torch.zeros((T, 1), dtype=torch.int32, device=dev)
        sh_sc = torch.ones((T, 1), dtype=torch.float32, device=dev)
        ysh = torch.empty((T, D), dtype=bf, device=dev)
        dws13 = torch.empty_like(lay["w13_shared"])
        dws2 = torch.empty_like(lay["w2_shared"])

    fused = args.workload == "bf16_fwd_fused"
    y32 = torch.empty((T, D), dtype=torch.float32, device=dev) if fused else None
    # the fused backward (BF16 and MXFP8 plans)
    bwd_flags = B.BWD_MEGA if args.pipeline == "mega" else 0

    def step():
        if fused:
            layer.route(lay["ids"])
            layer.forward_fused(lay["x"], lay["w13"], lay["w2"], lay["scores"], y, y32=y32)
            return
        if shared is not None:
            shared.route(sh_ids)
            shared.forward(lay["x"], lay["w13_shared"], lay["w2_shared"])
            shared.combine(sh_sc, ysh)
        layer.route(lay["ids"])
        if args.pipeline == "mega":
            layer.forward_mega(lay["x"], lay["w13"], lay["w2"])
        else:
            layer.forward(lay["x"], lay["w13"], lay["w2"])
        layer.combine(lay["scores"], y, y_addend=ysh if shared is not None else None)
        if training:
            layer.backward(lay["x"], lay["scores"], lay["dy"], lay["w13"], lay["w2"], dx, dw13,
                           dw2, dsc, flags=bwd_flags)
            if shared is not None:
                shared.backward(lay["x"], sh_sc, lay["dy"], lay["w13_shared"], lay["w2_shared"],
                                dx, dws13, dws2, None, flags=B.BWD_ACCUMULATE_DX)

    def meta():
        out = [("", layer_meta(layer, layer.readback(T), layer.status()[1] if training else 0, T))]
        if shared is not None:
            out.append(("shared:", layer_meta(shared, shared.readback(T), shared.status()[1], T)))
        return out

    def cpu():
        return cpu_baseline(lay, cfg, training,
                            args.cpu_experts or CPU_EXPERTS.get(cfg.prec, CPU_EXPERTS["bf16"]),
                            "routed experts only, " if shared is not None else "")

    return step, plans, meta, cpu, {}, cfg, training


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert "
              "parallelism over xGMI is a design note only). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_routed_03_amd import binding as B

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    step, plans, meta_fn, cpu_fn, info, cfg, training = setup(args, dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    metas = meta_fn()

    copy_gbs = None
    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record()
        dst.copy_(src)  # reads and writes copy_probe_mb MiB each
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = round(2 * n * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
        del src, dst

    # ---- timed region: K steps, bracketed by synchronize on both sides; an
    # event at each window boundary (up to 5 windows) gives window means
    n_win = min(5, args.steps)
    bounds = [round(i * args.steps / n_win) for i in range(n_win + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in bounds]
    torch.cuda.reset_peak_memory_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host = 0.0
    evs[0].record()
    w = 1
    for i in range(args.steps):
        h0 = time.perf_counter()
        step()
        host += time.perf_counter() - h0
        if i + 1 == bounds[w]:
            evs[w].record()
            w += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    win_ms = [evs[i].elapsed_time(evs[i + 1]) / (bounds[i + 1] - bounds[i]) for i in range(n_win)]
    peak_gib = torch.cuda.max_memory_allocated() / 2**30

    # ---- second pass with per-kernel events (on the library's launch stream)
    for p in plans.values():
        B.moe_timing_enable(p.plan, True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = {}
    for label, p in plans.items():
        for name, (tot, n) in B.moe_timing_read(p.plan).items():
            ktimes[label + name] = (tot, n)
        B.moe_timing_enable(p.plan, False)

    # ---- third pass: the same steps with the Infinity Cache flushed before
    # every kernel (outside its events); the row kernels' cold rates
    cold = {}
    if args.cold_steps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for p in plans.values():
            B.moe_timing_enable(p.plan, True)
            B.moe_timing_flush(p.plan, flush)
        for _ in range(args.cold_steps):
            step()
        torch.cuda.synchronize()
        for label, p in plans.items():
            if label:
                B.moe_timing_enable(p.plan, False)
                B.moe_timing_flush(p.plan, None)
                continue
            for name, (tot, n) in B.moe_timing_read(p.plan).items():
                if name in ("route", "gather", "combine", "combine_bwd", "dx_reduce") and n:
                    bsum = sum(alg_bytes(name, m) for lab, m in metas if lab == "")
                    ms = tot / args.cold_steps
                    cold[name] = {"us": round(tot / n * 1e3, 1),
                                  "GB/s": round(bsum / (ms * 1e-3) / 1e9, 1)}
            B.moe_timing_enable(p.plan, False)
            B.moe_timing_flush(p.plan, None)
        del flush

    # Useful work: routed layers only (the Dist-MoE explainer's count, section
    # 07, excludes shared experts, padding and replay); the shared expert's
    # time stays in the step.
    mult = 3 if training else 1
    useful = sum(6 * m["R"] * m["D"] * m["F"] * mult for lab, m in metas if lab == "")
    shared_flops = sum(6 * m["R"] * m["D"] * m["F"] * mult for lab, m in metas if lab != "")
    value = useful / (ms_step * 1e-3) / 1e12

    # per-kernel: algorithmic bytes and flops per step, time per step
    kernels = {}
    for key, (tot, n) in ktimes.items():
        if n == 0:
            continue
        label, name = (key.split(":", 1)[0] + ":", key.split(":", 1)[1]) if ":" in key else ("", key)
        ms = tot / args.steps
        ent = {"ms_per_step": round(ms, 4), "launches_per_step": n // args.steps,
               "avg_ms": round(tot / n, 4)}
        bsum, fsum, known = 0, 0, True
        for lab, m in metas:
            if lab != label:
                continue
            b = alg_bytes(name, m)
            if b is None:
                known = False
                break
            bsum += b
            f = kernel_flops(name, m)
            fsum += f or 0
        if known:
            ent["alg_bytes_per_step"] = int(bsum)
            ent["GB/s"] = round(bsum / (ms * 1e-3) / 1e9, 1)
            if fsum:
                ent["alg_flops_per_step"] = int(fsum)
                ent["TFLOP/s"] = round(fsum / (ms * 1e-3) / 1e12, 2)
        kernels[key] = ent
    dom = max((k for k in kernels if "GB/s" in kernels[k]), key=lambda k: kernels[k]["ms_per_step"])
    dom_name = dom.split(":", 1)[-1]
    n_launch = kernels[dom]["launches_per_step"]
    alg_per_launch = kernels[dom]["alg_bytes_per_step"] / max(1, n_launch)
    ach = kernels[dom]["GB/s"]
    prec_dom = "bf16" if dom.startswith("shared:") else cfg.prec
    # counters were taken at each workload's own width
    sym_key = "mxfp8_1x32" if prec_dom == "mxfp8" and cfg.mx_w1x32 else prec_dom
    traffic, prof_us = ((None, None) if args.width else
                        measured_profile(args.workload, sym_key, dom_name))
    roofline = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": int(alg_per_launch),
                "avg_launch_ms": kernels[dom]["avg_ms"],
                # the same kernel's average working-dispatch duration in the
                # committed rocprofv3 summary of this workload (null when its
                # code changed since)
                "profile_avg_launch_ms": None if prof_us is None else round(prof_us / 1e3, 4)}
    # A kernel whose useful FLOPs take longer at the MFMA peak than its bytes
    # at the HBM peak (many rows per expert) is reported against the MFMA peak.
    tfl = kernels[dom].get("TFLOP/s")
    if tfl:
        peak_t = PEAK_TFLOPS[prec_dom]
        if tfl / peak_t > ach / PEAK_HBM_GBS:
            roofline.update({"bound": "mfma", "achieved": tfl, "peak": peak_t, "unit": "TFLOP/s",
                             "frac": round(tfl / peak_t, 4),
                             "alg_flops_per_launch": int(kernels[dom]["alg_flops_per_step"] /
                                                         max(1, n_launch))})

    # Whole-step roofline: t* = max(useful FLOPs / MFMA peak, algorithmic
    # bytes of every modelled kernel / HBM peak).
    alg_step = sum(k.get("alg_bytes_per_step", 0) for k in kernels.values())
    t_flop = useful / (PEAK_TFLOPS[cfg.prec] * 1e12) * 1e3
    t_byte = alg_step / (PEAK_HBM_GBS * 1e9) * 1e3
    step_roof = {"t_star_ms": round(max(t_flop, t_byte), 4),
                 "bound": "hbm" if t_byte >= t_flop else "mfma",
                 "alg_bytes_per_step": int(alg_step),
                 "frac": round(max(t_flop, t_byte) / ms_step, 4)}

    cpu = None if args.no_cpu_baseline else cpu_fn()

    m0 = metas[0][1]
    prec = cfg.prec
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
        "dtype": prec,
        "data": "synthetic (seeded; N(0,1) tokens, N(0,1/fan_in) weights, "
                + ("Zipf-skewed" if cfg.zipf != (None,) else "balanced top-6") + " routing)",
        "config": {"workload": f"{args.workload}: T={cfg.T} D={cfg.D} F={cfg.F} E={cfg.E} "
                               f"K={cfg.K} {'fwd+bwd' if training else 'fwd'}"
                               + (f", {info['layers']} layers" if "layers" in info else "")
                               + (", + shared BF16 expert" if cfg.shared_expert else "")
                               + (f", SwiGLU clamped at {cfg.swiglu_limit:g}"
                                  if cfg.swiglu_limit else "")
                               + ((", fused (Mega) forward and backward"
                                   if training else ", fused (Mega) forward")
                                  if args.pipeline == "mega" else ""),
                   "routes_per_layer": [m["R"] for lab, m in metas if lab == ""],
                   "nonempty_experts": [m["ne"] for lab, m in metas if lab == ""],
                   "max_rows": max(m["max_rows"] for lab, m in metas if lab == ""),
                   "replayed_layers": [int(m["replay"]) for lab, m in metas if lab == ""],
                   "dw_dtype": "bf16" if m0["dwb"] == 2 else "f32", **info},
        "mfma_peak_frac": round(value / PEAK_TFLOPS[prec], 4),
        "tflops_incl_shared_expert": (round((useful + shared_flops) / (ms_step * 1e-3) / 1e12, 2)
                                      if shared_flops else None),
        # routing itself moves ~0.2 MB (ids in, permutation out): its time is
        # launch latency, so it is reported in microseconds beside its GB/s;
        # the bandwidth-bound half of the router is the permuted-row gather
        # (inside the W13 loader in the forward, a kernel of its own in the
        # BF16 backward)
        "route_GBps": kernels.get("route", {}).get("GB/s"),
        "route_us": (round(kernels["route"]["avg_ms"] * 1e3, 1) if "route" in kernels else None),
        "gather_GBps": kernels.get("gather", {}).get("GB/s"),
        # bandwidth-bound row kernels with the Infinity Cache flushed before
        # each launch (per-launch microseconds, algorithmic GB/s)
        "row_kernels_cold": cold or None,
        "wall_s_timed": round(wall, 3),
        "window_ms_per_step": [round(v, 4) for v in win_ms],
        "median_window_ms": round(sorted(win_ms)[len(win_ms) // 2], 4),
        "host_enqueue_ms_per_step": round(host / args.steps * 1e3, 3),
        "peak_device_GiB": round(peak_gib, 2),
        "copy_probe_GBps": copy_gbs,
        "step_roofline": step_roof,
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(lay, cfg, training, n_exp, what=""):
    """The fp64 oracle, as it stands, on the routes of the first n_exp experts
    (all their tokens): forward (+ backward), wall time on the host cores."""
    import numpy as np

    from oracle import moe as om
    from oracle import mx as omx
    from oracle import mxfp4 as o4

    ora = {"mxfp8": omx, "mxfp4": o4}.get(cfg.prec, om)
    ids = lay["ids"].cpu().numpy()
    ids_s = np.where((ids >= 0) & (ids < n_exp), ids, -1).astype(np.int32)
    R_s = int((ids_s >= 0).sum())
    x = lay["x"].cpu()
    sc = lay["scores"].cpu()
    w13 = lay["w13"][:n_exp].cpu()
    w2 = lay["w2"][:n_exp].cpu()
    clamp = {"w1x32": True} if cfg.mx_w1x32 else {}
    if cfg.swiglu_limit:
        clamp.update({"limit": cfg.swiglu_limit} if cfg.prec in ("mxfp8", "mxfp4") else
                     {"limit": cfg.swiglu_limit, "act": omx.bf16_round})
    if cfg.prec != "mxfp4":
        clamp["keep"] = True
    t0 = time.perf_counter()
    out = ora.forward(x, ids_s, sc, w13, w2, **clamp)
    if training:
        y, cache = out
        ora.backward(lay["dy"].cpu(), x, ids_s, sc, w13, w2, cache)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    flops = 6 * R_s * cfg.D * cfg.F * (3 if training else 1)
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{what}routes of experts 0..{n_exp - 1} ({R_s} of "
                      f"{int((ids >= 0).sum())} routes), "
                      f"{'forward+backward' if training else 'forward'}, fp64 NumPy"
                      + (f", quantization-faithful {cfg.prec.upper()}"
                         if cfg.prec in ("mxfp8", "mxfp4") else "")}


if __name__ == "__main__":
    main()
