"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only draws numbers: routing ids and scores, token rows, expert
weights and output gradients.  It holds none of the layer's arithmetic, so both
the GPU library's tests and the CPU oracle read exactly the tensors made here.

Shapes and value distributions follow the workloads the Dist-MoE explainer
describes (section 07: T = 2,048 tokens, D = 7,168, E = 384 experts, top-6)
and the grouped-GEMM blog's routing (section 1: top-k of router scores, softmax
over the selected scores).  Recipe:

* routing ``uniform``: per token, E i.i.d. N(0,1) logits; the K largest give the
  ids (uniform without replacement), and the scores are the softmax of those K
  logits (largest first).
* routing ``zipf`` (exponent s): expert ``perm[i]`` has weight (i+1)^-s over a
  seeded permutation ``perm``; K distinct ids per token come from Gumbel-top-K
  on the log weights (sequential sampling without replacement); scores are the
  softmax of K sorted N(0,1) logits.  s = 0 is uniform.
* padding: exactly ``n_pad`` (token, slot) pairs, drawn uniformly without
  replacement, get id -1 and score 0.
* dense tensors: N(0, std^2), rounded once to the storage dtype (round to
  nearest even).  Weights use std = 1/sqrt(fan_in); each expert's matrix is
  drawn from its own stream so one expert can be regenerated alone.

CPU tensors come from NumPy PCG64; CUDA tensors from torch's device generator
(much faster for the 34 GB of config-2 weights).  Either way a tensor is fully
determined by (seed, shape, device type).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Stream ids mixed into the seed so every tensor of a layer gets its own stream.
_STREAMS = {
    "routing": 1, "x": 2, "w13": 3, "w2": 4, "dy": 5, "pad": 6,
    "w13_shared": 7, "w2_shared": 8, "zipf_perm": 9,
}


def stream_seed(seed: int, layer: int, name: str) -> int:
    """A 63-bit seed for tensor ``name`` of layer ``layer`` under base ``seed``."""
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(layer, _STREAMS[name]))
    return int(ss.generate_state(2, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=1, keepdims=True)


def make_routing(T: int, E: int, K: int, *, zipf_s: float | None = None,
                 n_pad: int = 0, seed: int = 0, layer: int = 0):
    """Return ``ids`` int32 [T,K] and ``scores`` float32 [T,K] (NumPy arrays)."""
    if K > E:
        raise ValueError("K distinct experts per token need K <= E")
    rng = np.random.Generator(np.random.PCG64(stream_seed(seed, layer, "routing")))
    if zipf_s is None:
        logits = rng.standard_normal((T, E))
        idx = np.argsort(-logits, axis=1, kind="stable")[:, :K]
        sel = np.take_along_axis(logits, idx, axis=1)
        ids = idx
        scores = _softmax_rows(sel)
    else:
        prng = np.random.Generator(np.random.PCG64(stream_seed(seed, layer, "zipf_perm")))
        perm = prng.permutation(E)
        logw = np.empty(E)
        logw[perm] = -float(zipf_s) * np.log(np.arange(1, E + 1, dtype=np.float64))
        gumbel = -np.log(-np.log(rng.uniform(size=(T, E)).clip(1e-300, 1.0)))
        keys = logw[None, :] + gumbel
        ids = np.argsort(-keys, axis=1, kind="stable")[:, :K]
        sel = -np.sort(-rng.standard_normal((T, K)), axis=1)
        scores = _softmax_rows(sel)
    ids = ids.astype(np.int32)
    scores = scores.astype(np.float32)
    if n_pad:
        if n_pad > T * K:
            raise ValueError("more padding routes than routes")
        prng = np.random.Generator(np.random.PCG64(stream_seed(seed, layer, "pad")))
        flat = prng.choice(T * K, size=n_pad, replace=False)
        ids.reshape(-1)[flat] = -1
        scores.reshape(-1)[flat] = 0.0
    return ids, scores


def normal(shape, std: float, *, seed: int, dtype, device="cpu", chunk_rows: int | None = None):
    """A torch tensor of N(0, std^2) values in ``dtype`` on ``device``.

    CUDA tensors are filled chunk by chunk along dim 0 (bounded fp32 staging).
    """
    import torch

    shape = tuple(int(s) for s in shape)
    dev = torch.device(device)
    if dev.type == "cpu":
        rng = np.random.Generator(np.random.PCG64(seed))
        a = rng.standard_normal(shape, dtype=np.float32)
        a *= np.float32(std)
        return torch.from_numpy(a).to(dtype)
    out = torch.empty(shape, dtype=dtype, device=dev)
    if out.numel() == 0:
        return out
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    rows = shape[0]
    per_row = max(1, out.numel() // rows)
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 28) // per_row)  # <= 1 GiB of fp32 staging
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        tmp = torch.randn((r1 - r0,) + shape[1:], generator=g, device=dev, dtype=torch.float32)
        tmp.mul_(std)
        out[r0:r1].copy_(tmp)
        del tmp
    return out


def expert_normal(E, shape, std: float, *, seed: int, dtype, device="cpu", experts=None):
    """Expert weights [E, *shape] ~ N(0, std^2), expert e drawn from its own
    stream (seed, e), so any one expert can be regenerated alone.  With
    ``experts`` only those experts are drawn (stacked in that order)."""
    import torch

    idx = range(E) if experts is None else list(experts)
    out = torch.empty((len(idx),) + tuple(shape), dtype=dtype, device=torch.device(device))
    for i, e in enumerate(idx):
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(int(e),))
        es = int(ss.generate_state(2, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))
        out[i] = normal(shape, std, seed=es, dtype=dtype, device=device)
    return out


@dataclass(frozen=True)
class Config:
    """One workload: layer shape, precision, routing recipe and phases."""

    name: str
    T: int
    D: int
    F: int
    E: int
    K: int
    prec: str                      # "f32" | "bf16" | "mxfp8" | "mxfp4" (inference)
    zipf: tuple = (None,)          # per-layer routing: None = uniform top-K, else Zipf exponent
    pad_frac: float = 0.0
    training: bool = False
    layers: int = 1
    shared_expert: bool = False
    seed: int = 0
    note: str = ""
    swiglu_limit: float = 0.0      # > 0: clamped SwiGLU at this limit
    mx_w1x32: bool = False         # MXFP8 inference with 1x32-block prepared weights

    @property
    def n_pad(self) -> int:
        return int(round(self.pad_frac * self.T * self.K))

    def zipf_for(self, layer: int):
        return self.zipf[layer % len(self.zipf)]


CONFIGS = {
    "tiny_f32": Config("tiny_f32", 256, 256, 128, 8, 2, "f32", pad_frac=0.05,
                       note="tiny fp32 layer, 5% padded routes, forward only"),
    "bf16_fwd_balanced": Config("bf16_fwd_balanced", 2048, 7168, 2048, 384, 6, "bf16",
                                note="BF16 forward, balanced routing"),
    "bf16_train_zipf": Config("bf16_train_zipf", 2048, 7168, 2048, 384, 6, "bf16",
                              zipf=(1.2,), training=True,
                              note="BF16 forward+backward, Zipf(1.2) skewed routing"),
    "mxfp8_train_shared": Config("mxfp8_train_shared", 2048, 7168, 2048, 384, 6, "mxfp8",
                                 training=True, shared_expert=True,
                                 note="MXFP8 forward+backward, balanced, plus a shared BF16 expert"),
    "mxfp8_ten_layer": Config("mxfp8_ten_layer", 2048, 7168, 2048, 384, 6, "mxfp8",
                              zipf=(0.0, 0.6, 1.0, 1.4), training=True, layers=10,
                              note="ten MXFP8 layers, forwards then backwards, byte budget"),
    # One GPU's share of the same routed rows (R = 12,288) under expert
    # parallelism over 8 or 64 GPUs: 48 experts of ~256 rows, or 6 experts
    # of 2,048 rows (every token routes to all six).
    "bf16_train_clamped": Config("bf16_train_clamped", 2048, 7168, 2048, 384, 6, "bf16",
                                 training=True, swiglu_limit=1.0,
                                 note="balanced BF16 training layer with the SwiGLU clamped at "
                                      "1.0 (about a third of h1 clamped)"),
    "mxfp8_fwd_balanced": Config("mxfp8_fwd_balanced", 2048, 7168, 2048, 384, 6, "mxfp8",
                                 note="MXFP8 inference forward, 32x32-block weights"),
    "mxfp8_fwd_1x32": Config("mxfp8_fwd_1x32", 2048, 7168, 2048, 384, 6, "mxfp8", mx_w1x32=True,
                             note="MXFP8 inference forward, 1x32-block weights"),
    "mxfp4_fwd_balanced": Config("mxfp4_fwd_balanced", 2048, 7168, 2048, 384, 6, "mxfp4",
                                 note="MXFP4 inference forward: E2M1 activations and 1x32 weights"),
    "bf16_decode_t1": Config("bf16_decode_t1", 1, 7168, 2048, 384, 6, "bf16",
                             note="decode step: one token, six routed experts (one row each)"),
    "bf16_decode_t8": Config("bf16_decode_t8", 8, 7168, 2048, 384, 6, "bf16",
                             note="decode step: eight tokens, about one row per active expert"),
    "bf16_decode_t64": Config("bf16_decode_t64", 64, 7168, 2048, 384, 6, "bf16",
                              note="decode step: 64 tokens, about one row per expert"),
    "ep8_share": Config("ep8_share", 2048, 7168, 2048, 48, 6, "bf16", training=True,
                        note="EP8 share: 48 experts, ~256 rows each, BF16 forward+backward"),
    "ep64_share": Config("ep64_share", 2048, 7168, 2048, 6, 6, "bf16", training=True,
                         note="EP64 share: 6 experts, 2048 rows each, BF16 forward+backward"),
}


def ten_layer_budget(cfg: Config) -> int:
    """Arena budget of the ten-layer workload: 4.5 x the saved MXFP8 state of
    one layer with R = T*K routes and R_pad = T*K + 16*E padded rows (x and
    h2 column bundles with their exponents, BF16 h1), rounded up to 128 B."""
    R, Rp, D, F = cfg.T * cfg.K, cfg.T * cfg.K + 16 * cfg.E, cfg.D, cfg.F
    state = D * Rp + D * Rp // 32 + R * 2 * F * 2 + F * Rp + F * Rp // 32
    return -(-int(4.5 * state) // 128) * 128


def torch_dtype(prec: str):
    import torch
    return torch.float32 if prec == "f32" else torch.bfloat16


def make_layer(cfg: Config, layer: int = 0, device="cpu", *, T: int | None = None,
               weights: bool = True, grads: bool | None = None):
    """All inputs of one layer as a dict of torch tensors on ``device``.

    Keys: ids (int32 [T,K]), scores (f32 [T,K]), x [T,D], w13 [E,2F,D],
    w2 [E,D,F], and dy [T,D] when training.  MXFP8 layers carry bf16 weights
    (prepared to MXFP8 by the library).  ``T`` overrides the token count.
    """
    import torch

    T = cfg.T if T is None else T
    dt = torch.float32 if cfg.prec == "f32" else torch.bfloat16
    n_pad = int(round(cfg.pad_frac * T * cfg.K))
    ids, scores = make_routing(T, cfg.E, cfg.K, zipf_s=cfg.zipf_for(layer), n_pad=n_pad,
                               seed=cfg.seed, layer=layer)
    out = {
        "ids": torch.from_numpy(ids).to(device),
        "scores": torch.from_numpy(scores).to(device),
        "x": normal((T, cfg.D), 1.0, seed=stream_seed(cfg.seed, layer, "x"), dtype=dt, device=device),
    }
    if weights:
        out["w13"] = layer_weight(cfg, layer, "w13", device)
        out["w2"] = layer_weight(cfg, layer, "w2", device)
    if grads if grads is not None else cfg.training:
        out["dy"] = normal((T, cfg.D), 1.0, seed=stream_seed(cfg.seed, layer, "dy"), dtype=dt,
                           device=device)
    if cfg.shared_expert and weights:
        out["w13_shared"] = normal((1, 2 * cfg.F, cfg.D), 1.0 / math.sqrt(cfg.D),
                                   seed=stream_seed(cfg.seed, layer, "w13_shared"),
                                   dtype=torch.bfloat16, device=device)
        out["w2_shared"] = normal((1, cfg.D, cfg.F), 1.0 / math.sqrt(cfg.F),
                                  seed=stream_seed(cfg.seed, layer, "w2_shared"),
                                  dtype=torch.bfloat16, device=device)
    return out


def layer_weight(cfg: Config, layer: int, name: str, device="cpu", experts=None):
    """W13 [E, 2F, D] or W2 [E, D, F] of a layer (or the listed experts of it)."""
    dt = torch_dtype(cfg.prec)
    if name == "w13":
        shape, std = (2 * cfg.F, cfg.D), 1.0 / math.sqrt(cfg.D)
    else:
        shape, std = (cfg.D, cfg.F), 1.0 / math.sqrt(cfg.F)
    return expert_normal(cfg.E, shape, std, seed=stream_seed(cfg.seed, layer, name), dtype=dt,
                         device=device, experts=experts)


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller parity shapes)."""
    d = {f: getattr(cfg, f) for f in cfg.__dataclass_fields__}
    d.update(kw)
    return Config(**d)
