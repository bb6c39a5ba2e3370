"""GPU parity of the fused (Mega) expert forward (Dist-MoE explainer,
section 05, "Kernel Pipelines: Staged and Mega"): W13 + SwiGLU and W2 run
as records of one persistent grid, W2 records waiting on per-expert
readiness counters.  The fused launch uses the same tiles and epilogues as
the staged pair, so where the staged plan does not split the contraction
its route slots (and the combined y) must equal the staged forward's bit
for bit (BF16, F32, MXFP8 32x32 and 1x32, MXFP4); both are also checked
against the fp64
oracle, and a training step on the fused forward's saved h1 against the
oracle's backward."""
import numpy as np
import pytest
import torch

from mixture_experts_routed_03_amd import workloads as wl
from oracle import moe as om
from tests._harness import (TOL, banner, full_size_tokens, make_inputs, oracle_forward, report,
                            run_forward, sampled_forward_ref)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mixture_experts_routed_03_amd import binding
    binding.lib()
    assert torch.cuda.is_available()
    return binding


def _mega_y(layer, lay, y_addend=None):
    T = lay["x"].shape[0]
    y = torch.empty((T, layer.D), dtype=layer.act_dtype, device=layer.device)
    layer.route(lay["ids"])
    layer.forward_mega(lay["x"], lay["w13"], lay["w2"])
    layer.combine(lay["scores"], y, y_addend=y_addend)
    return y


@pytest.mark.parametrize("T,D,F,E,K,prec,zipf,n_pad", [
    (300, 256, 256, 8, 2, "bf16", None, 7),       # 8 experts over 8 XCDs: one each
    (512, 384, 128, 16, 4, "bf16", 1.3, 0),       # skew: experts of several m-tiles, empty experts
    (33, 512, 384, 40, 3, "bf16", 0.5, 5),        # more experts than rows; staged W13 splits
    (700, 128, 128, 2048, 4, "bf16", None, 0),    # E > 1024, most experts with 0-3 rows
    (200, 256, 256, 12, 3, "f32", None, 0),       # staged W13 splits
    (5, 256, 128, 3, 2, "bf16", None, 0),         # fewer experts than XCDs
])
def test_mega_forward_equals_staged_and_oracle(B, T, D, F, E, K, prec, zipf, n_pad):
    banner(f"mega forward T={T} D={D} F={F} E={E} K={K} {prec} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, prec, zipf=zipf, n_pad=n_pad, seed=T + E)
    layer = B.MoeLayer(T, D, F, E, K, prec, hot_tiles="never")
    ys = run_forward(layer, lay).clone()
    h3s = layer.h3.clone()
    ym = _mega_y(layer, lay)
    torch.cuda.synchronize()
    assert layer.status()[0] == 0
    if "split-K" not in layer.explain():
        # same tiles, same contraction order: bit-identical (a plan that
        # splits adds fp32 parts in another order in its staged forward)
        rt = om.route(lay["ids"].cpu().numpy(), E)
        valid = torch.from_numpy(rt["route_to_row"] >= 0).to(layer.device)
        assert torch.equal(layer.h3.view(T * K, D)[valid], h3s.view(T * K, D)[valid])
        assert torch.equal(ym, ys)
    else:
        assert om.max_abs_rel(ys, oracle_forward(lay)) < TOL[prec]
    ref = oracle_forward(lay)
    err = om.max_abs_rel(ym, ref)
    report(f"mega forward (bound {TOL[prec]:g})", y=err)
    assert err < TOL[prec]


def test_mega_repeated_calls_and_token_permutation(B):
    """Counters and tickets are cleared by each call's planner launch: a
    second fused call on the same routing gives the same output, and a
    permutation of the tokens permutes it."""
    banner("mega repeated / permuted")
    T, D, F, E, K = 256, 256, 256, 10, 3
    lay = make_inputs(T, D, F, E, K, "bf16", seed=12)
    layer = B.MoeLayer(T, D, F, E, K, "bf16")
    y1 = _mega_y(layer, lay).clone()
    layer.forward_mega(lay["x"], lay["w13"], lay["w2"])
    y2 = torch.empty_like(y1)
    layer.combine(lay["scores"], y2)
    p = torch.randperm(T, generator=torch.Generator().manual_seed(1)).cuda()
    lay_p = dict(lay, x=lay["x"][p].contiguous(), ids=lay["ids"][p].contiguous(),
                 scores=lay["scores"][p].contiguous())
    y3 = _mega_y(layer, lay_p)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(y3, y1[p])
    assert layer.status()[0] == 0


@pytest.mark.parametrize("arena_budget", [0, 128])
def test_mega_training_step_matches_oracle(B, arena_budget):
    """Backward after the fused forward: with the state saved it reads the
    h1 the fused launch stored; with replay it rebuilds h1 with the staged
    W13 kernel.  Both match the oracle, and equal the staged forward's
    training step bit for bit."""
    T, D, F, E, K = 200, 256, 256, 6, 2
    banner(f"mega training arena_budget={arena_budget}")
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=1.1, seed=44, training=True)
    outs = {}
    for mode in ("staged", "mega"):
        layer = B.MoeLayer(T, D, F, E, K, "bf16", training=True, arena_budget=arena_budget,
                           hot_tiles="never")
        y = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
        layer.route(lay["ids"])
        (layer.forward_mega if mode == "mega" else layer.forward)(lay["x"], lay["w13"], lay["w2"])
        layer.combine(lay["scores"], y)
        dx = torch.empty_like(y)
        dw13 = torch.empty((E, 2 * F, D), dtype=torch.bfloat16, device="cuda")
        dw2 = torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")
        ds = torch.empty((T, K), dtype=torch.float32, device="cuda")
        layer.backward(lay["x"], lay["scores"], lay["dy"], lay["w13"], lay["w2"], dx, dw13, dw2, ds)
        torch.cuda.synchronize()
        assert layer.status()[1] == (1 if arena_budget else 0)
        outs[mode] = (y, dx, dw13, dw2, ds)
    for u, v in zip(outs["staged"], outs["mega"]):
        assert torch.equal(u, v)
    ry, cache = oracle_forward(lay, keep=True)
    rdx, rdw13, rdw2, rds = om.backward(lay["dy"], lay["x"], lay["ids"], lay["scores"],
                                        lay["w13"].cpu(), lay["w2"].cpu(), cache)
    y, dx, dw13, dw2, ds = outs["mega"]
    errs = dict(y=om.max_abs_rel(y, ry), dx=om.max_abs_rel(dx, rdx), ds=om.max_abs_rel(ds, rds),
                dw13=om.max_abs_rel(dw13, rdw13), dw2=om.max_abs_rel(dw2, rdw2))
    report("mega training (bound 2e-2)", **errs)
    for k, v in errs.items():
        assert v < TOL["bf16"], k


@pytest.mark.parametrize("T,D,F,E,K,prec,w1,zipf", [
    (300, 512, 256, 8, 2, "mxfp8", False, None),
    (200, 384, 384, 5, 3, "mxfp8", False, 1.2),    # N an odd multiple of 128, skew
    (300, 512, 256, 8, 2, "mxfp8", True, None),    # 1x32 weights
    (128, 512, 512, 4, 2, "mxfp4", False, None),
    (40, 256, 256, 12, 3, "mxfp8", False, 0.8),     # more XCDs than busy experts
])
def test_mega_block_scaled_forward_equals_staged(B, T, D, F, E, K, prec, w1, zipf):
    """Block-scaled fused forward: the W13 records quantize h2 rows in their
    epilogue and the W2 records read them, as in the staged pair, so the
    route slots are bit-identical; against the quantization-faithful oracle
    within the MX bound."""
    from oracle import mx as omx
    from oracle import mxfp4 as o4
    banner(f"mega {prec} T={T} D={D} F={F} E={E} K={K} w1x32={w1} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, prec, zipf=zipf, seed=T + 3 * E)
    layer = B.MoeLayer(T, D, F, E, K, prec, mx_w1x32=w1)
    layer.prepare(lay["w13"], lay["w2"])
    ys = run_forward(layer, lay).clone()
    h3s = layer.h3.clone()
    ym = _mega_y(layer, lay)
    torch.cuda.synchronize()
    assert layer.status()[0] == 0
    rt = om.route(lay["ids"].cpu().numpy(), E)
    valid = torch.from_numpy(rt["route_to_row"] >= 0).to(layer.device)
    assert torch.equal(layer.h3.view(T * K, D)[valid], h3s.view(T * K, D)[valid])
    assert torch.equal(ym, ys)
    args = (lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu())
    ref = o4.forward(*args) if prec == "mxfp4" else omx.forward(*args, w1x32=w1)
    err = om.max_abs_rel(ym, ref)
    report(f"mega {prec} forward (bound 6e-2)", y=err)
    assert err < TOL["mxfp8"]


def test_mega_mxfp8_training_step_equals_staged(B):
    """MXFP8 training on the fused forward (its x and h2 column bundles and
    saved state as in the staged forward): forward and backward outputs equal
    the staged ones bit for bit and match the oracle."""
    from oracle import mx as omx
    T, D, F, E, K = 256, 512, 256, 6, 2
    banner("mega mxfp8 training")
    lay = make_inputs(T, D, F, E, K, "mxfp8", zipf=1.1, seed=61, training=True)
    outs = {}
    for mode in ("staged", "mega"):
        layer = B.MoeLayer(T, D, F, E, K, "mxfp8", training=True)
        layer.prepare(lay["w13"], lay["w2"])
        y = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
        layer.route(lay["ids"])
        (layer.forward_mega if mode == "mega" else layer.forward)(lay["x"], lay["w13"], lay["w2"])
        layer.combine(lay["scores"], y)
        dx = torch.empty_like(y)
        dw13 = torch.empty((E, 2 * F, D), dtype=torch.bfloat16, device="cuda")
        dw2 = torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")
        ds = torch.empty((T, K), dtype=torch.float32, device="cuda")
        layer.backward(lay["x"], lay["scores"], lay["dy"], lay["w13"], lay["w2"], dx, dw13, dw2, ds)
        torch.cuda.synchronize()
        assert layer.status()[0] == 0
        outs[mode] = (y, dx, dw13, dw2, ds)
    for u, v in zip(outs["staged"], outs["mega"]):
        assert torch.equal(u, v)
    args = (lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu())
    ry, cache = omx.forward(*args, keep=True)
    rdx, rdw13, rdw2, rds = omx.backward(lay["dy"], *args[:3], lay["w13"].cpu(), lay["w2"].cpu(),
                                         cache)
    y, dx, dw13, dw2, ds = outs["mega"]
    counts = cache["route"]["counts"]
    errs = dict(y=om.max_abs_rel(y, ry), dx=om.max_abs_rel(dx, rdx), ds=om.max_abs_rel(ds, rds))
    errs["dw13"] = max(om.max_abs_rel(dw13[e], rdw13[e]) for e in range(E) if counts[e])
    errs["dw2"] = max(om.max_abs_rel(dw2[e], rdw2[e]) for e in range(E) if counts[e])
    report("mega mxfp8 training (bound 6e-2)", **errs)
    for k, v in errs.items():
        assert v < TOL["mxfp8"], k


@pytest.mark.parametrize("cfg_name", ["bf16_fwd_balanced", "bf16_train_zipf", "mxfp8_fwd_balanced"])
def test_full_size_mega_equals_staged(B, cfg_name):
    """T=2048, D=7168, F=2048, E=384, K=6 (BF16 balanced and Zipf(1.2)
    routing; MXFP8 balanced): the fused forward's y equals the staged
    forward's (BF16: streaming tiles for every expert) bit for bit, and 32
    sampled tokens match the oracle."""
    cfg = wl.CONFIGS[cfg_name]
    banner(f"full-size mega {cfg_name}")
    lay = wl.make_layer(cfg, 0, device="cuda")
    T, D, F, E, K = cfg.T, cfg.D, cfg.F, cfg.E, cfg.K
    mx = cfg.prec == "mxfp8"
    layer = B.MoeLayer(T, D, F, E, K, cfg.prec, hot_tiles="never" if not mx else "auto")
    if mx:
        layer.prepare(lay["w13"], lay["w2"])
    ys = run_forward(layer, lay).clone()
    ym = _mega_y(layer, lay)
    torch.cuda.synchronize()
    assert layer.status()[0] == 0
    assert torch.equal(ym, ys)
    tokens = full_size_tokens(T, seed=9)
    lay["_wcache"] = {}
    err = om.max_abs_rel(ym[tokens], sampled_forward_ref(lay, tokens, mx=mx))
    tol = TOL["mxfp8"] if mx else TOL["bf16"]
    report(f"full-size mega {cfg_name}, {len(tokens)} tokens (bound {tol:g})", y=err)
    assert err < tol
