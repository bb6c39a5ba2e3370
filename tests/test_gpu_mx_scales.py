"""Block-scaled layers whose E8M0 scales differ from block to block.

With Gaussian weights almost every 32x32 block gets the same exponent, so a
kernel that read the scale of the wrong block (or read the 32x32 scale in the
wrong orientation in DGRAD) would still match.  Here each weight block is
multiplied by 2^((3 bn + 5 bk + e) mod 7 - 3) (non-symmetric in the block
indices, shifted per expert) and x and dY are scaled per 32 columns and per
run of 48 tokens, so every FPROP, DGRAD and WGRAD scale read meets several
distinct exponents (Dist-MoE explainer, section 02: 32x32 weight blocks are
shared by FPROP and DGRAD with two scale orientations; activations carry
1x32 scales along the contraction; weight gradients read 32x1 column
bundles).

Errors are checked block by block (max|got - ref| / max|ref| inside each
32 x 32 block of the output, so one wrong block cannot hide behind the
tensor's largest values) against the quantization-faithful oracle, and the
achieved values are printed beside the 6e-2 MXFP8 bound.  The distance to the
oracle without BF16 rounding points (act=None) is printed too: the two
readings differ by up to ~5e-2 on their own, so only the faithful one is
asserted.

Weight gradients get the per-expert max-abs-rel bound of 6e-2 and a
blockwise bound of 0.15.  The scaled FP8 matrix-core instruction accumulates
with less than fp32 precision (measured: about 1 % of BF16 h1 values round
differently from the fp64 oracle's, against 0.007 % on the BF16 path), and
re-quantizing h2 and dH1 to E4M3 turns some of those one-ulp differences
into whole E4M3 steps, so single dW blocks reach a few 1e-2 even against a
faithful oracle.  A scale read from the wrong block is a factor of two or
more on that block's contribution, 0.3 or more blockwise, so the 0.15 bound
still catches it.
"""
DW_BLOCK_TOL = 0.15
import numpy as np
import pytest
import torch

from oracle import moe as om
from oracle import mx as omx
from oracle import mxfp4 as o4
from tests._harness import (TOL, apply_designed_scales, banner, blockwise_max_abs_rel,
                            distinct_block_exponents, make_inputs, report, run_forward,
                            run_train)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mixture_experts_routed_03_amd import binding
    binding.lib()
    assert torch.cuda.is_available()
    return binding


def _check_spread(lay):
    # the pattern must really produce several exponents per expert matrix
    for e in range(min(2, lay["w13"].shape[0])):
        assert len(distinct_block_exponents(lay["w13"][e])) >= 5
        assert len(distinct_block_exponents(lay["w2"][e])) >= 5


@pytest.mark.parametrize("T,D,F,E,K,zipf,dw", [
    (256, 512, 256, 6, 2, 1.1, "bf16"),
    (200, 384, 384, 5, 3, None, "f32"),   # N an odd multiple of 128: half tiles
])
def test_mxfp8_designed_scales_forward_backward(B, T, D, F, E, K, zipf, dw):
    banner(f"mxfp8 designed scales T={T} D={D} F={F} E={E} K={K} zipf={zipf} dW={dw}")
    lay = apply_designed_scales(make_inputs(T, D, F, E, K, "mxfp8", zipf=zipf, seed=T + 41,
                                            training=True))
    _check_spread(lay)
    layer = B.MoeLayer(T, D, F, E, K, "mxfp8", dw_dtype=dw, training=True)
    y, dx, dw13, dw2, ds = run_train(layer, lay)
    torch.cuda.synchronize()
    args = (lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu())
    ry, cache = omx.forward(*args, keep=True)
    rdx, rdw13, rdw2, rds = omx.backward(lay["dy"], *args[:3], lay["w13"].cpu(),
                                         lay["w2"].cpu(), cache)
    ny, ncache = omx.forward(*args, keep=True, act=None)
    ndx, ndw13, ndw2, _ = omx.backward(lay["dy"], *args[:3], lay["w13"].cpu(), lay["w2"].cpu(),
                                       ncache)
    counts = cache["route"]["counts"]
    live = [e for e in range(E) if counts[e]]
    errs = dict(
        y=blockwise_max_abs_rel(y, ry), dx=blockwise_max_abs_rel(dx, rdx),
        ds=om.max_abs_rel(ds, rds),
        dw13=max(om.max_abs_rel(dw13[e], rdw13[e]) for e in live),
        dw2=max(om.max_abs_rel(dw2[e], rdw2[e]) for e in live))
    dwb = dict(dw13=max(blockwise_max_abs_rel(dw13[e], rdw13[e]) for e in live),
               dw2=max(blockwise_max_abs_rel(dw2[e], rdw2[e]) for e in live))
    report("mxfp8 designed scales (y, dx blockwise; ds, dW per expert; faithful oracle; "
           "bound 6e-2)", **errs)
    report("mxfp8 designed scales (dW blockwise; bound 0.15)", **dwb)
    report("mxfp8 designed scales (tensor max-abs-rel, oracle without BF16 rounding points)",
           y=om.max_abs_rel(y, ny), dx=om.max_abs_rel(dx, ndx),
           dw13=max(om.max_abs_rel(dw13[e], ndw13[e]) for e in live),
           dw2=max(om.max_abs_rel(dw2[e], ndw2[e]) for e in live))
    for k, v in errs.items():
        assert v < TOL["mxfp8"], (k, v)
    for k, v in dwb.items():
        assert v < DW_BLOCK_TOL, (k, v)
    for e in range(E):
        if not counts[e]:
            assert torch.all(dw13[e] == 0) and torch.all(dw2[e] == 0)
    for t in (y, dx, dw13, dw2, ds):
        assert torch.isfinite(t.float()).all()


@pytest.mark.parametrize("T,D,F,E,K", [(300, 512, 256, 8, 2), (128, 384, 640, 4, 3)])
def test_mxfp8_1x32_designed_scales_forward(B, T, D, F, E, K):
    banner(f"mxfp8 1x32 designed scales T={T} D={D} F={F} E={E} K={K}")
    lay = apply_designed_scales(make_inputs(T, D, F, E, K, "mxfp8", seed=T + 43), row_jitter=True)
    _check_spread(lay)
    layer = B.MoeLayer(T, D, F, E, K, "mxfp8", mx_w1x32=True)
    y = run_forward(layer, lay)
    yf = torch.empty_like(y)
    layer.forward_fused(lay["x"], lay["w13"], lay["w2"], lay["scores"], yf)
    torch.cuda.synchronize()
    args = (lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu())
    ref = omx.forward(*args, w1x32=True)
    errs = dict(y=blockwise_max_abs_rel(y, ref), y_fused=blockwise_max_abs_rel(yf, ref))
    report("mxfp8 1x32 designed scales (blockwise, faithful oracle; bound 6e-2)", **errs)
    report("mxfp8 1x32 designed scales (oracle without BF16 rounding points)",
           y=om.max_abs_rel(y, omx.forward(*args, w1x32=True, act=None)))
    for k, v in errs.items():
        assert v < TOL["mxfp8"], (k, v)


@pytest.mark.parametrize("T,D,F,E,K", [(300, 512, 256, 8, 2), (96, 768, 512, 4, 3)])
def test_mxfp4_designed_scales_forward(B, T, D, F, E, K):
    banner(f"mxfp4 designed scales T={T} D={D} F={F} E={E} K={K}")
    lay = apply_designed_scales(make_inputs(T, D, F, E, K, "mxfp4", seed=T + 47), row_jitter=True)
    _check_spread(lay)
    layer = B.MoeLayer(T, D, F, E, K, "mxfp4")
    y = run_forward(layer, lay)
    yf = torch.empty_like(y)
    layer.forward_fused(lay["x"], lay["w13"], lay["w2"], lay["scores"], yf)
    torch.cuda.synchronize()
    args = (lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu())
    ref = o4.forward(*args)
    # E2M1 has one fraction bit, so a re-quantized h2 value that moves by one
    # BF16 ulp can move by a third of its size: blocks get the looser 0.15
    errs = dict(y=om.max_abs_rel(y, ref), y_fused=om.max_abs_rel(yf, ref))
    blk = dict(y=blockwise_max_abs_rel(y, ref), y_fused=blockwise_max_abs_rel(yf, ref))
    report("mxfp4 designed scales (tensor, faithful oracle; bound 6e-2)", **errs)
    report("mxfp4 designed scales (blockwise; bound 0.15)", **blk)
    report("mxfp4 designed scales (oracle without BF16 rounding points)",
           y=om.max_abs_rel(y, o4.forward(*args, act=None)))
    for k, v in errs.items():
        assert v < TOL["mxfp8"], (k, v)
    for k, v in blk.items():
        assert v < DW_BLOCK_TOL, (k, v)
