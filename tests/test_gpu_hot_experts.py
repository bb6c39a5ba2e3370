"""GPU parity of the BF16 forward when experts are hot (at least 256 rows):
those experts run on the 256 x 256 MFMA tiles, the others on the
weight-streaming tiles, through the C ABI against the fp64 oracle.  The
plans here ask for the large tiles always (hot_tiles="always"): in automatic
mode these small calls would keep every expert on the streaming tiles."""
import numpy as np
import pytest
import torch

from oracle import moe as om
from oracle import mx as omx
from tests._harness import (TOL, banner, check_route, make_inputs, oracle_forward, run_forward,
                            run_train)

pytestmark = pytest.mark.gpu

HOT = 256   # rows from which an expert takes the large tiles
HOT_WG = 256   # rows from which its BF16 weight gradients take them


@pytest.fixture(scope="module")
def B():
    from mixture_experts_routed_03_amd import binding
    binding.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return binding


def _counts(lay, E):
    ids = lay["ids"].cpu().numpy()
    return np.bincount(ids[ids >= 0].ravel(), minlength=E)


# (T, D, F, E, K, zipf, n_pad): every case has hot experts; the comments say
# which tile shapes they reach
CASES = [
    (1024, 512, 256, 4, 2, None, 0),     # all hot, ~512 rows: whole 256-row m-tiles, 2 n-tiles each
    (1500, 256, 384, 6, 3, 1.2, 9),      # uneven hot experts (368-1348 rows), F = 3 x 128, padded routes
    (600, 256, 256, 1, 1, None, 0),      # one expert, 600 rows: last m-tile 88 rows (waves with 2, 1, 0 live blocks)
    (900, 768, 128, 3, 1, 0.6, 0),       # a cold expert beside hot ones (256 and 436 rows), D = 3 x 256
    (5000, 256, 128, 1500, 4, 1.2, 0),   # E > 1024: the split prefixes carried across scan passes
    (400, 256, 128, 2, 2, None, 0),      # 800 routes: the one-launch routing path writes the split
]


@pytest.mark.parametrize("T,D,F,E,K,zipf,n_pad", CASES)
def test_hot_forward_matches_oracle(B, T, D, F, E, K, zipf, n_pad):
    banner(f"hot bf16 forward T={T} D={D} F={F} E={E} K={K} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=zipf, n_pad=n_pad, seed=T + 11)
    assert _counts(lay, E).max() >= HOT
    layer = B.MoeLayer(T, D, F, E, K, "bf16", hot_tiles="always")
    y = run_forward(layer, lay)
    torch.cuda.synchronize()
    check_route(layer.readback(T), lay["ids"].cpu().numpy(), E)
    ref, cache = oracle_forward(lay, keep=True)
    assert om.max_abs_rel(y, ref) < TOL["bf16"]
    assert torch.isfinite(y.float()).all()
    # h1 in packed row order, written by both tile kinds
    _, h1p = layer.saved_ptrs()
    R = cache["route"]["R"]
    h1 = layer.view(h1p, (R, 2 * F), torch.bfloat16)
    assert om.max_abs_rel(h1, cache["H1"]) < TOL["bf16"]
    assert layer.status()[0] == 0


def test_hot_forward_deterministic(B):
    banner("hot forward determinism")
    T, D, F, E, K = 800, 256, 256, 3, 2
    lay = make_inputs(T, D, F, E, K, "bf16", seed=5)
    layer = B.MoeLayer(T, D, F, E, K, "bf16", hot_tiles="always")
    y1 = run_forward(layer, lay).clone()
    y2 = run_forward(layer, lay).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_hot_fused_combine_matches_oracle(B):
    banner("hot fused combine")
    T, D, F, E, K = 1200, 512, 128, 5, 2
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=1.0, seed=21)
    assert _counts(lay, E).max() >= HOT
    layer = B.MoeLayer(T, D, F, E, K, "bf16", hot_tiles="always")
    y_slots = run_forward(layer, lay).clone()
    addend = torch.randn((T, D), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16).cuda()
    y = torch.empty_like(y_slots)
    layer.route(lay["ids"])
    layer.forward_fused(lay["x"], lay["w13"], lay["w2"], lay["scores"], y, y_addend=addend)
    torch.cuda.synchronize()
    ref = oracle_forward(lay)
    assert om.max_abs_rel(y.float() - addend.float(), ref) < TOL["bf16"]
    assert om.max_abs_rel(y.float() - addend.float(), y_slots) < 1e-2
    assert layer.status()[0] == 0


def test_hot_training_matches_oracle(B):
    """Forward h1 from the large tiles feeds the backward (dX, dW13, dW2, dS)."""
    banner("hot bf16 training")
    T, D, F, E, K = 700, 256, 256, 4, 2
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=0.8, seed=17, training=True)
    assert _counts(lay, E).max() >= HOT
    layer = B.MoeLayer(T, D, F, E, K, "bf16", training=True, hot_tiles="always")
    y, dx, dw13, dw2, ds = run_train(layer, lay)
    torch.cuda.synchronize()
    ref_y, cache = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(),
                              lay["w2"].cpu(), keep=True)
    rdx, rdw13, rdw2, rds = om.backward(lay["dy"], lay["x"], lay["ids"], lay["scores"],
                                        lay["w13"].cpu(), lay["w2"].cpu(), cache)
    tol = TOL["bf16"]
    assert om.max_abs_rel(y, ref_y) < tol
    assert om.max_abs_rel(dx, rdx) < tol
    assert om.max_abs_rel(ds, rds) < tol
    for e in range(E):
        assert om.max_abs_rel(dw13[e], rdw13[e]) < tol, e
        assert om.max_abs_rel(dw2[e], rdw2[e]) < tol, e
    assert layer.status() == (0, 0)


def test_hot_replay_and_clamp_match_saved_state(B):
    """A layer that replays its forward in backward rebuilds h1 with the same
    large tiles bit for bit; the clamped SwiGLU epilogue matches the oracle."""
    banner("hot replay + clamped SwiGLU")
    T, D, F, E, K = 640, 256, 256, 2, 1
    lay = make_inputs(T, D, F, E, K, "bf16", seed=8, training=True)
    assert _counts(lay, E).max() >= HOT
    _, c0 = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu(),
                       keep=True)
    L = float(np.median(np.abs(c0["H1"])))
    saved = B.MoeLayer(T, D, F, E, K, "bf16", training=True, swiglu_limit=L,
                       hot_tiles="always")
    a = [t.clone() for t in run_train(saved, lay)]
    replay = B.MoeLayer(T, D, F, E, K, "bf16", training=True, swiglu_limit=L, arena_budget=128,
                        hot_tiles="always")
    b = run_train(replay, lay)
    torch.cuda.synchronize()
    assert saved.status()[1] == 0 and replay.status()[1] == 1
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    ry, _ = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu(),
                       keep=True, limit=L, act=omx.bf16_round)
    assert om.max_abs_rel(a[0], ry) < TOL["bf16"]


def test_hot_sized_experts_on_streaming_tiles_bf16(B):
    """Experts of 256+ rows in a BF16 plan whose D is not a multiple of 256:
    every expert stays on the streaming tiles; forward and backward still
    match the oracle."""
    T, D, F, E, K = 800, 384, 128, 3, 2
    banner(f"hot-sized experts, streaming tiles bf16 T={T} D={D} F={F} E={E} K={K}")
    lay = make_inputs(T, D, F, E, K, "bf16", seed=T + 2, training=True)
    assert _counts(lay, E).min() >= HOT
    layer = B.MoeLayer(T, D, F, E, K, "bf16", training=True, hot_tiles="always")
    y, dx, dw13, dw2, ds = run_train(layer, lay)
    torch.cuda.synchronize()
    ref_y, cache = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(),
                              lay["w2"].cpu(), keep=True)
    rdx, rdw13, rdw2, rds = om.backward(lay["dy"], lay["x"], lay["ids"], lay["scores"],
                                        lay["w13"].cpu(), lay["w2"].cpu(), cache)
    tol = TOL["bf16"]
    assert om.max_abs_rel(y, ref_y) < tol
    assert om.max_abs_rel(dx, rdx) < tol
    assert om.max_abs_rel(ds, rds) < tol
    for e in range(E):
        assert om.max_abs_rel(dw13[e], rdw13[e]) < tol, e
        assert om.max_abs_rel(dw2[e], rdw2[e]) < tol, e


def test_hot_sized_experts_fp32_forward(B):
    """FP32 plans (forward only) never take the large BF16 tiles."""
    T, D, F, E, K = 600, 256, 128, 2, 1
    banner(f"hot-sized experts, fp32 forward T={T} D={D} F={F} E={E} K={K}")
    lay = make_inputs(T, D, F, E, K, "f32", seed=T + 2)
    assert _counts(lay, E).min() >= HOT
    layer = B.MoeLayer(T, D, F, E, K, "f32", hot_tiles="always")
    y = run_forward(layer, lay)
    torch.cuda.synchronize()
    assert om.max_abs_rel(y, oracle_forward(lay)) < TOL["f32"]


def test_tile_modes_agree(B):
    """The same skewed call under the three tile policies: "always" and
    "never" differ only in summation order; "auto" keeps this small call on
    the streaming tiles, so it equals "never" bit for bit."""
    banner("hot tile modes")
    T, D, F, E, K = 1500, 256, 384, 6, 3
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=1.2, seed=T + 11)
    ys = {}
    for mode in ("always", "never", "auto"):
        layer = B.MoeLayer(T, D, F, E, K, "bf16", hot_tiles=mode)
        ys[mode] = run_forward(layer, lay).clone()
    torch.cuda.synchronize()
    assert torch.equal(ys["auto"], ys["never"])
    assert om.max_abs_rel(ys["always"].float(), ys["never"].float()) < 1e-2


@pytest.mark.parametrize("T,D,F,E,K,zipf", [
    (1200, 512, 256, 5, 2, 1.0),    # 865, 574, 413, 301 rows on the 256 x 256 tiles; 247 streaming
    (1500, 256, 384, 6, 3, 1.2),    # dW13 of the experts of 256+ rows on them; dW2 (rows of F = 384 values) streaming
    (2000, 512, 256, 3, 1, None),   # every expert on them, ~670 rows (last stage partly past the end)
])
def test_hot_weight_gradient_tiles_equal_streaming(B, T, D, F, E, K, zipf):
    """BF16 weight gradients of experts with 256+ rows run on 256 x 256
    tiles (k_wgrad_hot) in automatic mode, those of smaller experts and the
    forward of these small calls on the streaming tiles; "never" keeps every
    weight gradient on the streaming tiles.  Both contract the same token
    rows in the same 16-row MFMA steps, so every gradient is bit-identical;
    against the oracle within the BF16 bound."""
    banner(f"hot weight-gradient tiles T={T} D={D} F={F} E={E} K={K} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=zipf, seed=T + 31, training=True)
    counts = _counts(lay, E)
    assert counts.max() >= HOT_WG
    outs = {}
    for mode in ("auto", "never"):
        layer = B.MoeLayer(T, D, F, E, K, "bf16", training=True, hot_tiles=mode)
        outs[mode] = [t.clone() for t in run_train(layer, lay)]
        torch.cuda.synchronize()
        assert layer.status() == (0, 0)
    for name, u, v in zip(("y", "dx", "dw13", "dw2", "ds"), outs["auto"], outs["never"]):
        assert torch.equal(u, v), name
    _, cache = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(),
                          lay["w2"].cpu(), keep=True)
    _, rdw13, rdw2, _ = om.backward(lay["dy"], lay["x"], lay["ids"], lay["scores"],
                                    lay["w13"].cpu(), lay["w2"].cpu(), cache)
    dw13, dw2 = outs["auto"][2], outs["auto"][3]
    for e in range(E):
        assert om.max_abs_rel(dw13[e], rdw13[e]) < TOL["bf16"], e
        assert om.max_abs_rel(dw2[e], rdw2[e]) < TOL["bf16"], e


@pytest.mark.parametrize("T,D,F,E,K,zipf", [
    (1200, 512, 256, 5, 2, 1.0),    # mixed: dW13 and dW2 of the 256+ row experts on the large tiles
    (1500, 256, 384, 6, 3, 1.2),    # dW13 on them; dW2 (rows of F = 384 values) streaming
    (2000, 512, 256, 3, 1, None),   # every expert on them; padded rows end half-way through a
                                    # 64-row stage; the last expert's exponent windows reach the
                                    # end of the bundles' exponent arrays
])
def test_mx_hot_weight_gradient_tiles_equal_streaming(B, T, D, F, E, K, zipf):
    """MXFP8 weight gradients of experts with 256+ rows run on 256 x 256
    tiles (k_mx_wgrad_hot) in automatic mode; "never" keeps them on the
    streaming tiles.  Both contract the same 64-token MFMA steps of the same
    column bundles with the same block scales (scale 2^0 and zero codes past
    an expert's padded rows), so every gradient is bit-identical; against
    the quantization-faithful oracle within the MXFP8 bound."""
    banner(f"mx hot weight-gradient tiles T={T} D={D} F={F} E={E} K={K} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, "mxfp8", zipf=zipf, seed=T + 37, training=True)
    counts = _counts(lay, E)
    assert counts.max() >= HOT_WG
    outs = {}
    for mode in ("auto", "never"):
        layer = B.MoeLayer(T, D, F, E, K, "mxfp8", training=True, hot_tiles=mode)
        outs[mode] = [t.clone() for t in run_train(layer, lay)]
        torch.cuda.synchronize()
        assert layer.status() == (0, 0)
    for name, u, v in zip(("y", "dx", "dw13", "dw2", "ds"), outs["auto"], outs["never"]):
        assert torch.equal(u, v), name
    ids = lay["ids"].cpu().numpy()
    _, cache = omx.forward(lay["x"], ids, lay["scores"], lay["w13"].cpu(), lay["w2"].cpu(),
                           keep=True)
    _, rdw13, rdw2, _ = omx.backward(lay["dy"], lay["x"], ids, lay["scores"],
                                     lay["w13"].cpu(), lay["w2"].cpu(), cache)
    dw13, dw2 = outs["auto"][2], outs["auto"][3]
    for e in range(E):
        assert om.max_abs_rel(dw13[e], rdw13[e]) < TOL["mxfp8"], e
        assert om.max_abs_rel(dw2[e], rdw2[e]) < TOL["mxfp8"], e
