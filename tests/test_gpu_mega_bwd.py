"""GPU parity of the fused (Mega) backward (Dist-MoE explainer, section 05,
Mega backward; section 0, the MXFP8 Mega path's two fused backward
operations): for each projection one persistent grid runs the DGRAD and
WGRAD work records, each expert's DGRAD range next to its WGRAD range.  In
BF16 the W2 launch's dW2 records wait on per-block counters for the h2
columns that its DGRAD records rebuild from h1; in MXFP8 no record waits.
Every record is one of the staged kernels' tiles with the same contraction
order, so each gradient must equal the staged backward's bit for bit (the
staged backward's 256 x 256 dW tiles of large experts agree bit for bit
with the streaming tiles too); the fused gradients are also checked against
the fp64 oracle (MXFP8: the quantization-faithful one)."""
import numpy as np
import pytest
import torch

from mixture_experts_routed_03_amd import workloads as wl
from oracle import moe as om
from oracle import mx as omx
from tests._harness import (TOL, banner, full_size_tokens, make_inputs, report, run_train,
                            sampled_backward_ref)

pytestmark = pytest.mark.gpu

NAMES = ("y", "dx", "dw13", "dw2", "ds")


@pytest.fixture(scope="module")
def B():
    from mixture_experts_routed_03_amd import binding
    binding.lib()
    assert torch.cuda.is_available()
    return binding


def _both(B, lay, T, D, F, E, K, flags=0, dw_init=None, **kw):
    """The training step with the staged and with the fused backward, each
    on a layer of its own; returns {mode: (y, dx, dw13, dw2, ds)}."""
    outs = {}
    for mode in ("staged", "mega"):
        layer = B.MoeLayer(T, D, F, E, K, "bf16", training=True, **kw)
        f = flags | (B.BWD_MEGA if mode == "mega" else 0)
        outs[mode] = [t.clone() for t in run_train(layer, lay, flags=f, dw_init=dw_init)]
        torch.cuda.synchronize()
        assert layer.status()[0] == 0, mode   # no status bit (SYNC_TIMEOUT among them)
    return outs


def _equal(outs):
    for name, u, v in zip(NAMES, outs["staged"], outs["mega"]):
        assert torch.equal(u, v), name


def _oracle(lay, got, tol):
    _, cache = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(),
                          lay["w2"].cpu(), keep=True)
    rdx, rdw13, rdw2, rds = om.backward(lay["dy"], lay["x"], lay["ids"], lay["scores"],
                                        lay["w13"].cpu(), lay["w2"].cpu(), cache)
    _, dx, dw13, dw2, ds = got
    errs = dict(dx=om.max_abs_rel(dx, rdx), ds=om.max_abs_rel(ds, rds),
                dw13=om.max_abs_rel(dw13, rdw13), dw2=om.max_abs_rel(dw2, rdw2))
    report(f"mega backward (bound {tol:g})", **errs)
    for k, v in errs.items():
        assert v < tol, k


@pytest.mark.parametrize("T,D,F,E,K,zipf,n_pad", [
    (300, 256, 256, 8, 2, None, 7),      # one expert per XCD, padded routes
    (1500, 256, 384, 6, 3, 1.2, 0),      # 351-1352 rows: 128-row DGRAD m-tiles, W2 waits on several
                                         # DGRAD records per expert; F = 3 x 128: half tiles
    (33, 512, 384, 40, 3, 0.5, 5),       # more experts than rows: empty experts store zero dW
    (700, 128, 128, 2048, 4, None, 0),   # E > 1024: most experts with 0-3 rows
    (5, 256, 128, 3, 2, None, 0),        # fewer experts than XCDs
])
def test_mega_backward_equals_staged_and_oracle(B, T, D, F, E, K, zipf, n_pad):
    banner(f"mega backward T={T} D={D} F={F} E={E} K={K} zipf={zipf} n_pad={n_pad}")
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=zipf, n_pad=n_pad, seed=T + E + 1,
                      training=True)
    outs = _both(B, lay, T, D, F, E, K)
    _equal(outs)
    if E <= 64:
        _oracle(lay, outs["mega"], TOL["bf16"])


def test_mega_backward_accumulate_fp32_dw_and_replay(B):
    """MOE_BWD_ACCUMULATE_DW into fp32 dW, on a layer that replays its
    forward (arena too small to save it), with clamped SwiGLU (the limit is
    the median |h1|, so about half of the gate and up values are clamped):
    the fused records add onto the caller's dW like the staged ones, and
    match the oracle (clamps decided on h1 as stored: bf16)."""
    T, D, F, E, K = 400, 384, 256, 9, 2
    banner("mega backward: accumulate, fp32 dW, replay, clamped SwiGLU")
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=1.3, seed=71, training=True)
    _, c0 = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu(),
                       keep=True)
    limit = float(np.median(np.abs(c0["H1"])))
    g = torch.Generator(device="cpu").manual_seed(5)
    start = (0.05 * torch.randn((E, 2 * F, D), generator=g)).float().cuda(), \
            (0.05 * torch.randn((E, D, F), generator=g)).float().cuda()
    outs = _both(B, lay, T, D, F, E, K, flags=B.BWD_ACCUMULATE_DW, dw_init=start,
                 dw_dtype="f32", arena_budget=128, swiglu_limit=limit)
    _equal(outs)
    _, cache = om.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu(),
                          keep=True, limit=limit, act=omx.bf16_round)
    _, rdw13, rdw2, _ = om.backward(lay["dy"], lay["x"], lay["ids"], lay["scores"],
                                    lay["w13"].cpu(), lay["w2"].cpu(), cache)
    _, _, dw13, dw2, _ = outs["mega"]
    errs = dict(dw13=om.max_abs_rel(dw13, om.as_f64(start[0]) + rdw13),
                dw2=om.max_abs_rel(dw2, om.as_f64(start[1]) + rdw2))
    report("mega backward accumulate (bound 2e-2)", **errs)
    for k, v in errs.items():
        assert v < TOL["bf16"], k


def test_mega_backward_repeated_calls(B):
    """Two fused backward steps in a row on one layer, the second with fewer
    tokens: the planner launch re-arms the tickets and counters each time."""
    T, D, F, E, K = 600, 256, 256, 12, 2
    banner("mega backward repeated calls")
    layer = B.MoeLayer(T, D, F, E, K, "bf16", training=True)
    ref = B.MoeLayer(T, D, F, E, K, "bf16", training=True)
    for n in (T, 257):
        lay = make_inputs(n, D, F, E, K, "bf16", zipf=0.8, seed=n, training=True)
        got = [t.clone() for t in run_train(layer, lay, flags=B.BWD_MEGA)]
        want = [t.clone() for t in run_train(ref, lay)]
        torch.cuda.synchronize()
        assert layer.status()[0] == 0
        for name, u, v in zip(NAMES, want, got):
            assert torch.equal(u, v), (n, name)


@pytest.mark.parametrize("T,D,F,E,K,zipf,n_pad,dw", [
    (300, 256, 256, 8, 2, None, 7, "bf16"),     # one expert per XCD, padded routes
    (1500, 256, 384, 6, 3, 1.2, 0, "bf16"),     # skew: many 64-row m-tiles; F = 3 x 128: half tiles
    (33, 512, 384, 40, 3, 0.5, 5, "f32"),       # more experts than rows; fp32 dW
    (700, 128, 128, 2048, 4, None, 0, "bf16"),  # E > 1024
])
def test_mega_backward_mxfp8_equals_staged(B, T, D, F, E, K, zipf, n_pad, dw):
    """MXFP8: the fused backward's records are the staged block-scaled
    kernels' tiles (no record waits: both of a projection's records read
    operands quantized before the launch), so every gradient equals the
    staged backward's bit for bit; against the quantization-faithful oracle
    as well (small E)."""
    banner(f"mega backward mxfp8 T={T} D={D} F={F} E={E} K={K} zipf={zipf} dW={dw}")
    lay = make_inputs(T, D, F, E, K, "mxfp8", zipf=zipf, n_pad=n_pad, seed=T + E + 7,
                      training=True)
    outs = {}
    for mode in ("staged", "mega"):
        layer = B.MoeLayer(T, D, F, E, K, "mxfp8", dw_dtype=dw, training=True)
        f = B.BWD_MEGA if mode == "mega" else 0
        outs[mode] = [t.clone() for t in run_train(layer, lay, flags=f)]
        torch.cuda.synchronize()
        assert layer.status()[0] == 0, mode
    _equal(outs)
    if E <= 64:
        ids = lay["ids"].cpu().numpy()
        _, cache = omx.forward(lay["x"], ids, lay["scores"], lay["w13"].cpu(), lay["w2"].cpu(),
                               keep=True)
        rdx, rdw13, rdw2, rds = omx.backward(lay["dy"], lay["x"], ids, lay["scores"],
                                             lay["w13"].cpu(), lay["w2"].cpu(), cache)
        _, dx, dw13, dw2, ds = outs["mega"]
        errs = dict(dx=om.max_abs_rel(dx, rdx), ds=om.max_abs_rel(ds, rds),
                    dw13=om.max_abs_rel(dw13, rdw13), dw2=om.max_abs_rel(dw2, rdw2))
        report(f"mega backward mxfp8 (bound {TOL['mxfp8']:g})", **errs)
        for k, v in errs.items():
            assert v < TOL["mxfp8"], k


def test_full_size_mega_backward_mxfp8_equals_staged(B):
    """T=2048, D=7168, F=2048, E=384, K=6, MXFP8 with Zipf(1.4) routing (the
    most skewed layer of the ten-layer stack): the fused backward equals the
    staged backward bit for bit; 32 sampled tokens' dX and dS and the
    hottest expert's dW match the quantization-faithful oracle."""
    cfg = wl.CONFIGS["mxfp8_ten_layer"]
    banner("full-size mega backward mxfp8 zipf 1.4")
    lay = wl.make_layer(cfg, 3, device="cuda")   # layer 3: Zipf(1.4)
    T, D, F, E, K = cfg.T, cfg.D, cfg.F, cfg.E, cfg.K
    outs = {}
    for mode in ("staged", "mega"):
        layer = B.MoeLayer(T, D, F, E, K, "mxfp8", training=True)
        f = B.BWD_MEGA if mode == "mega" else 0
        outs[mode] = [t.clone() for t in run_train(layer, lay, flags=f)]
        torch.cuda.synchronize()
        assert layer.status()[0] == 0, mode
        del layer
    _equal(outs)
    del outs["staged"]
    _, dx, dw13, dw2, ds = outs["mega"]
    tokens = full_size_tokens(T, seed=12)
    ids = lay["ids"].cpu().numpy()
    counts = torch.bincount(torch.from_numpy(ids[ids >= 0]).long(), minlength=E)
    experts = [int(torch.argmax(counts))]
    lay["_wcache"] = {}
    rdx, rds, rdw13, rdw2 = sampled_backward_ref(lay, tokens, experts, mx=True)
    errs = dict(dx=om.max_abs_rel(dx[tokens], rdx), ds=om.max_abs_rel(ds[tokens], rds),
                dw13=om.max_abs_rel(dw13[experts[0]], rdw13[0]),
                dw2=om.max_abs_rel(dw2[experts[0]], rdw2[0]))
    report(f"full-size mega backward mxfp8, hottest expert {experts[0]} ({int(counts[experts[0]])} "
           f"rows) (bound {TOL['mxfp8']:g})", **errs)
    for k, v in errs.items():
        assert v < TOL["mxfp8"], k


@pytest.mark.parametrize("cfg_name", ["bf16_train_zipf", "bf16_fwd_balanced"])
def test_full_size_mega_backward_equals_staged(B, cfg_name):
    """T=2048, D=7168, F=2048, E=384, K=6, Zipf(1.2) and balanced routing:
    the fused backward's dX, dW13, dW2 and dS equal the staged backward's
    bit for bit; 32 sampled tokens' dX and dS and the hottest and two other
    experts' dW match the oracle."""
    cfg = wl.CONFIGS[cfg_name]
    banner(f"full-size mega backward {cfg_name}")
    lay = wl.make_layer(cfg, 0, device="cuda", grads=True)
    T, D, F, E, K = cfg.T, cfg.D, cfg.F, cfg.E, cfg.K
    outs = _both(B, lay, T, D, F, E, K)
    _equal(outs)
    del outs["staged"]
    _, dx, dw13, dw2, ds = outs["mega"]
    tokens = full_size_tokens(T, seed=11)
    ids = lay["ids"].cpu().numpy()
    counts = torch.bincount(torch.from_numpy(ids[ids >= 0]).long(), minlength=E)
    hot = int(torch.argmax(counts))
    experts = sorted({hot, int(ids[tokens[0], 0]), int(ids[tokens[1], 1])} - {-1})
    lay["_wcache"] = {}
    rdx, rds, rdw13, rdw2 = sampled_backward_ref(lay, tokens, experts)
    errs = dict(dx=om.max_abs_rel(dx[tokens], rdx), ds=om.max_abs_rel(ds[tokens], rds),
                dw13=max(om.max_abs_rel(dw13[e], rdw13[i]) for i, e in enumerate(experts)),
                dw2=max(om.max_abs_rel(dw2[e], rdw2[i]) for i, e in enumerate(experts)))
    report(f"full-size mega backward {cfg_name} (bound {TOL['bf16']:g})", **errs)
    for k, v in errs.items():
        assert v < TOL["bf16"], k
