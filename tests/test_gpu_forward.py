"""GPU parity of routing, the expert forward and the combine, through the C ABI."""
import numpy as np
import pytest
import torch

from mixture_experts_routed_03_amd import workloads as wl
from oracle import moe as om
from tests._harness import (TOL, banner, check_route, full_size_tokens, make_inputs,
                            oracle_forward, report, run_forward, sampled_forward_ref)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mixture_experts_routed_03_amd import binding
    binding.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return binding


@pytest.mark.parametrize("T,E,K,zipf,n_pad", [
    (256, 8, 2, None, 26), (2048, 384, 6, None, 0), (2048, 384, 6, 1.2, 0), (1, 4, 2, None, 0),
    (0, 4, 2, None, 0), (777, 64, 8, 0.8, 300), (5, 3, 3, None, 15),
    (5000, 1500, 4, None, 0),             # E > 1024: the scan runs two passes over experts
    (3000, 4096, 8, 1.0, 100),            # E = 4096, the largest expert count
    (128, 2048, 8, None, 10),             # 1,024 routes: the one-launch path, two scan passes
    (205, 4096, 5, 1.0, 0),               # 1,025 routes: just past the one-launch path
    (64, 384, 6, None, 0), (170, 384, 6, 1.3, 9),   # decode-sized calls
])
def test_route_bit_exact(B, T, E, K, zipf, n_pad):
    banner(f"route T={T} E={E} K={K} zipf={zipf} pad={n_pad}")
    layer = B.MoeLayer(max(T, 1), 128, 128, E, K, "bf16")
    ids, _ = wl.make_routing(T, E, K, zipf_s=zipf, n_pad=n_pad, seed=3)
    layer.route(torch.from_numpy(ids).cuda())
    got = layer.readback(T)
    check_route(got, ids, E)
    st, _ = layer.status()
    assert st == 0


def test_route_maximum_route_count(B):
    """T*K = 2^24 routes (the plan's limit): 65,536 counting-sort chunks."""
    T, E, K = 1 << 21, 16, 8
    banner(f"route T={T} E={E} K={K} (2^24 routes)")
    layer = B.MoeLayer(T, 128, 128, E, K, "bf16")
    rng = np.random.default_rng(9)
    ids = np.argsort(rng.random((T, E), dtype=np.float32), axis=1)[:, :K].astype(np.int32)
    ids[rng.random((T, K)) < 0.01] = -1
    layer.route(torch.from_numpy(ids).cuda())
    check_route(layer.readback(T), ids, E)
    assert layer.status()[0] == 0


def test_route_unaligned_ids(B):
    """ids at an address that is 4-byte but not 16-byte aligned (a slice of a
    larger buffer): the same permutation as the oracle's."""
    T, E, K = 2048, 384, 6
    banner("route unaligned ids")
    layer = B.MoeLayer(T, 128, 128, E, K, "bf16")
    ids, _ = wl.make_routing(T, E, K, zipf_s=1.2, seed=5)
    buf = torch.full((T * K + 4,), -1, dtype=torch.int32, device="cuda")
    buf[1:1 + T * K] = torch.from_numpy(ids.ravel()).cuda()
    layer.route(buf[1:1 + T * K].view(T, K))
    check_route(layer.readback(T), ids, E)
    assert layer.status()[0] == 0


def test_route_bad_ids_flagged(B):
    banner("route bad ids")
    layer = B.MoeLayer(4, 128, 128, 4, 2, "bf16")
    ids = np.array([[0, 7], [-3, 1], [-1, 2], [3, 3]], dtype=np.int32)
    layer.route(torch.from_numpy(ids).cuda())
    got = layer.readback(4)
    ref = om.route(ids, 4)
    assert ref["bad_id"]
    np.testing.assert_array_equal(got["sorted_route"], ref["sorted_route"])
    np.testing.assert_array_equal(got["route_to_row"], ref["route_to_row"])
    st, _ = layer.status()
    assert st & B.STATUS_BAD_ID


def test_tiny_fp32_layer_matches_oracle(B):
    """T=256, D=256, F=128, E=8, K=2, fp32, 5% padded routes, forward."""
    cfg = wl.CONFIGS["tiny_f32"]
    banner("tiny fp32 forward")
    lay = wl.make_layer(cfg, 0, device="cuda")
    layer = B.MoeLayer(cfg.T, cfg.D, cfg.F, cfg.E, cfg.K, "f32")
    y = run_forward(layer, lay)
    torch.cuda.synchronize()
    ref, cache = oracle_forward(lay, keep=True)
    assert om.max_abs_rel(y, ref) < TOL["f32"]
    # intermediate h1 in packed row order
    _, h1p = layer.saved_ptrs()
    R = cache["route"]["R"]
    h1 = layer.view(h1p, (R, 2 * cfg.F), torch.float32)
    assert om.max_abs_rel(h1, cache["H1"]) < TOL["f32"]
    # padded tokens: none is all-padded here, but padded slots contribute nothing
    st, _ = layer.status()
    assert st == 0


@pytest.mark.parametrize("T,D,F,E,K,zipf,n_pad", [
    (300, 256, 256, 8, 2, None, 7),       # ragged m-tiles, several n-tiles
    (512, 384, 128, 16, 4, 1.3, 0),      # skew: hot experts span several m-tiles, empty experts
    (64, 128, 128, 4, 1, None, 0),
    (33, 512, 384, 40, 3, 0.5, 5),       # more experts than rows per expert
    (50, 256, 128, 24, 7, None, 11),      # K between the route-array bounds
    (40, 128, 128, 16, 16, 1.1, 0),       # K = 16 (the maximum)
    (700, 128, 128, 2048, 4, None, 0),    # E > 1024, most experts with 0-3 rows
])
def test_bf16_forward_matches_oracle(B, T, D, F, E, K, zipf, n_pad):
    banner(f"bf16 forward T={T} D={D} F={F} E={E} K={K} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, "bf16", zipf=zipf, n_pad=n_pad, seed=T)
    layer = B.MoeLayer(T, D, F, E, K, "bf16")
    y = run_forward(layer, lay)
    torch.cuda.synchronize()
    ref = oracle_forward(lay)
    check_route(layer.readback(T), lay["ids"].cpu().numpy(), E)
    assert om.max_abs_rel(y, ref) < TOL["bf16"]
    assert torch.isfinite(y.float()).all()


def test_all_padded_token_exact_zero_and_addend(B):
    banner("padding + addend")
    T, D, F, E, K = 40, 256, 128, 6, 2
    lay = make_inputs(T, D, F, E, K, "bf16", seed=9)
    ids = lay["ids"].clone(); sc = lay["scores"].clone()
    ids[3] = -1; sc[3] = 0.0
    ids[17] = -1; sc[17] = 0.0
    lay["ids"], lay["scores"] = ids, sc
    layer = B.MoeLayer(T, D, F, E, K, "bf16")
    y = run_forward(layer, lay)
    assert torch.all(y[3] == 0) and torch.all(y[17] == 0)
    add = torch.randn(T, D, device="cuda").to(torch.bfloat16)
    y2 = run_forward(layer, lay, y_addend=add)
    torch.cuda.synchronize()
    assert torch.equal(y2[3], add[3])
    ref = oracle_forward(lay) + om.as_f64(add)
    assert om.max_abs_rel(y2, ref) < TOL["bf16"]
    # a nonzero score on a -1 route is ignored and reported
    sc2 = sc.clone(); sc2[3, 0] = 5.0
    layer.combine(sc2, y2)
    assert torch.all(y2[3] == 0)
    st, _ = layer.status()
    assert st & B.STATUS_PAD_SCORE


def test_deterministic_and_token_permutation_invariant(B):
    banner("determinism / permutation")
    T, D, F, E, K = 200, 256, 256, 12, 3
    lay = make_inputs(T, D, F, E, K, "bf16", seed=4)
    layer = B.MoeLayer(T, D, F, E, K, "bf16")
    y1 = run_forward(layer, lay).clone()
    y2 = run_forward(layer, lay).clone()
    assert torch.equal(y1, y2)
    p = torch.randperm(T, generator=torch.Generator().manual_seed(0)).cuda()
    lay_p = dict(lay, x=lay["x"][p].contiguous(), ids=lay["ids"][p].contiguous(),
                 scores=lay["scores"][p].contiguous())
    y3 = run_forward(layer, lay_p)
    assert torch.equal(y3, y1[p])


def test_empty_call(B):
    banner("T=0")
    layer = B.MoeLayer(8, 128, 128, 4, 2, "bf16")
    lay = make_inputs(0, 128, 128, 4, 2, "bf16")
    y = run_forward(layer, lay)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


def test_full_size_bf16_forward_sampled(B):
    """T=2048, D=7168, F=2048, E=384, K=6 balanced (the benchmark's launch
    configuration): routing bit-exact, Y on sampled tokens vs the oracle."""
    cfg = wl.CONFIGS["bf16_fwd_balanced"]
    banner("full-size bf16 forward")
    lay = wl.make_layer(cfg, 0, device="cuda")
    layer = B.MoeLayer(cfg.T, cfg.D, cfg.F, cfg.E, cfg.K, "bf16")
    y = run_forward(layer, lay)
    torch.cuda.synchronize()
    check_route(layer.readback(cfg.T), lay["ids"].cpu().numpy(), cfg.E)
    tokens = full_size_tokens(cfg.T)
    lay["_wcache"] = {}
    ref = sampled_forward_ref(lay, tokens)
    err = om.max_abs_rel(y[tokens], ref)
    report(f"full-size bf16 forward, {len(tokens)} tokens (bound 2e-2)", y=err)
    assert err < TOL["bf16"]
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("T", [1, 8, 64])
def test_decode_shapes_forward(B, T):
    """Decode steps at the full layer shape (D=7168, F=2048, E=384, K=6, BF16):
    about one row per active expert.  Every token's Y (slot combine and FUSED
    combine) against the oracle, routing bit-exact."""
    cfg = wl.CONFIGS[f"bf16_decode_t{T}"]
    banner(f"decode forward T={T}")
    lay = wl.make_layer(cfg, 0, device="cuda")
    layer = B.MoeLayer(cfg.T, cfg.D, cfg.F, cfg.E, cfg.K, "bf16")
    y = run_forward(layer, lay)
    yf = torch.empty_like(y)
    layer.forward_fused(lay["x"], lay["w13"], lay["w2"], lay["scores"], yf)
    torch.cuda.synchronize()
    check_route(layer.readback(cfg.T), lay["ids"].cpu().numpy(), cfg.E)
    lay["_wcache"] = {}
    ref = sampled_forward_ref(lay, list(range(T)))
    errs = dict(y=om.max_abs_rel(y, ref), y_fused=om.max_abs_rel(yf, ref))
    report(f"decode T={T} (bound 2e-2)", **errs)
    for v in errs.values():
        assert v < TOL["bf16"]
    assert layer.status()[0] == 0


@pytest.mark.parametrize("prec,T,D,F,E,K,zipf,n_pad", [
    ("bf16", 300, 256, 256, 8, 2, None, 7),
    ("bf16", 200, 384, 128, 12, 6, 1.2, 0),
    ("f32", 256, 256, 128, 8, 2, None, 26),
    ("mxfp8", 160, 256, 128, 6, 3, None, 5),
])
def test_fused_combine_matches_oracle(B, prec, T, D, F, E, K, zipf, n_pad):
    """Combine fused into the W2 epilogue (fp32 atomics): same result as the
    slot combine up to the order of the K additions per token."""
    banner(f"fused combine {prec} T={T} D={D} F={F} E={E} K={K} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, prec, zipf=zipf, n_pad=n_pad, seed=T + 3)
    ids = lay["ids"].clone(); sc = lay["scores"].clone()
    ids[1] = -1; sc[1] = 0.0                      # an all-padded token
    lay["ids"], lay["scores"] = ids, sc
    layer = B.MoeLayer(T, D, F, E, K, prec)
    y_slots = run_forward(layer, lay)
    addend = torch.randn((T, D), generator=torch.Generator().manual_seed(5)).to(layer.act_dtype).cuda()
    y = torch.empty_like(y_slots)
    layer.route(lay["ids"])
    layer.forward_fused(lay["x"], lay["w13"], lay["w2"], lay["scores"], y, y_addend=addend)
    torch.cuda.synchronize()
    if prec == "mxfp8":
        from oracle import mx as omx
        ref = omx.forward(lay["x"], ids, sc, lay["w13"].cpu(), lay["w2"].cpu())
    else:
        ref = oracle_forward(lay)
    tol = TOL[prec]
    assert om.max_abs_rel(y.float() - addend.float(), ref) < tol
    assert torch.equal(y[1], addend[1])           # padding contributes exactly nothing
    # against the slot combine: only the summation order differs
    assert om.max_abs_rel(y.float() - addend.float(), y_slots) < (1e-5 if prec == "f32" else 1e-2)
    assert layer.status()[0] == 0


def test_fused_combine_needs_inference_plan(B):
    layer = B.MoeLayer(8, 128, 128, 4, 2, "bf16", training=True)
    x = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        layer.forward_fused(x, torch.zeros((4, 256, 128), dtype=torch.bfloat16, device="cuda"),
                            torch.zeros((4, 128, 128), dtype=torch.bfloat16, device="cuda"),
                            torch.zeros((8, 2), device="cuda"), torch.empty_like(x))
    assert ei.value.code == 3
