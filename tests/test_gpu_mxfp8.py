"""GPU parity of the MXFP8 path (weight preparation, quantize-after-gather,
scaled-MFMA grouped GEMMs forward and backward), through the C ABI, against
the quantization-faithful fp64 oracle."""
import numpy as np
import pytest
import torch

from mixture_experts_routed_03_amd import workloads as wl
from oracle import moe as om
from oracle import mx as omx
from tests._harness import (TOL, banner, full_size_tokens, make_inputs, report, run_forward,
                            run_train, sampled_backward_ref, sampled_forward_ref)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mixture_experts_routed_03_amd import binding
    binding.lib()
    assert torch.cuda.is_available()
    return binding


def _wide(shape, seed):
    """bf16 values spanning many binades, with exact zeros and tiny values."""
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(shape, generator=g) * torch.exp(3 * torch.randn(shape, generator=g))
    v[..., 5] = 0.0
    v.view(-1)[::97] *= 1e-30
    return v.to(torch.bfloat16)


def test_prepare_weights_bit_exact(B):
    banner("mx weight prep")
    E, D, F = 3, 256, 128
    layer = B.MoeLayer(8, D, F, E, 2, "mxfp8")
    w13 = _wide((E, 2 * F, D), 1).cuda()
    w2 = _wide((E, D, F), 2).cuda()
    w13[1, :32, :32] = 0.0        # an all-zero block
    q13, s13, q2, s2 = layer.prepare(w13, w2)
    torch.cuda.synchronize()
    for e in range(E):
        for w, q, sc in ((w13, q13, s13), (w2, q2, s2)):
            rq, re = omx.quantize_32x32(om.as_f64(w[e]))
            np.testing.assert_array_equal(q[e].cpu().numpy(), rq)
            np.testing.assert_array_equal(sc[e].cpu().numpy().astype(np.int64), re + 127)


def test_row_and_column_quantizers_bit_exact(B):
    banner("mx row/column quantizers")
    T, E, K, n = 120, 6, 2, 256
    layer = B.MoeLayer(T, n, 128, E, K, "mxfp8")
    ids, _ = wl.make_routing(T, E, K, zipf_s=1.5, seed=4)
    ids[3, 1] = -1
    layer.route(torch.from_numpy(ids).cuda())
    rt = om.route(ids, E)
    src = _wide((rt["R"], n), 3).cuda()
    q, sc, rb = layer.quantize(src, 0)
    torch.cuda.synchronize()
    rq, re = omx.quantize_rows(om.as_f64(src))
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(sc.cpu().numpy().astype(np.int64), re + 127)
    q, sc, rb = layer.quantize(src, 1)
    torch.cuda.synchronize()
    q, sc = q.cpu().numpy(), sc.cpu().numpy().astype(np.int64)
    S = om.as_f64(src)
    for e in range(E):
        a, b = rt["offsets"][e], rt["offsets"][e + 1]
        pb, mp = rt["poffsets"][e], rt["poffsets"][e + 1] - rt["poffsets"][e]
        if mp == 0:
            continue
        cq, ce = omx.quantize_cols(S[a:b])
        np.testing.assert_array_equal(q[n * pb:n * (pb + mp)].reshape(n, mp), cq)
        np.testing.assert_array_equal(sc[n * pb // 32:n * (pb + mp) // 32].reshape(n, mp // 32), ce + 127)


@pytest.mark.parametrize("T,D,F,E,K,zipf,n_pad", [
    (300, 256, 256, 8, 2, None, 7),
    (200, 384, 128, 10, 3, 1.3, 0),
    (64, 128, 256, 3, 1, None, 0),
    (1024, 896, 640, 16, 4, 1.0, 11),   # several items per workgroup: prefetch across items (odd stage counts)
])
def test_mx_forward_matches_oracle(B, T, D, F, E, K, zipf, n_pad):
    banner(f"mx forward T={T} D={D} F={F} E={E} K={K} zipf={zipf}")
    lay = make_inputs(T, D, F, E, K, "mxfp8", zipf=zipf, n_pad=n_pad, seed=T + 7)
    layer = B.MoeLayer(T, D, F, E, K, "mxfp8")
    y = run_forward(layer, lay)
    torch.cuda.synchronize()
    ref = omx.forward(lay["x"], lay["ids"], lay["scores"], lay["w13"].cpu(), lay["w2"].cpu())
    assert om.max_abs_rel(y, ref) < TOL["mxfp8"]
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("T,D,F,E,K,zipf,dw", [
    (256, 256, 256, 6, 2, 1.2, "bf16"),
    (90, 128, 128, 4, 3, None, "f32"),
])
def test_mx_backward_matches_oracle(B, T, D, F, E, K, zipf, dw):
    banner(f"mx backward T={T} D={D} F={F} E={E} K={K} zipf={zipf} dW={dw}")
    lay = make_inputs(T, D, F, E, K, "mxfp8", zipf=zipf, seed=T + 9, training=True)
    ids = lay["ids"].clone(); sc = lay["scores"].clone()
    ids[7] = -1; sc[7] = 0.0
    ids[ids == E - 1] = 0                 # expert E-1 gets no rows
    lay["ids"], lay["scores"] = ids, sc
    layer = B.MoeLayer(T, D, F, E, K, "mxfp8", dw_dtype=dw, training=True)
    y, dx, dw13, dw2, ds = run_train(layer, lay)
    torch.cuda.synchronize()
    ry, cache = omx.forward(lay["x"], ids, sc, lay["w13"].cpu(), lay["w2"].cpu(), keep=True)
    rdx, rdw13, rdw2, rds = omx.backward(lay["dy"], lay["x"], ids, sc, lay["w13"].cpu(),
                                         lay["w2"].cpu(), cache)
    tol = TOL["mxfp8"]
    assert om.max_abs_rel(y, ry) < tol
    assert om.max_abs_rel(dx, rdx) < tol
    assert om.max_abs_rel(ds, rds) < tol
    assert torch.all(dx[7] == 0) and torch.all(ds[7] == 0)
    counts = cache["route"]["counts"]
    for e in range(E):
        if counts[e] == 0:
            assert torch.all(dw13[e] == 0) and torch.all(dw2[e] == 0)
        else:
            assert om.max_abs_rel(dw13[e], rdw13[e]) < tol, e
            assert om.max_abs_rel(dw2[e], rdw2[e]) < tol, e


def test_mx_replay_matches_saved_state(B):
    banner("mx replay vs save")
    T, D, F, E, K = 160, 256, 128, 5, 2
    lay = make_inputs(T, D, F, E, K, "mxfp8", seed=31, training=True)
    saved = B.MoeLayer(T, D, F, E, K, "mxfp8", training=True)
    a = [t.clone() for t in run_train(saved, lay)]
    assert saved.status()[1] == 0
    replay = B.MoeLayer(T, D, F, E, K, "mxfp8", training=True, arena_budget=128)
    b = run_train(replay, lay)
    torch.cuda.synchronize()
    assert replay.status()[1] == 1
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_full_size_mxfp8_train_with_shared_expert_sampled(B):
    """T=2048, D=7168, F=2048, E=384, K=6, balanced routing, MXFP8 forward +
    backward plus one shared BF16 SwiGLU expert applied to every token (a
    second plan with E=1, K=1, score 1); sampled tokens and experts vs the
    oracle (quantization-faithful routed part, fp64 dense shared part)."""
    cfg = wl.CONFIGS["mxfp8_train_shared"]
    banner("full-size mxfp8 + shared expert")
    lay = wl.make_layer(cfg, 0, device="cuda")
    T, D, F, E, K = cfg.T, cfg.D, cfg.F, cfg.E, cfg.K
    routed = B.MoeLayer(T, D, F, E, K, "mxfp8", training=True)
    shared = B.MoeLayer(T, D, F, 1, 1, "bf16", training=True)
    sh_ids = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    sh_sc = torch.ones((T, 1), dtype=torch.float32, device="cuda")
    ysh = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    shared.route(sh_ids)
    shared.forward(lay["x"], lay["w13_shared"], lay["w2_shared"])
    shared.combine(sh_sc, ysh)
    routed.prepare(lay["w13"], lay["w2"])
    y = run_forward(routed, lay, y_addend=ysh)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    dw13 = torch.empty((E, 2 * F, D), dtype=torch.bfloat16, device="cuda")
    dw2 = torch.empty((E, D, F), dtype=torch.bfloat16, device="cuda")
    ds = torch.empty((T, K), dtype=torch.float32, device="cuda")
    routed.backward(lay["x"], lay["scores"], lay["dy"], lay["w13"], lay["w2"], dx, dw13, dw2, ds)
    dws13 = torch.empty_like(lay["w13_shared"]); dws2 = torch.empty_like(lay["w2_shared"])
    shared.backward(lay["x"], sh_sc, lay["dy"], lay["w13_shared"], lay["w2_shared"], dx, dws13,
                    dws2, None, flags=B.BWD_ACCUMULATE_DX)
    torch.cuda.synchronize()
    tokens = full_size_tokens(T, seed=4)
    lay["_wcache"] = {}
    sh = om.as_f64(lay["w13_shared"][0]), om.as_f64(lay["w2_shared"][0])
    xs = om.as_f64(lay["x"][tokens])
    h1s, _, h3s = om.expert_ffn(xs, *sh)
    ref_y = sampled_forward_ref(lay, tokens, mx=True) + h3s
    counts = np.bincount(lay["ids"].cpu().numpy().reshape(-1), minlength=E)
    experts = [int(np.argmax(counts)), int(np.argmin(counts)), 17, 200]
    rdx, rds, rdw13, rdw2 = sampled_backward_ref(lay, tokens, experts, mx=True)
    dxs, _, _, _ = om.expert_ffn_backward(xs, *sh, h1s, om.as_f64(lay["dy"][tokens]))
    errs = dict(y=om.max_abs_rel(y[tokens], ref_y), dx=om.max_abs_rel(dx[tokens], rdx + dxs),
                ds=om.max_abs_rel(ds[tokens], rds))
    for i, e in enumerate(experts):
        errs[f"dw13[{e}]"] = om.max_abs_rel(dw13[e], rdw13[i])
        errs[f"dw2[{e}]"] = om.max_abs_rel(dw2[e], rdw2[i])
    report(f"full-size mxfp8 + shared, {len(tokens)} tokens (bound 6e-2)", **errs)
    for k, v in errs.items():
        assert v < TOL["mxfp8"], k
    for t in (y, dx, dw13, dw2, ds):
        assert torch.isfinite(t.float()).all()
