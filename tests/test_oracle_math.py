"""Pins for the oracle's expert math, combine and backward (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import moe
from tests._golden import load


def _rand_layer(rng, T, D, F, E, K, pad=0):
    x = rng.standard_normal((T, D))
    w13 = rng.standard_normal((E, 2 * F, D)) / np.sqrt(D)
    w2 = rng.standard_normal((E, D, F)) / np.sqrt(F)
    ids = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)])
    s = rng.random((T, K))
    if pad:
        flat = rng.choice(T * K, size=pad, replace=False)
        ids.reshape(-1)[flat] = -1
        s.reshape(-1)[flat] = 0.0
    return x, ids, s, w13, w2


@pytest.mark.parametrize("T,D,F", [(1, 8, 4), (7, 32, 16), (33, 64, 96)])
def test_single_expert_is_dense_swiglu(T, D, F):
    """E = 1, K = 1, score 1: the routed layer is a dense SwiGLU FFN."""
    rng = np.random.default_rng(T)
    x = rng.standard_normal((T, D))
    w13 = rng.standard_normal((1, 2 * F, D))
    w2 = rng.standard_normal((1, D, F))
    y = moe.forward(x, np.zeros((T, 1), int), np.ones((T, 1)), w13, w2)
    xt = torch.from_numpy(x)
    wg = torch.from_numpy(w13[0, :F])
    wu = torch.from_numpy(w13[0, F:])
    wd = torch.from_numpy(w2[0])
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, wg)) * torch.nn.functional.linear(xt, wu), wd)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_silu_grad_matches_finite_difference():
    z = np.linspace(-30, 30, 2001)
    h = 1e-6
    fd = (moe.silu(z + h) - moe.silu(z - h)) / (2 * h)
    np.testing.assert_allclose(moe.silu_grad(z), fd, rtol=1e-6, atol=1e-8)
    # sigmoid does not overflow at the extremes
    assert np.all(np.isfinite(moe.sigmoid(np.array([-1e4, 1e4]))))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(seed)
    T, D, F, E, K = 4, 8, 4, 3, 2
    x, ids, s, w13, w2 = _rand_layer(rng, T, D, F, E, K, pad=1)
    dy = rng.standard_normal((T, D))

    def loss(x_, s_, w13_, w2_):
        return float(np.sum(moe.forward(x_, ids, s_, w13_, w2_) * dy))

    y, cache = moe.forward(x, ids, s, w13, w2, keep=True)
    dx, dw13, dw2, ds = moe.backward(dy, x, ids, s, w13, w2, cache)
    h = 1e-6
    for name, arr, grad in (("x", x, dx), ("w13", w13, dw13), ("w2", w2, dw2), ("s", s, ds)):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args = {"x": x, "s": s, "w13": w13, "w2": w2}
            p = arr.copy(); p[i] += h
            m = arr.copy(); m[i] -= h
            args_p = dict(args); args_p[name] = p
            args_m = dict(args); args_m[name] = m
            fd[i] = (loss(args_p["x"], args_p["s"], args_p["w13"], args_p["w2"])
                     - loss(args_m["x"], args_m["s"], args_m["w13"], args_m["w2"])) / (2 * h)
        if name == "s":  # padded routes have no gradient by contract
            fd = np.where(ids >= 0, fd, 0.0)
        err = np.max(np.abs(grad - fd)) / max(np.max(np.abs(fd)), 1e-300)
        assert err < 1e-6, (name, err)


def test_padded_route_equals_deleted_route():
    rng = np.random.default_rng(5)
    T, D, F, E, K = 6, 16, 8, 4, 3
    x, ids, s, w13, w2 = _rand_layer(rng, T, D, F, E, K)
    ids_p = ids.copy(); s_p = s.copy()
    ids_p[2, 1] = -1; s_p[2, 1] = 0.0
    y_p = moe.forward(x, ids_p, s_p, w13, w2)
    # Deleting the route: token 2 alone as a K = 2 problem with slots 0 and 2;
    # every other token is unchanged from the unpadded layer.
    y_alone = moe.forward(x[2:3], ids[2:3, [0, 2]], s[2:3, [0, 2]], w13, w2)
    np.testing.assert_allclose(y_p[2], y_alone[0], rtol=1e-13, atol=1e-14)
    y_full = moe.forward(x, ids, s, w13, w2)
    others = [t for t in range(T) if t != 2]
    np.testing.assert_array_equal(y_p[others], y_full[others])
    # A nonzero score on a -1 route is ignored.
    s_bad = s_p.copy(); s_bad[2, 1] = 123.0
    np.testing.assert_array_equal(moe.forward(x, ids_p, s_bad, w13, w2), y_p)


def test_all_padded_token_is_exact_zero_and_empty_expert_has_zero_dw():
    rng = np.random.default_rng(6)
    T, D, F, E, K = 5, 16, 8, 4, 2
    x, ids, s, w13, w2 = _rand_layer(rng, T, D, F, E, K)
    ids[3] = -1; s[3] = 0.0
    ids[ids == 2] = 1            # expert 2 gets no rows
    dy = rng.standard_normal((T, D))
    y, cache = moe.forward(x, ids, s, w13, w2, keep=True)
    assert np.all(y[3] == 0.0)
    dx, dw13, dw2, ds = moe.backward(dy, x, ids, s, w13, w2, cache)
    assert np.all(dx[3] == 0.0) and np.all(ds[3] == 0.0)
    assert np.all(dw13[2] == 0.0) and np.all(dw2[2] == 0.0)


def test_token_permutation_and_expert_relabeling():
    rng = np.random.default_rng(7)
    T, D, F, E, K = 9, 16, 8, 5, 2
    x, ids, s, w13, w2 = _rand_layer(rng, T, D, F, E, K, pad=2)
    dy = rng.standard_normal((T, D))
    y, c = moe.forward(x, ids, s, w13, w2, keep=True)
    dx, dw13, dw2, ds = moe.backward(dy, x, ids, s, w13, w2, c)
    p = rng.permutation(T)
    y2, c2 = moe.forward(x[p], ids[p], s[p], w13, w2, keep=True)
    dx2, dw13b, dw2b, ds2 = moe.backward(dy[p], x[p], ids[p], s[p], w13, w2, c2)
    np.testing.assert_allclose(y2, y[p], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx2, dx[p], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ds2, ds[p], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw13b, dw13, rtol=1e-10, atol=1e-12)
    # Relabel experts: expert e becomes q[e], its weights move with it.
    q = rng.permutation(E)
    ids_q = np.where(ids >= 0, q[np.maximum(ids, 0)], -1)
    w13_q = np.empty_like(w13); w13_q[q] = w13
    w2_q = np.empty_like(w2); w2_q[q] = w2
    np.testing.assert_allclose(moe.forward(x, ids_q, s, w13_q, w2_q), y, rtol=1e-12, atol=1e-12)


def test_output_is_linear_in_scores():
    rng = np.random.default_rng(8)
    T, D, F, E, K = 6, 16, 8, 4, 2
    x, ids, s, w13, w2 = _rand_layer(rng, T, D, F, E, K)
    s2 = rng.random((T, K))
    y = moe.forward(x, ids, 0.5 * s - 2.0 * s2, w13, w2)
    ref = 0.5 * moe.forward(x, ids, s, w13, w2) - 2.0 * moe.forward(x, ids, s2, w13, w2)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_useful_flops_and_scratch_worked_values():
    g = load("useful_work.txt")
    R = g["T"] * g["K"]
    assert moe.useful_flops(R, g["D"], g["F"]) == g["forward_flops"]
    assert moe.useful_flops(R, g["D"], g["F"], backward=True) == g["backward_flops"]
    from oracle import planner
    assert planner.bf16_forward_scratch_bytes(g["scratch_R"], g["D"], g["F"]) == g["scratch_bytes"]


def test_max_abs_rel_metric():
    assert moe.max_abs_rel(np.array([1.0, 2.0]), np.array([1.0, 2.0])) == 0.0
    assert moe.max_abs_rel(np.array([1.0, 2.5]), np.array([1.0, 2.0])) == 0.25
    assert moe.max_abs_rel(np.zeros(3), np.zeros(3)) == 0.0
    assert moe.max_abs_rel(np.ones(3), np.zeros(3)) == float("inf")


# ---------------------------------------------------------------- clamped SwiGLU
# (the reading of the clamped SwiGLU named under Supported modes in the explainx.ai post on Dist-MoE:
# h2 = SiLU(min(g, L)) * clamp(u, -L, L), no gradient through a clamped value)

def test_clamped_swiglu_worked_values():
    L = 1.0
    g = np.array([3.0, 0.5, -2.0, 3.0])
    u = np.array([-5.0, 0.25, 4.0, 0.5])
    s1 = 1.0 / (1.0 + np.exp(-1.0))                     # sigmoid(1)
    s05 = 1.0 / (1.0 + np.exp(-0.5))
    sm2 = 1.0 / (1.0 + np.exp(2.0))
    want = np.array([-1.0 * s1,                          # g -> 1, u -> -1
                     0.5 * s05 * 0.25,                   # inside: plain SwiGLU
                     -2.0 * sm2 * 1.0,                   # u -> +1 (g below the limit)
                     1.0 * s1 * 0.5])                    # g -> 1 only
    np.testing.assert_allclose(moe.swiglu(g, u, L), want, rtol=1e-15)
    dg, du = moe.swiglu_backward(g, u, np.ones(4), L)
    np.testing.assert_array_equal(dg[[0, 3]], 0.0)       # clamped gate: no gradient
    np.testing.assert_array_equal(du[[0, 2]], 0.0)       # clamped up: no gradient
    np.testing.assert_allclose(dg[1], 0.25 * moe.silu_grad(np.array([0.5]))[0], rtol=1e-15)
    np.testing.assert_allclose(du[1], 0.5 * s05, rtol=1e-15)
    np.testing.assert_allclose(du[3], s1, rtol=1e-15)    # d/du of SiLU(1) * u


def test_clamped_swiglu_limits_and_decisions():
    rng = np.random.default_rng(3)
    g, u = rng.standard_normal(1000) * 3, rng.standard_normal(1000) * 3
    np.testing.assert_array_equal(moe.swiglu(g, u, 1e30), moe.swiglu(g, u))
    np.testing.assert_array_equal(moe.swiglu(g, u, 0), moe.swiglu(g, u))   # 0 = plain
    # the clamp decisions follow ``decide`` (the stored activation), the
    # values the computation: just above the limit in fp64, at it when stored
    gg, uu = np.array([1.0 + 1e-9]), np.array([-(1.0 + 1e-9)])
    h = moe.swiglu(gg, uu, 1.0, decide=(np.array([1.0]), np.array([-1.0])))
    np.testing.assert_allclose(h, moe.silu(gg) * uu, rtol=1e-15)
    assert moe.swiglu(gg, uu, 1.0)[0] == moe.silu(np.array([1.0]))[0] * -1.0


@pytest.mark.parametrize("seed", [0, 1])
def test_clamped_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(10 + seed)
    T, D, F, E, K = 4, 8, 4, 3, 2
    x, ids, s, w13, w2 = _rand_layer(rng, T, D, F, E, K, pad=1)
    dy = rng.standard_normal((T, D))
    _, cache = moe.forward(x, ids, s, w13, w2, keep=True)
    L = float(np.median(np.abs(cache["H1"])))            # clamps about half the values
    g, u = cache["H1"][:, :F], cache["H1"][:, F:]
    assert 0.2 < np.mean((g > L) | (np.abs(u) > L)) < 0.95

    def loss(x_, s_, w13_, w2_):
        return float(np.sum(moe.forward(x_, ids, s_, w13_, w2_, limit=L) * dy))

    _, cache = moe.forward(x, ids, s, w13, w2, keep=True, limit=L)
    dx, dw13, dw2, ds = moe.backward(dy, x, ids, s, w13, w2, cache)
    h = 1e-7
    for name, arr, grad in (("x", x, dx), ("w13", w13, dw13), ("w2", w2, dw2), ("s", s, ds)):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args = {"x": x, "s": s, "w13": w13, "w2": w2}
            p = arr.copy(); p[i] += h
            m = arr.copy(); m[i] -= h
            args_p = dict(args); args_p[name] = p
            args_m = dict(args); args_m[name] = m
            fd[i] = (loss(args_p["x"], args_p["s"], args_p["w13"], args_p["w2"])
                     - loss(args_m["x"], args_m["s"], args_m["w13"], args_m["w2"])) / (2 * h)
        if name == "s":
            fd = np.where(ids >= 0, fd, 0.0)
        err = np.max(np.abs(grad - fd)) / max(np.max(np.abs(fd)), 1e-300)
        assert err < 1e-5, (name, err)
