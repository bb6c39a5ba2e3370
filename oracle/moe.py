"""Routed-expert MoE layer, computed by definition in fp64 (test infrastructure).

Sources (titles of the pages; sections and equations as printed there):
  [DM]  "Dist-MoE - Speed-of-light distributed Mixture-of-Experts kernels",
        visual explainer: section 01 (caller inputs table: x [T,D], ids/scores
        [T,K], W13 [E,2,F,D] gate then up, W2 [E,D,F]; id -1 disables a route
        and an all-inactive row returns exact zero; the owner applies scores
        and sums the K routes in fp32), section 02 (h1 = W13 x = [g; u],
        h2 = SiLU(g) * u, h3 = W2 h2).
  [GG]  "Mixture of Experts: How Routing Becomes GPU Computation": section 1
        (SwiGLU FFN, SiLU(z) = z / (1 + e^-z), M_e = rows of expert e with
        sum_e M_e = T k), section 2 (packing by stable argsort, exclusive
        prefix offsets with the worked example [4,3,3,2] -> [0,4,7,10,12],
        the inverse permutation, grouped GEMM C_e = A_e B_e^T and its two
        gradients, the weighted combine and its gradients dH = p dY,
        dp = <H, dY>, silu'(z) = s (1 + z (1 - s)) with s = sigmoid(z)),
        section 5 (the source sums the returned input gradients).

Conventions: route r = t*K + k.  A route is valid iff 0 <= id < E; ids < -1 or
>= E are reported (``bad_id``) and then treated like padding.  Rows of an
expert are its valid routes in ascending r (the stable sort of [GG] s.2).
All inputs are decoded exactly to float64; no intermediate is rounded.
"""

from __future__ import annotations

import numpy as np


def as_f64(a) -> np.ndarray:
    """Exact float64 copy of a NumPy array or a torch tensor (any float dtype)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def as_i64(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.int64)


# --------------------------------------------------------------------------
# Routing metadata ([GG] section 2 "Packing"; [DM] section 01 padding rules)
# --------------------------------------------------------------------------

def route(ids, E: int, pad: int = 32) -> dict:
    """Group routes by expert.

    Returns counts [E], offsets [E+1] (exclusive prefix of counts),
    poffsets [E+1] (prefix of counts rounded up to ``pad``), sorted_route [R]
    (the route id r of each packed row, expert-major, ascending r inside an
    expert), route_to_row [T*K] (inverse permutation, -1 for padding) and
    bad_id (some id outside [-1, E)).
    """
    flat = as_i64(ids).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    bad_id = bool(np.any((flat < -1) | (flat >= E)))
    # Invalid routes get key E so they sort after every expert; the sort is
    # stable, so rows of one expert keep ascending route order.
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    R = int(valid.sum())
    sorted_route = order[:R].astype(np.int64)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    pcounts = -(-counts // pad) * pad
    poffsets = np.concatenate([[0], np.cumsum(pcounts)]).astype(np.int64)
    route_to_row = np.full(flat.shape[0], -1, dtype=np.int64)
    route_to_row[sorted_route] = np.arange(R, dtype=np.int64)
    return dict(counts=counts, offsets=offsets, poffsets=poffsets,
                sorted_route=sorted_route, route_to_row=route_to_row,
                bad_id=bad_id, R=R)


# --------------------------------------------------------------------------
# Expert FFN ([DM] section 02; [GG] section 1)
# --------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-z), evaluated without overflow for either sign of z."""
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z * sigmoid(z)


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d SiLU / dz = s (1 + z (1 - s)), s = sigmoid(z) ([GG] s.2 SwiGLU backward)."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


# Clamped SwiGLU.  The Supported modes section of the explainx.ai post "Meta
# Dist-MoE: Open-Source Fused MoE Kernels for Blackwell" names a clamped SwiGLU
# beside the plain one, without a formula; the reading taken here is the plainest
# one: before the activation the gate is clamped from above and the up
# projection to [-L, L], h2 = SiLU(min(g, L)) * clamp(u, -L, L), and a
# clamped value passes no gradient (dg = 0 where g > L, du = 0 where |u| > L).
# Each clamp is a decision at a threshold, so it is taken on the values the
# kernel decides on: ``decide`` = (g, u) as stored in the activation dtype
# (default: g, u themselves).  limit None or 0 is the plain SwiGLU.
#   (SiLU and its derivative from [GG] s.1, s.2.)

def _clamped(g, u, limit, decide):
    if not limit:
        return g, u, np.ones_like(g, dtype=bool), np.ones_like(u, dtype=bool)
    gd, ud = (g, u) if decide is None else decide
    g_in = ~(gd > limit)
    u_in = ~((ud > limit) | (ud < -limit))
    gc = np.where(g_in, g, limit)
    uc = np.where(u_in, u, np.where(ud > limit, limit, -limit))
    return gc, uc, g_in, u_in


def swiglu(g, u, limit=None, decide=None):
    """h2 = SiLU(g) * u ([DM] s.02), clamped as above when ``limit`` is set."""
    gc, uc, _, _ = _clamped(g, u, limit, decide)
    return silu(gc) * uc


def swiglu_backward(g, u, dh2, limit=None, decide=None):
    """(dg, du) of h2 = swiglu(g, u): dg = dh2 * u * silu'(g), du = dh2 * SiLU(g)
    ([GG] s.2 SwiGLU backward), on the clamped values, zero where clamped."""
    gc, uc, g_in, u_in = _clamped(g, u, limit, decide)
    dg = np.where(g_in, dh2 * uc * silu_grad(gc), 0.0)
    du = np.where(u_in, dh2 * silu(gc), 0.0)
    return dg, du


def expert_ffn(x_rows: np.ndarray, w13: np.ndarray, w2: np.ndarray, limit=None, act=None):
    """One expert on its rows: h1 = x W13^T = [g | u], h2 = SiLU(g) * u, h3 = h2 W2^T.

    x_rows [M, D], w13 [2F, D] (gate rows first), w2 [D, F]; all float64.
    ``limit``: clamped SwiGLU (see above), its clamp decisions taken on
    act(h1), the activation dtype's rounding (None: h1 itself).
    """
    F = w2.shape[1]
    h1 = x_rows @ w13.T
    g, u = h1[:, :F], h1[:, F:]
    dec = None if act is None else (act(g), act(u))
    h2 = swiglu(g, u, limit, dec)
    h3 = h2 @ w2.T
    return h1, h2, h3


def expert_ffn_backward(x_rows, w13, w2, h1, dh3, limit=None, act=None):
    """Gradients of one expert given dL/dh3 for its rows.

    dh2 = dh3 W2; dW2 = dh3^T h2; dg = dh2 * u * silu'(g); du = dh2 * SiLU(g);
    dh1 = [dg | du]; dx = dh1 W13; dW13 = dh1^T x  ([GG] s.2, grouped GEMM
    backward for C = A B^T: dA = dC B, dB = dC^T A).  ``limit``/``act`` as in
    expert_ffn.
    """
    F = w2.shape[1]
    g, u = h1[:, :F], h1[:, F:]
    dec = None if act is None else (act(g), act(u))
    h2 = swiglu(g, u, limit, dec)
    dh2 = dh3 @ w2
    dw2 = dh3.T @ h2
    dg, du = swiglu_backward(g, u, dh2, limit, dec)
    dh1 = np.concatenate([dg, du], axis=1)
    dx = dh1 @ w13
    dw13 = dh1.T @ x_rows
    return dx, dw13, dw2, dh1


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def forward(x, ids, scores, w13, w2, *, y_addend=None, keep=False, limit=None, act=None):
    """Y[t] = sum over valid k (ascending) of scores[t,k] * h3(t,k) (+ y_addend).

    Returns Y [T, D] float64 and, with ``keep``, a cache for ``backward``
    holding the routing metadata, per-row h1, h2 and the route outputs
    H3S [T*K, D] (zero rows for padding).  ``limit``/``act``: clamped SwiGLU
    (see expert_ffn).
    """
    X = as_f64(x)
    S = as_f64(scores)
    T, D = X.shape
    ids_a = as_i64(ids)
    K = ids_a.shape[1]
    E = w13.shape[0]
    F = w2.shape[2]
    rt = route(ids_a, E)
    R = rt["R"]
    H1 = np.zeros((R, 2 * F))
    H2 = np.zeros((R, F))
    H3S = np.zeros((T * K, D))
    for e in range(E):
        a, b = rt["offsets"][e], rt["offsets"][e + 1]
        if a == b:
            continue
        routes = rt["sorted_route"][a:b]
        xe = X[routes // K]
        h1, h2, h3 = expert_ffn(xe, as_f64(w13[e]), as_f64(w2[e]), limit, act)
        H1[a:b], H2[a:b], H3S[routes] = h1, h2, h3
    Y = combine(H3S, S, ids_a, E)
    if y_addend is not None:
        Y = Y + as_f64(y_addend)
    if keep:
        return Y, dict(route=rt, H1=H1, H2=H2, H3S=H3S, K=K, E=E, limit=limit, act=act)
    return Y


def combine(H3S, S, ids, E):
    """Token owner's weighted sum over the K route slots, k ascending."""
    T, K = ids.shape
    D = H3S.shape[1]
    Y = np.zeros((T, D))
    valid = (ids >= 0) & (ids < E)
    for k in range(K):
        w = np.where(valid[:, k], S[:, k], 0.0)
        Y += w[:, None] * H3S[k::K][:T]
    return Y


def backward(dy, x, ids, scores, w13, w2, cache):
    """dX [T,D], dW13 [E,2F,D], dW2 [E,D,F], dS [T,K] (all float64).

    Combine backward ([GG] s.2 / s.5): dH(t,k) = s[t,k] dY[t] and
    dS[t,k] = <H3(t,k), dY[t]>, zero for padding; each expert back-propagates
    its rows; dX[t] sums the valid route input gradients.  Experts with no
    rows get dW = 0.
    """
    dY = as_f64(dy)
    X = as_f64(x)
    S = as_f64(scores)
    ids_a = as_i64(ids)
    T, K = ids_a.shape
    rt = cache["route"]
    E = cache["E"]
    D = X.shape[1]
    F = w2.shape[2]
    valid = ((ids_a >= 0) & (ids_a < E)).reshape(-1)
    H3S = cache["H3S"]
    tok = np.arange(T * K) // K
    dS = np.where(valid, np.einsum("rd,rd->r", H3S, dY[tok]), 0.0).reshape(T, K)
    dH3S = np.where(valid[:, None], S.reshape(-1)[:, None] * dY[tok], 0.0)
    dX = np.zeros((T, D))
    dW13 = np.zeros((E, 2 * F, D))
    dW2 = np.zeros((E, D, F))
    dXr = np.zeros((T * K, D))
    for e in range(E):
        a, b = rt["offsets"][e], rt["offsets"][e + 1]
        if a == b:
            continue
        routes = rt["sorted_route"][a:b]
        xe = X[routes // K]
        dxe, dw13e, dw2e, _ = expert_ffn_backward(xe, as_f64(w13[e]), as_f64(w2[e]),
                                                  cache["H1"][a:b], dH3S[routes],
                                                  cache.get("limit"), cache.get("act"))
        dW13[e], dW2[e] = dw13e, dw2e
        dXr[routes] = dxe
    for k in range(K):
        dX += np.where(valid[k::K][:, None], dXr[k::K], 0.0)
    return dX, dW13, dW2, dS


# --------------------------------------------------------------------------
# Work accounting (Dist-MoE explainer, section 07 "Useful GEMM Work")
# --------------------------------------------------------------------------

def useful_flops(n_valid_routes: int, D: int, F: int, *, backward: bool = False) -> int:
    """Forward: gate/up/down GEMMs = 6 * routes * D * F (multiply-add = 2 FLOPs);
    backward (DGRAD + WGRAD) is twice forward."""
    fwd = 6 * int(n_valid_routes) * int(D) * int(F)
    return 2 * fwd if backward else fwd


def max_abs_rel(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 when both are all zero)."""
    g = as_f64(got)
    r = as_f64(ref)
    den = np.max(np.abs(r)) if r.size else 0.0
    num = np.max(np.abs(g - r)) if r.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
