"""MXFP8 codecs and the quantization-faithful MXFP8 expert path (test infrastructure).

Source: "Dist-MoE - Speed-of-light distributed Mixture-of-Experts kernels",
section 02 "Expert Computation and Tensor Precision".  What that section
fixes, restated:
  * the element format E4M3 (one sign bit, a 4-bit exponent and a 3-bit
    fraction) tops out at 448; the scale format E8M0 is a single byte that
    holds a power of two;
  * an MXFP8 tensor is E4M3 data plus one E8M0 scale for every 32
    consecutive logical values, and whoever produces the tensor chooses the
    scale, rounds the data with it and hands out both;
  * the scale axis follows the contraction: forward GEMMs sum over features,
    so activation rows are scaled in 1x32 runs along the features; weight
    gradients sum over token rows, so they read a column bundle quantized in
    32x1 runs down the rows; prepared weights use 32x32 tiles, whose data is
    shared by the forward and input-gradient GEMMs, each reading the scale
    in its own orientation;
  * in training the rows are quantized after the gather, from their BF16
    form.

Readings taken where the page is silent (each is a choice, listed in the
design notes):
  * E4M3 is the finite-only variant: exponent bias 7, subnormals down to
    2^-9, no infinities, S.1111.111 is NaN, so 448 = 1.75 * 2^8 is the top.
    Rounding is to nearest, ties to even; magnitudes above 448 saturate.
  * E8M0 scale of a block: the smallest integer e with amax <= 448 * 2^e,
    clamped to [-127, 127]; an all-zero block gets e = -127.  With this rule
    no scaled value exceeds 448 (parity unpinned: the rule itself is a choice).
  * Blocks start at index 0 of each axis of each expert's matrix; column
    bundles pad an expert's rows with zero rows up to a multiple of 32.
  * Every tensor that is quantized is first materialized in BF16, as the
    page describes for the gathered rows (BF16 rows are published and
    quantized afterwards): h1 is stored BF16 and h2 = SiLU(g) * u is formed
    from it and rounded to BF16; the route gradients s * dY and the h1
    gradient are rounded to BF16 before their row and column blocks are
    quantized.  The E4M3 codes are integer decisions, so they are taken on
    the same BF16 values the kernels quantize.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
BLOCK = 32


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits,
    exponent range of fp32, subnormals down to 2^-133), ties to even;
    magnitudes that round past the largest finite value become infinite."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, p = np.frexp(a)                          # a in [2^(p-1), 2^p)
    step = np.ldexp(1.0, np.maximum(p - 8, -133).astype(np.int64))
    q = np.rint(a / step) * step
    q = np.where(q > 3.3895313892515355e38, np.inf, q)
    return np.copysign(q, v)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(exp == 0, man / 8.0 * 2.0 ** -6,
                   (1.0 + man / 8.0) * np.ldexp(1.0, (exp - 7).astype(np.int64)))
    val = np.where((exp == 0xF) & (man == 0x7), np.nan, val)
    return sign * val


def e4m3_round(v) -> np.ndarray:
    """Round float64 values onto the E4M3 grid (nearest, ties to even; saturate at 448)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, p = np.frexp(a)                    # a = m * 2^p, m in [0.5, 1)
    # Normal binade [2^(p-1), 2^p) has 8 steps of 2^(p-4); below 2^-6 the
    # subnormal step is 2^-9.
    step = np.where(a >= E4M3_MIN_NORMAL, np.ldexp(1.0, (p - 4).astype(np.int64)),
                    E4M3_MIN_SUBNORMAL)
    q = np.rint(a / step) * step          # rint rounds half to even
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, v)


def e4m3_encode(v) -> np.ndarray:
    """E4M3 byte of each value after ``e4m3_round``."""
    q = e4m3_round(v)
    a = np.abs(q)
    sign = np.where(np.signbit(q), 0x80, 0)
    _, p = np.frexp(a)
    normal = a >= E4M3_MIN_NORMAL
    exp = np.where(normal, p - 1 + 7, 0)
    man = np.where(normal, np.rint((a / np.ldexp(1.0, (p - 1).astype(np.int64)) - 1.0) * 8.0),
                   np.rint(a / E4M3_MIN_SUBNORMAL))
    return (sign | (exp.astype(np.int64) << 3) | man.astype(np.int64)).astype(np.uint8)


def e8m0_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127] (-127 for 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, p = np.frexp(amax)                 # 448 = 0.875 * 2^9
    e = np.where(m <= 0.875, p - 9, p - 8)
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def _qdq_blocks(blocks: np.ndarray, axes) -> np.ndarray:
    amax = np.max(np.abs(blocks), axis=axes, keepdims=True)
    e = e8m0_exponent(amax)
    scale = np.ldexp(1.0, e)
    return e4m3_round(blocks / scale) * scale


def qdq_rows(v: np.ndarray) -> np.ndarray:
    """Quantize-dequantize with 1x32 blocks along the last axis (length % 32 == 0)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("row length must be a multiple of 32")
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    return _qdq_blocks(b, -1).reshape(v.shape)


def qdq_cols(v: np.ndarray) -> np.ndarray:
    """32x1 blocks down the rows of one expert's [M, N] matrix; rows are padded
    with zeros to a multiple of 32 for blocking and the pad is dropped again."""
    v = np.asarray(v, dtype=np.float64)
    M, N = v.shape
    Mp = -(-M // BLOCK) * BLOCK
    pad = np.zeros((Mp, N))
    pad[:M] = v
    b = pad.reshape(Mp // BLOCK, BLOCK, N)
    return _qdq_blocks(b, 1).reshape(Mp, N)[:M]


def qdq_32x32(w: np.ndarray) -> np.ndarray:
    """32x32 blocks over a weight matrix [N, K] (both multiples of 32)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if N % BLOCK or K % BLOCK:
        raise ValueError("weight dims must be multiples of 32")
    b = w.reshape(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    return _qdq_blocks(b, (1, 3)).reshape(N, K)


# --------------------------------------------------------------------------
# Quantization-faithful expert FFN: quantize -> dequantize at every operand
# the MXFP8 path feeds to a block-scaled GEMM, fp64 everywhere else.
# --------------------------------------------------------------------------

def _identity(v):
    return v


def expert_ffn_mx(x_rows, w13q, w2q, limit=None, act=bf16_round):
    """Forward.  x rows (BF16) quantized 1x32 along D after the gather; h1
    stored BF16; h2 = SiLU(g) * u from it (clamped SwiGLU with ``limit``, see
    oracle.moe.swiglu), rounded to BF16 and quantized 1x32 along F for the W2
    GEMM.  ``w13q``/``w2q`` are 32x32-block dequantized weights.  Returns h1
    (BF16 values), h2 (BF16 values) and h3.

    ``act`` is the rounding applied where an intermediate is materialized
    before it is quantized (h1, h2): BF16 by default (the reading above);
    ``act=None`` keeps them in fp64, the reading in which only the block
    quantizers round (used to show that the BF16 rounding points are not
    what makes a comparison pass)."""
    from .moe import swiglu
    act = act or _identity
    F = w2q.shape[1]
    h1 = act(qdq_rows(x_rows) @ w13q.T)
    g, u = h1[:, :F], h1[:, F:]
    h2 = act(swiglu(g, u, limit))
    h3 = qdq_rows(h2) @ w2q.T
    return h1, h2, h3


def expert_ffn_backward_mx(x_rows, w13q, w2q, h1, dh3, limit=None, act=bf16_round):
    """Backward.  ``h1`` is the stored BF16 h1, ``dh3`` the route gradient
    (rounded to BF16 here).  DGRAD operands are quantized along their
    contraction axis (dh3 1x32 along D, dh1 1x32 along 2F) and use the same
    32x32 weight values; WGRAD operands are column bundles (32x1 down the
    expert's rows) of dh3, h2, dh1 and x.  ``limit``: clamped SwiGLU.
    ``act``: rounding of the materialized intermediates (h2, dh3, dh1), as
    in ``expert_ffn_mx``."""
    from .moe import swiglu, swiglu_backward
    act = act or _identity
    F = w2q.shape[1]
    g, u = h1[:, :F], h1[:, F:]
    h2 = act(swiglu(g, u, limit))
    dh3 = act(dh3)
    dh2 = qdq_rows(dh3) @ w2q
    dw2 = qdq_cols(dh3).T @ qdq_cols(h2)
    dg, du = swiglu_backward(g, u, dh2, limit)
    dh1 = act(np.concatenate([dg, du], axis=1))
    dx = qdq_rows(dh1) @ w13q
    dw13 = qdq_cols(dh1).T @ qdq_cols(x_rows)
    return dx, dw13, dw2, dh1


# --------------------------------------------------------------------------
# Codes (what a producer publishes): E4M3 bytes and E8M0 exponents.
# --------------------------------------------------------------------------

def quantize_rows(v):
    """1x32 blocks along the last axis: (E4M3 bytes, E8M0 exponents e)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    e = e8m0_exponent(np.max(np.abs(b), axis=-1))
    q = e4m3_encode(b / np.ldexp(1.0, e)[..., None])
    return q.reshape(v.shape), e


def quantize_32x32(w):
    """32x32 blocks over [N, K]: (E4M3 bytes [N, K], exponents [N/32, K/32])."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    b = w.reshape(N // BLOCK, BLOCK, K // BLOCK, BLOCK)
    e = e8m0_exponent(np.max(np.abs(b), axis=(1, 3)))
    q = e4m3_encode(b / np.ldexp(1.0, e)[:, None, :, None])
    return q.reshape(N, K), e


def quantize_cols(v):
    """32x1 blocks down the rows of one expert's [M, N] matrix, rows padded
    with zeros to Mp = a multiple of 32.  Returns the column bundle as the
    transposed codes [N, Mp] and exponents [N, Mp/32]."""
    v = np.asarray(v, dtype=np.float64)
    M, N = v.shape
    Mp = -(-M // BLOCK) * BLOCK
    pad = np.zeros((Mp, N))
    pad[:M] = v
    b = pad.T.reshape(N, Mp // BLOCK, BLOCK)
    e = e8m0_exponent(np.max(np.abs(b), axis=-1))
    q = e4m3_encode(b / np.ldexp(1.0, e)[..., None])
    return q.reshape(N, Mp), e


# --------------------------------------------------------------------------
# Whole layer, quantization-faithful (same routing and combine as moe.py)
# --------------------------------------------------------------------------

def forward(x, ids, scores, w13, w2, *, y_addend=None, keep=False, limit=None, w1x32=False,
            act=bf16_round):
    """MXFP8 layer forward: weights in 32x32 blocks (``w1x32``: 1x32 blocks
    along each weight row, the inference preparation that the Supported modes
    section of the explainx.ai post on Dist-MoE names beside the training-compatible 32x32), activations per
    the expert functions above; combine in fp64.  ``limit``: clamped SwiGLU.
    ``act``: rounding of materialized intermediates (BF16; None = none)."""
    wq = qdq_rows if w1x32 else qdq_32x32
    from . import moe
    X = moe.as_f64(x)
    S = moe.as_f64(scores)
    T, D = X.shape
    ids_a = moe.as_i64(ids)
    K = ids_a.shape[1]
    E = w13.shape[0]
    F = w2.shape[2]
    rt = moe.route(ids_a, E)
    H1 = np.zeros((rt["R"], 2 * F))
    H3S = np.zeros((T * K, D))
    for e in range(E):
        a, b = rt["offsets"][e], rt["offsets"][e + 1]
        if a == b:
            continue
        routes = rt["sorted_route"][a:b]
        h1, _, h3 = expert_ffn_mx(X[routes // K], wq(moe.as_f64(w13[e])),
                                  wq(moe.as_f64(w2[e])), limit, act)
        H1[a:b], H3S[routes] = h1, h3
    Y = moe.combine(H3S, S, ids_a, E)
    if y_addend is not None:
        Y = Y + moe.as_f64(y_addend)
    if keep:
        return Y, dict(route=rt, H1=H1, H3S=H3S, K=K, E=E, limit=limit, act=act)
    return Y


def backward(dy, x, ids, scores, w13, w2, cache):
    """MXFP8 layer backward (dX, dW13, dW2, dS), quantization-faithful."""
    from . import moe
    dY = moe.as_f64(dy)
    X = moe.as_f64(x)
    S = moe.as_f64(scores)
    ids_a = moe.as_i64(ids)
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
        dxe, dw13e, dw2e, _ = expert_ffn_backward_mx(
            X[routes // K], qdq_32x32(moe.as_f64(w13[e])), qdq_32x32(moe.as_f64(w2[e])),
            cache["H1"][a:b], dH3S[routes], cache.get("limit"), cache.get("act", bf16_round))
        dW13[e], dW2[e] = dw13e, dw2e
        dXr[routes] = dxe
    for k in range(K):
        dX += np.where(valid[k::K][:, None], dXr[k::K], 0.0)
    return dX, dW13, dW2, dS
