"""MXFP4 inference layer, quantization-faithful (test infrastructure: only the
tests, the smoke check and the bench's CPU baseline use it).

Source: "Dist-MoE - Speed-of-light distributed Mixture-of-Experts kernels",
section 02 "Expert Computation and Tensor Precision": E2M1 packs a sign, two
exponent bits and one fraction bit into four bits, two values per byte; the
4-bit inference mode quantizes the activations on the producing side and
multiplies them with expert weights prepared once (the support table of the
same page: the 4-bit format is inference-only, with prepared weights).  The
Supported modes section of the explainx.ai post "Meta Dist-MoE: Open-Source
Fused MoE Kernels for Blackwell (MXFP8, NVFP4)" names 1x32 blocks as the
inference weight preparation.

The pages' 4-bit mode is NVFP4 (E4M3 block scales plus a global scale).  This
module is its OCP-MX counterpart, the 4-bit block format that gfx950's scaled
matrix instructions take: E2M1 values with one E8M0 power-of-two scale per 32
values along the contraction axis, for activations and weights alike, and no
global scale (an E8M0 scale spans the whole fp32 exponent range).  Readings
where the pages are silent (each listed in the design notes):
  * E2M1: exponent bias 1, no infinities or NaN; exponent field 0 holds the
    subnormal 0.5 (and zero), so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4
    and 6.  Rounding is to nearest, ties to the even code (fraction bit 0);
    magnitudes above 6 saturate.
  * E8M0 scale of a block: the smallest integer e with amax <= 6 * 2^e,
    clamped to [-127, 127]; an all-zero block gets -127.  No scaled value
    exceeds 6 (parity unpinned as a rule: a choice, checked for its property).
  * Packing: value 2i of a row in the low nibble of byte i, value 2i + 1 in
    the high nibble.
  * Rounding points as in the MXFP8 forward: x rows (BF16) quantized 1x32
    along D after the gather; h1 stored BF16; h2 = SiLU(g) * u formed from it
    and rounded to BF16, then quantized 1x32 along F; h3 and the combine as
    in the BF16 layer.  The E2M1 codes are integer decisions, taken on the
    same BF16 values the kernels quantize.
"""

from __future__ import annotations

import numpy as np

from .mx import BLOCK, bf16_round

E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit E2M1 code (sign in bit 3, exponent in bits 2..1,
    fraction in bit 0, bias 1; exponent 0 is the subnormal range)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    exp = (c >> 1) & 0x3
    frac = c & 0x1
    val = np.where(exp == 0, 0.5 * frac,
                   (1.0 + 0.5 * frac) * np.ldexp(1.0, (exp - 1).astype(np.int64)))
    return sign * val


def e2m1_round(v) -> np.ndarray:
    """Round float64 values onto the E2M1 grid (nearest, ties to even; saturate at 6)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    # spacing of the grid: 0.5 below 2 (subnormal 0.5 and the binade [1, 2)),
    # 1 in [2, 4), 2 in [4, 6]; each binade edge is on the grid, so rounding
    # with the spacing of the binade a falls in is exact nearest rounding
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.rint(a / step) * step          # rint rounds half to even
    return np.copysign(np.minimum(q, E2M1_MAX), v)


def e2m1_encode(v) -> np.ndarray:
    """4-bit code of each value after ``e2m1_round`` (one code per uint8)."""
    q = e2m1_round(v)
    a = np.abs(q)
    sign = np.where(np.signbit(q), 0x8, 0)
    _, p = np.frexp(a)                    # a = m * 2^p, m in [0.5, 1)
    normal = a >= 1.0
    exp = np.where(normal, p, 0)          # a in [2^(p-1), 2^p): exponent field p
    frac = np.where(normal, np.rint((a / np.ldexp(1.0, np.maximum(p - 1, 0).astype(np.int64))
                                     - 1.0) * 2.0),
                    np.rint(a * 2.0))
    return (sign | (exp.astype(np.int64) << 1) | frac.astype(np.int64)).astype(np.uint8)


def e8m0_exponent_fp4(amax) -> np.ndarray:
    """Smallest integer e with amax <= 6 * 2^e, clamped to [-127, 127] (-127 for 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, p = np.frexp(amax)                 # 6 = 0.75 * 2^3
    e = np.where(m <= 0.75, p - 3, p - 2)
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def qdq_rows_fp4(v: np.ndarray) -> np.ndarray:
    """Quantize-dequantize with 1x32 E2M1 blocks along the last axis."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("row length must be a multiple of 32")
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    scale = np.ldexp(1.0, e8m0_exponent_fp4(np.max(np.abs(b), axis=-1, keepdims=True)))
    return (e2m1_round(b / scale) * scale).reshape(v.shape)


def quantize_rows_fp4(v):
    """1x32 blocks along the last axis: (packed E2M1 bytes [..., n/2], E8M0 exponents e)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    e = e8m0_exponent_fp4(np.max(np.abs(b), axis=-1))
    codes = e2m1_encode(b / np.ldexp(1.0, e)[..., None]).reshape(v.shape)
    return pack_e2m1(codes), e


def pack_e2m1(codes) -> np.ndarray:
    """Two codes per byte along the last axis: code 2i low nibble, 2i + 1 high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def expert_ffn_mxfp4(x_rows, w13q, w2q, limit=None, act=bf16_round):
    """One expert's forward with MXFP4 operands.  ``w13q``/``w2q`` are the
    dequantized 1x32-block E2M1 weights.  Returns h1, h2 (BF16 values) and h3.
    ``act``: rounding of the materialized h1 and h2 (BF16; None = none)."""
    from .moe import swiglu
    act = act or (lambda v: v)
    F = w2q.shape[1]
    h1 = act(qdq_rows_fp4(x_rows) @ w13q.T)
    h2 = act(swiglu(h1[:, :F], h1[:, F:], limit))
    h3 = qdq_rows_fp4(h2) @ w2q.T
    return h1, h2, h3


def forward(x, ids, scores, w13, w2, *, y_addend=None, limit=None, experts=None,
            act=bf16_round):
    """MXFP4 layer forward (inference): weights quantized 1x32 along their
    contraction axis, activations per ``expert_ffn_mxfp4``, routing and the
    fp64 combine of the BF16 layer.  ``experts``: optional subset of experts
    to evaluate (the routes of the others contribute nothing)."""
    from . import moe
    X = moe.as_f64(x)
    S = moe.as_f64(scores)
    ids_a = moe.as_i64(ids)
    T, K = ids_a.shape
    E = w13.shape[0]
    D = X.shape[1]
    rt = moe.route(ids_a, E)
    H3S = np.zeros((T * K, D))
    for e in (range(E) if experts is None else experts):
        a, b = rt["offsets"][e], rt["offsets"][e + 1]
        if a == b:
            continue
        routes = rt["sorted_route"][a:b]
        _, _, h3 = expert_ffn_mxfp4(X[routes // K], qdq_rows_fp4(moe.as_f64(w13[e])),
                                    qdq_rows_fp4(moe.as_f64(w2[e])), limit, act)
        H3S[routes] = h3
    Y = moe.combine(H3S, S, ids_a, E)
    if y_addend is not None:
        Y = Y + moe.as_f64(y_addend)
    return Y
