"""Pins for the oracle's MXFP8 codecs and quantization-faithful path (CPU only)."""
import numpy as np
import pytest

from oracle import moe, mx
from tests._golden import load


def _grid():
    vals = mx.e4m3_decode(np.arange(256))
    return vals


def test_e4m3_code_table_facts():
    g = load("formats.txt")
    vals = _grid()
    finite = vals[np.isfinite(vals)]
    assert np.nanmax(vals) == g["e4m3_max"] == 448.0
    # exactly two NaN codes (S.1111.111) and no infinities in the FN variant
    assert np.isnan(vals).sum() == 2 and np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert not np.any(np.isinf(vals))
    # 2^(exponent bits + fraction bits) - 1 non-NaN codes per sign
    assert len(finite) == 2 * (2 ** (g["e4m3_exponent_bits"] + g["e4m3_fraction_bits"]) - 1)
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)            # codes 0x00..0x7E increase
    assert pos[1] == 2.0 ** -9                 # smallest subnormal
    assert pos[8] == 2.0 ** -6                 # smallest normal
    assert vals[0x38] == 1.0                   # exponent field 7 = bias
    np.testing.assert_array_equal(vals[0x80:0xFF], -pos)
    # every normal binade holds 2^fraction_bits values
    for e in range(-6, 9):
        inb = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(inb) == 2 ** g["e4m3_fraction_bits"] or (e == 8 and len(inb) == 7)


def test_e4m3_round_is_nearest_ties_to_even():
    grid = np.unique(np.abs(_grid()[np.isfinite(_grid())]))
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.7, 20000),
        (grid[:-1] + grid[1:]) / 2.0,          # exact ties
        grid, -grid, [0.0, -0.0, 447.9, 448.0, 460.0, 1e6],
    ])
    q = mx.e4m3_round(v)
    a = np.minimum(np.abs(v), 448.0)
    idx = np.searchsorted(grid, a)
    lo = grid[np.clip(idx - 1, 0, len(grid) - 1)]
    hi = grid[np.clip(idx, 0, len(grid) - 1)]
    dlo, dhi = a - lo, hi - a
    even_hi = (np.searchsorted(grid, hi) % 2) == 0   # even mantissa = even code index
    pick_hi = (dhi < dlo) | ((dhi == dlo) & even_hi)
    exp = np.where(a == hi, hi, np.where(pick_hi, hi, lo))
    np.testing.assert_array_equal(np.abs(q), exp)
    assert np.all(np.signbit(q) == np.signbit(v))
    # encode/decode round trip
    np.testing.assert_array_equal(mx.e4m3_decode(mx.e4m3_encode(v)), q)


def test_e8m0_rule_is_smallest_fitting_power_of_two():
    rng = np.random.default_rng(1)
    amax = np.concatenate([10.0 ** rng.uniform(-30, 30, 50000),
                           448.0 * 2.0 ** np.arange(-20, 20),
                           np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), 0),
                           np.nextafter(448.0 * 2.0 ** np.arange(-20, 20), np.inf)])
    e = mx.e8m0_exponent(amax)
    assert np.all(amax <= 448.0 * np.ldexp(1.0, e))
    assert np.all(amax > 448.0 * np.ldexp(1.0, e - 1))
    assert mx.e8m0_exponent(0.0) == -127
    assert mx.e8m0_exponent(1e-300) == -127 and mx.e8m0_exponent(1e300) == 127


def test_block_quantization_properties():
    g = load("formats.txt")
    rng = np.random.default_rng(2)
    w = rng.standard_normal((64, 96)) * np.exp(rng.standard_normal((64, 96)))
    q = mx.qdq_32x32(w)
    np.testing.assert_array_equal(mx.qdq_32x32(w.T), q.T)     # shared by both orientations
    # rows: every 1x32 block; error <= half a step of the block's grid
    r = mx.qdq_rows(w[:, :g["mx_block"] * 3])
    for blk in range(3):
        v = w[:, 32 * blk:32 * blk + 32]
        e = mx.e8m0_exponent(np.abs(v).max(axis=1))
        s = np.ldexp(1.0, e)[:, None]
        assert np.all(np.abs(v / s) <= 448.0)
        assert np.all(np.abs(r[:, 32 * blk:32 * blk + 32] - v) <= s * np.maximum(np.abs(v / s) / 16.0, 2.0 ** -10) + 1e-300)
    # columns of a ragged expert: pad rows do not change the real rows' blocks
    c = mx.qdq_cols(w[:45])
    np.testing.assert_array_equal(c[:32], mx.qdq_cols(w[:32]))
    np.testing.assert_array_equal(c[32:45], mx.qdq_cols(w[32:45]))
    assert np.all(mx.qdq_rows(np.zeros((2, 32))) == 0.0)


def test_mx_path_reduces_to_exact_path_without_rounding(monkeypatch):
    """With every quantize-dequantize replaced by identity, the MXFP8 expert
    path must be the fp64 expert path: checks each operand feeds the right GEMM."""
    rng = np.random.default_rng(3)
    M, D, F = 7, 64, 32
    x = rng.standard_normal((M, D)); w13 = rng.standard_normal((2 * F, D)); w2 = rng.standard_normal((D, F))
    dh3 = rng.standard_normal((M, D))
    for name in ("qdq_rows", "qdq_cols"):
        monkeypatch.setattr(mx, name, lambda v: np.asarray(v, dtype=np.float64))
    # act=None: the switch that drops the BF16 rounding of materialized
    # intermediates; with the block quantizers off too, nothing rounds
    h1, h2, h3 = mx.expert_ffn_mx(x, w13, w2, act=None)
    r1, r2, r3 = moe.expert_ffn(x, w13, w2)
    np.testing.assert_allclose(h3, r3, rtol=1e-12, atol=1e-12)
    got = mx.expert_ffn_backward_mx(x, w13, w2, h1, dh3, act=None)
    ref = moe.expert_ffn_backward(x, w13, w2, r1, dh3)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


def test_mx_path_error_is_quantization_sized():
    rng = np.random.default_rng(4)
    M, D, F = 40, 256, 128
    x = rng.standard_normal((M, D))
    w13 = rng.standard_normal((2 * F, D)) / 16; w2 = rng.standard_normal((D, F)) / np.sqrt(F)
    h1, h2, h3 = mx.expert_ffn_mx(x, mx.qdq_32x32(w13), mx.qdq_32x32(w2))
    r3 = moe.expert_ffn(x, w13, w2)[2]
    err = moe.max_abs_rel(h3, r3)
    assert 1e-3 < err < 0.1


def test_codes_match_quantize_dequantize():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((5, 64)) * np.exp(2 * rng.standard_normal((5, 64)))
    q, e = mx.quantize_rows(v)
    np.testing.assert_array_equal(mx.e4m3_decode(q) * np.ldexp(1.0, np.repeat(e, 32, 1)),
                                  mx.qdq_rows(v))
    w = rng.standard_normal((64, 96))
    q, e = mx.quantize_32x32(w)
    np.testing.assert_array_equal(
        mx.e4m3_decode(q) * np.ldexp(1.0, np.repeat(np.repeat(e, 32, 0), 32, 1)), mx.qdq_32x32(w))
    m = rng.standard_normal((45, 64))
    q, e = mx.quantize_cols(m)
    assert q.shape == (64, 64) and e.shape == (64, 2)
    deq = mx.e4m3_decode(q) * np.ldexp(1.0, np.repeat(e, 32, 1))
    np.testing.assert_array_equal(deq.T[:45], mx.qdq_cols(m))
    assert np.all(q[:, 45:] == 0)          # pad rows quantize to +0


def test_mx_layer_reduces_to_fp64_layer_without_rounding(monkeypatch):
    from oracle import moe
    rng = np.random.default_rng(8)
    T, D, F, E, K = 6, 64, 32, 3, 2
    x = rng.standard_normal((T, D)); w13 = rng.standard_normal((E, 2 * F, D))
    w2 = rng.standard_normal((E, D, F)); ids = np.array([[0, 1], [1, 2], [2, -1], [0, 2], [1, 0], [-1, -1]])
    s = rng.random((T, K)); s[ids < 0] = 0; dy = rng.standard_normal((T, D))
    for name in ("qdq_rows", "qdq_cols", "qdq_32x32"):
        monkeypatch.setattr(mx, name, lambda v: np.asarray(v, dtype=np.float64))
    y, c = mx.forward(x, ids, s, w13, w2, keep=True, act=None)
    ry, rc = moe.forward(x, ids, s, w13, w2, keep=True)
    np.testing.assert_allclose(y, ry, rtol=1e-12, atol=1e-12)
    for a, b in zip(mx.backward(dy, x, ids, s, w13, w2, c), moe.backward(dy, x, ids, s, w13, w2, rc)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_bf16_round_matches_library_conversion():
    """RNE to bfloat16 from the definition equals torch's float32 -> bfloat16
    conversion (a library routine) on values across all binades, on exact
    ties and on the special cases."""
    import torch
    rng = np.random.default_rng(9)
    f32 = np.concatenate([
        (rng.standard_normal(200000) * np.exp(rng.uniform(-95, 88, 200000))),
        rng.standard_normal(20000) * 1e-40,                      # fp32 subnormals
        np.array([0.0, -0.0, 3.3895313e38, 3.4e38, -3.4e38, 1.0, 1.00390625, 1.01171875]),
    ]).astype(np.float32)
    # exact ties: bf16 values plus half an ulp
    base = torch.from_numpy(rng.standard_normal(20000).astype(np.float32)).to(torch.bfloat16)
    b32 = base.float().numpy()
    ulp = np.abs(b32) * 2.0 ** -7
    ties = (b32 + np.sign(b32) * ulp / 2).astype(np.float32)
    x = np.concatenate([f32, ties, b32])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = mx.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_mx_bf16_rounding_points_are_load_bearing():
    """The two readings of the rounding points (BF16 materialization before
    each quantizer, or none) are not interchangeable at the MXFP8 tolerance:
    moving h2 by one BF16 rounding pushes a few percent of its values across
    an E4M3 rounding boundary, and each such value then moves by a whole
    E4M3 step (6-12 %).  Over ten seeds the two readings' h3 differ by 2-5e-2
    max-abs-rel, most of the 6e-2 bound, while each stays within the bound of
    the unquantized-activation product.  So the oracle must quantize the same
    BF16 values the kernels store; the GPU tests report their distance to
    both readings."""
    errs, errq = [], []
    for seed in range(11, 21):
        rng = np.random.default_rng(seed)
        M, D, F = 48, 256, 128
        x = rng.standard_normal((M, D))
        w13 = mx.qdq_32x32(rng.standard_normal((2 * F, D)) / 16)
        w2 = mx.qdq_32x32(rng.standard_normal((D, F)) / np.sqrt(F))
        a = mx.expert_ffn_mx(x, w13, w2)[2]
        b = mx.expert_ffn_mx(x, w13, w2, act=None)[2]
        errs.append(moe.max_abs_rel(a, b))
        errq.append(moe.max_abs_rel(a, moe.expert_ffn(x, w13, w2)[2]))
    assert 1e-2 < min(errs) and max(errs) < 6e-2
    assert max(errq) < 6e-2
