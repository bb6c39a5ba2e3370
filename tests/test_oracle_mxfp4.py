"""Pins for the oracle's MXFP4 codecs and quantization-faithful inference
layer (CPU only)."""
import numpy as np

from oracle import moe, mxfp4
from tests._golden import load

# Magnitudes of the E2M1 element format as tabulated by the OCP Microscaling
# Formats (MX) v1.0 specification (bias 1, no infinities or NaN).
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_code_table():
    g = load("formats.txt")
    vals = mxfp4.e2m1_decode(np.arange(16))
    n_pos = 2 ** (g["e2m1_exponent_bits"] + g["e2m1_fraction_bits"])
    assert len(vals) == 2 * n_pos == 16 // (2 // g["e2m1_values_per_byte"])
    np.testing.assert_array_equal(vals[:8], OCP_E2M1)
    np.testing.assert_array_equal(vals[8:], -np.array(OCP_E2M1))
    assert np.signbit(vals[8]) and not np.signbit(vals[0])
    # every code survives encode(decode(c)), -0 included
    np.testing.assert_array_equal(mxfp4.e2m1_encode(vals), np.arange(16))


def test_e2m1_round_is_nearest_ties_to_even():
    grid = np.array(OCP_E2M1)
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-9.0, 9.0, 50000), (grid[:-1] + grid[1:]) / 2.0,
                        -(grid[:-1] + grid[1:]) / 2.0, grid, -grid,
                        [5.999, 6.0, 6.001, 7.0, 100.0, -1e9, 0.0, -0.0]])
    q = mxfp4.e2m1_round(v)
    a = np.minimum(np.abs(v), 6.0)
    d = np.abs(a[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # on a tie the even code (fraction bit 0: code index even) wins
    even = (np.arange(8) % 2) == 0
    pick = np.where(cand.sum(1) > 1, np.argmax(cand & even[None, :], axis=1), np.argmax(cand, axis=1))
    np.testing.assert_array_equal(np.abs(q), grid[pick])
    assert np.all(np.signbit(q) == np.signbit(v))
    np.testing.assert_array_equal(mxfp4.e2m1_decode(mxfp4.e2m1_encode(v)), q)


def test_e8m0_fp4_rule_is_smallest_fitting_power_of_two():
    rng = np.random.default_rng(1)
    amax = np.concatenate([10.0 ** rng.uniform(-30, 30, 50000), 6.0 * 2.0 ** np.arange(-20, 20),
                           np.nextafter(6.0 * 2.0 ** np.arange(-20, 20), 0),
                           np.nextafter(6.0 * 2.0 ** np.arange(-20, 20), np.inf)])
    e = mxfp4.e8m0_exponent_fp4(amax)
    assert np.all(amax <= 6.0 * np.ldexp(1.0, e))
    assert np.all(amax > 6.0 * np.ldexp(1.0, e - 1))
    assert mxfp4.e8m0_exponent_fp4(0.0) == -127
    assert mxfp4.e8m0_exponent_fp4(1e-300) == -127 and mxfp4.e8m0_exponent_fp4(1e300) == 127


def test_worked_block():
    """One 32-value block worked by hand: amax 12 -> e = 1 (6 * 2^0 < 12 <=
    6 * 2^1); scaled values 0.15 -> 0, -0.85 -> -1, 2.75 -> 3, 6 -> 6,
    1.25 -> 1 (tie, even code), -0.25 -> -0 (tie, even code), 2.5 -> 2 (tie)."""
    v = np.zeros(32)
    v[:7] = [0.3, -1.7, 5.5, 12.0, 2.5, -0.5, 5.0]
    packed, e = mxfp4.quantize_rows_fp4(v[None, :])
    assert e.tolist() == [[1]]
    codes = mxfp4.unpack_e2m1(packed)[0]
    assert codes[:7].tolist() == [0x0, 0xA, 0x5, 0x7, 0x2, 0x8, 0x4]
    assert packed[0, :4].tolist() == [0xA0, 0x75, 0x82, 0x04]
    np.testing.assert_array_equal(mxfp4.qdq_rows_fp4(v[None, :])[0, :7],
                                  [0.0, -2.0, 6.0, 12.0, 2.0, -0.0, 4.0])


def test_fp4_block_properties():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((40, 96)) * np.exp(rng.standard_normal((40, 96)))
    r = mxfp4.qdq_rows_fp4(w)
    for blk in range(3):
        v = w[:, 32 * blk:32 * blk + 32]
        s = np.ldexp(1.0, mxfp4.e8m0_exponent_fp4(np.abs(v).max(axis=1)))[:, None]
        assert np.all(np.abs(v / s) <= 6.0)
        # error <= half the grid spacing at the value (0.25, 0.5 or 1 times the scale)
        half = np.where(np.abs(v / s) < 2, 0.25, np.where(np.abs(v / s) < 4, 0.5, 1.0)) * s
        assert np.all(np.abs(r[:, 32 * blk:32 * blk + 32] - v) <= half)
    # power-of-two scaling commutes with the quantizer; grid values are fixed points
    np.testing.assert_array_equal(mxfp4.qdq_rows_fp4(w * 2.0 ** 7), r * 2.0 ** 7)
    np.testing.assert_array_equal(mxfp4.qdq_rows_fp4(r), r)
    # codes: unpacked, decoded and scaled, they are the quantize-dequantize values
    packed, e = mxfp4.quantize_rows_fp4(w)
    assert packed.shape == (40, 48) and e.shape == (40, 3)
    deq = mxfp4.e2m1_decode(mxfp4.unpack_e2m1(packed)) * np.ldexp(1.0, np.repeat(e, 32, 1))
    np.testing.assert_array_equal(deq, r)
    assert np.all(mxfp4.qdq_rows_fp4(np.zeros((2, 32))) == 0.0)


def test_mxfp4_expert_reduces_to_exact_path_without_rounding(monkeypatch):
    """With the E2M1 rounding and the BF16 rounding replaced by identity, the
    MXFP4 expert and layer must be the fp64 ones: every operand feeds the
    right GEMM, with the right scales."""
    rng = np.random.default_rng(3)
    T, D, F, E, K = 6, 64, 32, 3, 2
    x = rng.standard_normal((T, D)); w13 = rng.standard_normal((E, 2 * F, D))
    w2 = rng.standard_normal((E, D, F))
    ids = np.array([[0, 1], [1, 2], [2, -1], [0, 2], [1, 0], [-1, -1]])
    s = rng.random((T, K)); s[ids < 0] = 0
    ident = lambda v: np.asarray(v, dtype=np.float64)
    monkeypatch.setattr(mxfp4, "e2m1_round", ident)
    # act=None drops the BF16 rounding of the materialized h1 and h2
    np.testing.assert_allclose(mxfp4.expert_ffn_mxfp4(x, w13[0], w2[0], act=None)[2],
                               moe.expert_ffn(x, w13[0], w2[0])[2], rtol=1e-12, atol=1e-12)
    add = rng.standard_normal((T, D))
    np.testing.assert_allclose(mxfp4.forward(x, ids, s, w13, w2, y_addend=add, act=None),
                               moe.forward(x, ids, s, w13, w2, y_addend=add), rtol=1e-12, atol=1e-12)


def test_mxfp4_error_is_quantization_sized():
    """Four-bit operands: the layer moves away from the fp64 result by a few
    tens of percent of its largest output at most, and by much more than MXFP8
    does on the same inputs."""
    from oracle import mx
    rng = np.random.default_rng(4)
    M, D, F = 40, 256, 128
    x = rng.standard_normal((M, D))
    w13 = rng.standard_normal((2 * F, D)) / 16; w2 = rng.standard_normal((D, F)) / np.sqrt(F)
    r3 = moe.expert_ffn(x, w13, w2)[2]
    h3 = mxfp4.expert_ffn_mxfp4(x, mxfp4.qdq_rows_fp4(w13), mxfp4.qdq_rows_fp4(w2))[2]
    e4 = moe.max_abs_rel(h3, r3)
    e8 = moe.max_abs_rel(mx.expert_ffn_mx(x, mx.qdq_rows(w13), mx.qdq_rows(w2))[2], r3)
    assert 4 * e8 < e4 < 0.5


def test_subset_of_experts_sums_to_the_layer():
    rng = np.random.default_rng(5)
    T, D, F, E, K = 9, 64, 32, 4, 2
    x = rng.standard_normal((T, D)); w13 = rng.standard_normal((E, 2 * F, D))
    w2 = rng.standard_normal((E, D, F))
    ids = rng.integers(0, E, (T, K)); s = rng.random((T, K))
    full = mxfp4.forward(x, ids, s, w13, w2)
    parts = sum(mxfp4.forward(x, ids, s, w13, w2, experts=[e]) for e in range(E))
    np.testing.assert_allclose(parts, full, rtol=1e-12, atol=1e-12)
