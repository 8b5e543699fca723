"""Pins of oracle/fp8_blockwise.py: a 1x128 block's exponent is the largest
of its four 1x32 MXFP8 exponents (the rule is monotone in the amax) and the
codes of every 32-value sub-block with that same exponent equal MXFP8's; the
exponent is found by brute force on small blocks; values on one power of two
times the E4M3 grid dequantize exactly; the relative error of normal-range
elements is at most 2^-4; the 128x128 tile's exponent is the largest of its
rows' 1x128 exponents and its copy of x^T is the same codes transposed; a
planted wrong block size (32 for 128) is rejected."""

import numpy as np

from oracle import formats as F
from oracle import fp8_blockwise as B
from oracle import mxfp8 as M


def _bf16(x):
    return F.bf16_bits_to_f64(F.bf16_rne(np.asarray(x, dtype=np.float64)))


def _x(rows, cols, seed):
    rs = np.random.default_rng(seed)
    return _bf16(rs.standard_normal((rows, cols)) * np.exp(rs.standard_normal((rows, cols // 32)).repeat(32, 1) * 2))


def test_row_exponent_is_max_of_mxfp8_exponents_and_codes_agree():
    x = _x(64, 512, 1)
    c, s = B.quantize_rows(x)
    mc, ms = M.quantize_rowwise(x)
    s4 = ms.reshape(64, 4, 4)
    assert np.array_equal(s, s4.max(axis=-1))
    same = (s4 == s[..., None]).repeat(32, axis=-1).reshape(64, 512)
    assert same.mean() > 0.2
    assert np.array_equal(c[same], mc[same])
    # a planted block size of 32 gives different scales
    assert not np.array_equal(np.repeat(s, 4, axis=1), ms)


def test_exponent_by_brute_force():
    rs = np.random.default_rng(2)
    for _ in range(200):
        row = _bf16(rs.standard_normal(128) * 2.0 ** rs.integers(-40, 40))
        _, s = B.quantize_rows(row[None])
        a = np.abs(row).max()
        es = [e for e in range(-127, 128) if a <= 448.0 * 2.0 ** e]
        assert int(s[0, 0]) - 127 == min(es)
    z = np.zeros((1, 128))
    c, s = B.quantize_rows(z)
    assert s[0, 0] == 0 and np.all(c == 0)


def test_exact_values_round_trip_and_error_bound():
    rs = np.random.default_rng(3)
    grid = F.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8))
    vals = rs.choice(grid, (32, 256)) * rs.choice([-1.0, 1.0], (32, 256))
    vals[:, ::128] = 448.0                       # each block's max on the grid top
    x = vals * 2.0 ** 5
    c, s = B.quantize_rows(x)
    assert np.array_equal(B.dequantize_f64(c, s), x)
    y = _x(32, 1024, 4)
    c, s = B.quantize_rows(y)
    d = B.dequantize_f64(c, s)
    e = B.scale_per_element(s, y.shape, "1x128").astype(np.float64)
    normal = np.abs(y) >= 2.0 ** -6 * np.exp2(e)
    assert np.all(np.abs(d - y)[normal] <= 2.0 ** -4 * np.abs(y)[normal])


def test_columnwise_copy_is_rows_of_the_transpose():
    x = _x(256, 128, 5)
    c, s = B.quantize_cols(x)
    c2, s2 = B.quantize_rows(np.ascontiguousarray(x.T))
    assert c.shape == (128, 256) and np.array_equal(c, c2) and np.array_equal(s, s2)


def test_tile_exponent_and_transposed_copy():
    x = _x(256, 384, 6)
    c, s = B.quantize_tile(x)
    _, sr = B.quantize_rows(x)
    assert s.shape == (2, 3)
    assert np.array_equal(s, sr.reshape(2, 128, 3).max(axis=1))
    ct, st = B.quantize_tile(np.ascontiguousarray(x.T))
    assert np.array_equal(ct, c.T) and np.array_equal(st, s.T)
    d = B.dequantize_f64(c, s, "128x128")
    assert np.max(np.abs(d - x)) <= 2.0 ** -4 * np.abs(x).max()
