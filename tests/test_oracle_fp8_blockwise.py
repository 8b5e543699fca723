"""Pins of oracle/fp8_blockwise.py: a 1x128 block's exponent is the largest
of its four 1x32 MXFP8 exponents (the rule is monotone in the amax) and the
codes of every 32-value sub-block with that same exponent equal MXFP8's; the
exponent is found by brute force on small blocks; values on one power of two
times the E4M3 grid dequantize exactly; the relative error of normal-range
elements is at most 2^-4; the 128x128 tile's exponent is the largest of its
rows' 1x128 exponents and its copy of x^T is the same codes transposed; a
planted wrong block size (32 for 128) is rejected.  The binary32-scale arm
has pins of its own (below)."""

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


# ------------------------------------------------------------ FP32 scales
# Pins of the binary32-scale arm: s is amax / 448 rounded once to binary32
# (checked against the float64 quotient rounded to binary32, a different
# route); the block maximum always encodes to +-448; blocks whose maximum is
# 448 * 2^k reduce to the power-of-two rule (same codes, s = 2^k); every
# element lies within half an E4M3 step of x / s; zero blocks; tiles take the
# largest row scale; the transposed tile copy; the GEMM's block-sum form.

def _mixed_blocks(rows, seed):
    """Blocks of 128 with magnitudes from BF16 subnormals to 2^60."""
    rs = np.random.default_rng(seed)
    x = rs.standard_normal((rows, 512)) * np.exp2(rs.integers(-140, 60, (rows, 4)).repeat(128, 1))
    return _bf16(x)


def test_f32_scale_is_rounded_quotient_and_max_code_is_448():
    x = _mixed_blocks(64, 11)
    c, s = B.quantize_rows_f32(x)
    assert s.dtype == np.float32 and s.shape == (64, 4)
    amax = np.abs(x).reshape(64, 4, 128).max(-1)
    assert np.array_equal(s, (amax / 448.0).astype(np.float32))
    v = F.e4m3_value(c).reshape(64, 4, 128)
    assert np.all(np.abs(v).max(-1)[amax > 0] == 448.0)
    # the element holding the maximum carries its sign
    xb = x.reshape(64, 4, 128)
    i = np.abs(xb).argmax(-1)[..., None]
    assert np.array_equal(np.sign(np.take_along_axis(v, i, -1)), np.sign(np.take_along_axis(xb, i, -1)))


def test_f32_power_of_two_blocks_reduce_to_the_pow2_rule():
    rs = np.random.default_rng(12)
    grid = F.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8))
    vals = rs.choice(grid, (16, 256)) * rs.choice([-1.0, 1.0], (16, 256))
    vals[:, ::128] = 448.0
    k = rs.integers(-20, 20, (16, 2)).repeat(128, 1)
    x = vals * np.exp2(k)
    c, s = B.quantize_rows_f32(x)
    c2, s2 = B.quantize_rows(x)
    assert np.array_equal(c, c2)
    assert np.array_equal(s.astype(np.float64), np.exp2(s2.astype(np.float64) - 127))
    assert np.array_equal(B.dequantize_f32s_f64(c, s), x)


def test_f32_error_within_half_an_e4m3_step():
    x = _mixed_blocks(128, 13)
    c, s = B.quantize_rows_f32(x)
    se = B.scale_f32_per_element(s, "1x128")
    q = x / np.where(se == 0, 1, se)
    d = F.e4m3_value(c)
    # half an E4M3 step at |q| (2^-10 below the normal range 2^-6), plus the
    # binary32 rounding of the quotient
    step = np.where(np.abs(q) >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(np.abs(q), 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(d - q) <= step / 2 + np.abs(q) * 2.0 ** -23 + 1e-300)
    # relative error of normal-range elements of the dequantized copy
    normal = np.abs(q) >= 2.0 ** -6
    dq = B.dequantize_f32s_f64(c, s)
    assert np.all(np.abs(dq - x)[normal] <= (2.0 ** -4 + 2.0 ** -22) * np.abs(x)[normal])


def test_f32_zero_blocks_and_bf16_copy():
    x = _mixed_blocks(8, 14)
    x[3, 128:256] = 0
    x[5] = -0.0
    c, s = B.quantize_rows_f32(x)
    assert s[3, 1] == 0 and np.all(c[3, 128:256] & 0x7F == 0)
    assert np.all(s[5] == 0) and np.all(B.dequantize_f32s_f64(c[5:6], s[5:6]) == 0)
    exact = B.dequantize_f32s_f64(c, s)
    b = F.bf16_bits_to_f64(B.dequantize_f32s_bf16(c, s))
    fin = np.isfinite(b) & (np.abs(exact) > 2.0 ** -120)
    ulp = np.exp2(np.floor(np.log2(np.abs(exact[fin]))) - 7)
    assert np.all(np.abs(b[fin] - exact[fin]) <= ulp / 2 + np.abs(exact[fin]) * 2.0 ** -24)


def test_f32_tile_scale_and_transposed_copy_and_columns():
    x = _bf16(np.random.default_rng(15).standard_normal((256, 384)) * 3)
    c, s = B.quantize_tile_f32(x)
    _, sr = B.quantize_rows_f32(x)
    assert s.shape == (2, 3) and np.array_equal(s, sr.reshape(2, 128, 3).max(axis=1))
    ct, st = B.quantize_tile_f32(np.ascontiguousarray(x.T))
    assert np.array_equal(ct, c.T) and np.array_equal(st, s.T)
    cc, sc = B.quantize_cols_f32(x)
    c2, s2 = B.quantize_rows_f32(np.ascontiguousarray(x.T))
    assert np.array_equal(cc, c2) and np.array_equal(sc, s2)
    # a planted block of 64 gives other scales
    amax64 = np.abs(x).reshape(256, 6, 64).max(-1)
    assert not np.array_equal(np.repeat(sr, 2, axis=1), (amax64 / 448.0).astype(np.float32))


def test_f32_gemm_block_sum_form():
    """sum_kb s_a[m,kb] s_b[n,kb] (C_a C_b^T)_kb equals the dequantize-then-
    matmul product: the per-block scale indexing of both operands."""
    rs = np.random.default_rng(16)
    a = _bf16(rs.standard_normal((96, 512)) * np.exp2(rs.integers(-3, 3, (96, 4)).repeat(128, 1)))
    b = _bf16(rs.standard_normal((256, 512)) * 0.05)
    ca, sa = B.quantize_rows_f32(a)
    cb, sb = B.quantize_tile_f32(b)
    ref = B.dequantize_f32s_f64(ca, sa) @ B.dequantize_f32s_f64(cb, sb, "128x128").T
    va, vb = F.e4m3_value(ca), F.e4m3_value(cb)
    out = np.zeros((96, 256))
    for kb in range(4):
        k = slice(128 * kb, 128 * kb + 128)
        p = va[:, k] @ vb[:, k].T
        out += sa[:, kb, None].astype(np.float64) * np.repeat(sb[:, kb], 128)[None, :].astype(np.float64) * p
    mag = np.abs(B.dequantize_f32s_f64(ca, sa)) @ np.abs(B.dequantize_f32s_f64(cb, sb, "128x128")).T
    assert np.all(np.abs(out - ref) <= 1e-13 * mag)
    # a planted wrong K-block index for the weight scale breaks it
    bad = np.zeros((96, 256))
    for kb in range(4):
        k = slice(128 * kb, 128 * kb + 128)
        bad += sa[:, kb, None] * np.repeat(sb.T[kb % 2 if sb.shape[0] > 1 else 0], 128)[None, :256] * (va[:, k] @ vb[:, k].T)
    assert not np.all(np.abs(bad - ref) <= 1e-13 * mag)
