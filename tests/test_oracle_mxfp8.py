"""Pins of oracle/mxfp8.py: brute-force search of the block exponent, closed
forms for special blocks, the no-overflow rule, idempotence as characterised,
transpose consistency, batch invariance, and exact dequantization checked
against PyTorch's float8 decoder."""

import itertools

import numpy as np
import torch

from oracle import formats as F
from oracle import mxfp8 as M


def _bf16_set64():
    vals = [0.0, 2.0 ** -133, 3 * 2.0 ** -133, 2.0 ** -127, 2.0 ** -126, 2.0 ** -120,
            1e-30, 2.0 ** -10, 0.001, 0.1, 0.5, 0.875, 1.0, 1.5, 1.75, 1.7578125, 2.0, 3.0,
            7.0, 100.0, 224.0, 232.0, 240.0, 255.0, 256.0, 448.0, 456.0, 464.0, 480.0, 500.0,
            1e4, 65504.0, 1e20, 3.3895313892515355e38]
    x = np.array(vals, dtype=np.float32)
    x = F.bf16_bits_to_f64(F.bf16_rne(x.astype(np.float64)))
    x = np.unique(np.concatenate([x, -x[x > 0][:30]]))
    return x[:64]


def test_block_exponent_bruteforce_two_element_blocks():
    vals = _bf16_set64()
    es = np.arange(-127, 128)
    for a, b in itertools.product(vals, vals):
        amax = max(abs(a), abs(b))
        fits = [e for e in es if abs(a) * 2.0 ** -e <= 448 and abs(b) * 2.0 ** -e <= 448]
        want = min(fits)
        got = int(M.block_exponent(np.array([amax]))[0])
        assert got == want, (a, b, got, want)


def test_power_of_two_and_448_blocks():
    rs = np.random.default_rng(0)
    for k in range(-100, 100, 7):
        x = rs.uniform(-1, 1, (1, 32)) * 2.0 ** k
        x = F.bf16_bits_to_f64(F.bf16_rne(x))
        x[0, 5] = 2.0 ** k
        codes, sc = M.quantize_rowwise(x)
        assert codes[0, 5] == 0x78 and sc[0, 0] == k - 8 + 127
        x[0, 5] = 448.0 * 2.0 ** k
        codes, sc = M.quantize_rowwise(x)
        assert codes[0, 5] == 0x7E and sc[0, 0] == k + 127


def test_zero_block_and_signed_zero():
    x = np.zeros((1, 64))
    x[0, 33] = -0.0
    x[0, 40] = -1.0
    codes, sc = M.quantize_rowwise(x)
    assert sc[0, 0] == 0 and np.all(codes[0, :32] == 0)
    assert codes[0, 33] == 0x80
    assert codes[0, 40] == 0xF8 and sc[0, 1] == 127 - 8


def _rand_bf16(shape, seed, spread=4.0):
    rs = np.random.default_rng(seed)
    x = rs.standard_normal(shape) * np.exp(rs.standard_normal(shape[:-1] + (1,)) * spread)
    return F.bf16_bits_to_f64(F.bf16_rne(x))


def test_no_overflow_and_scale_minimal():
    x = _rand_bf16((64, 256), 1)
    codes, sc = M.quantize_rowwise(x)
    e = sc.astype(np.int64) - 127
    amax = np.abs(x).reshape(64, 8, 32).max(-1)
    assert np.all(amax <= 448 * 2.0 ** e)
    assert np.all((amax <= 448 * 2.0 ** (e - 1)) == (amax == 0) | (e == -127))
    assert np.all((codes & 0x7F) <= 0x7E)


def test_idempotence_as_characterised():
    """DQ(Q(DQ(Q(x)))) == DQ(Q(x)) in value; bytes equal unless the block's
    largest magnitude code is 224 (then the re-derived exponent is one lower and
    every code doubles)."""
    x = _rand_bf16((128, 512), 2, spread=2.0)
    c1, s1 = M.quantize_rowwise(x)
    d1 = M.dequantize_bf16(c1, s1)
    c2, s2 = M.quantize_rowwise(F.bf16_bits_to_f64(d1))
    d2 = M.dequantize_bf16(c2, s2)
    assert np.array_equal(d1, d2)
    cmax = np.abs(F.e4m3_value(c1)).reshape(128, 16, 32).max(-1)
    same = cmax != 224.0
    assert np.array_equal(s1[same], s2[same])
    cb1 = c1.reshape(128, 16, 32)
    cb2 = c2.reshape(128, 16, 32)
    assert np.array_equal(cb1[same], cb2[same])
    assert np.array_equal(s2[~same].astype(int), s1[~same].astype(int) - 1)
    assert np.array_equal(F.e4m3_value(cb2[~same]), 2 * F.e4m3_value(cb1[~same]))
    assert (~same).any()          # the special case does occur in this sample


def test_tile32_transpose_consistency():
    x = _rand_bf16((96, 160), 3)
    c, s = M.quantize_tile32(x)
    ct, st = M.quantize_tile32(np.ascontiguousarray(x.T))
    assert np.array_equal(ct, c.T) and np.array_equal(st, s.T)


def test_colwise_is_rowwise_blocks_along_rows():
    x = _rand_bf16((64, 96), 4)
    c, s = M.quantize_colwise(x)
    for col in range(96):
        for rb in range(2):
            blk = x[rb * 32:(rb + 1) * 32, col]
            cc, ss = M.quantize_rowwise(blk.reshape(1, 32))
            assert np.array_equal(c[col, rb * 32:(rb + 1) * 32], cc[0]) and s[col, rb] == ss[0, 0]


def test_batch_composition_invariance():
    x = _rand_bf16((48, 128), 5)
    c, s = M.quantize_rowwise(x)
    for r in (0, 17, 47):
        c1, s1 = M.quantize_rowwise(x[r:r + 1])
        assert np.array_equal(c1[0], c[r]) and np.array_equal(s1[0], s[r])


def test_dequantize_matches_torch_float8_decode():
    x = _rand_bf16((32, 128), 6)
    c, s = M.quantize_rowwise(x)
    dec = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    want = np.ldexp(dec, e)
    assert np.array_equal(M.dequantize_f64(c, s), want)
    # BF16 DQ is exact in the normal range
    assert np.array_equal(F.bf16_bits_to_f64(M.dequantize_bf16(c, s)), want)


def test_max_bf16_input():
    x = np.zeros((1, 32))
    x[0, 0] = 3.3895313892515355e38       # largest finite BF16
    x[0, 1] = -1.0
    c, s = M.quantize_rowwise(x)
    assert s[0, 0] == 120 + 127 and c[0, 0] == 0x78   # 255 * 2^120 rounds to 256 * 2^120
    assert c[0, 1] == 0x80                             # far below the block's range
