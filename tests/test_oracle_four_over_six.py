"""Pins of oracle/four_over_six.py against facts the pages and the arithmetic
fix: blocks that one candidate represents exactly pick that candidate; a tie
keeps 6 (a planted ">=" rule changes the bytes); a block that picks 4 with an
exact block scale has error at most 1/8 of its max (the page's bound) while
6 allows up to 1/6; when every block picks 6 the result is plain NVFP4; the
choice agrees with exact rational sums of squares wherever those differ by
more than the binary32 rounding; the tile variant sums the squares over all
256 values; the pairwise tree is the stated order."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import four_over_six as Q
from oracle import nvfp4 as N

def _bf16(x):
    return F.bf16_bits_to_f64(F.bf16_rne(np.asarray(x, dtype=np.float64)))


def _dq_rows(c, s, S):
    return N.dequantize_f64(c, s, np.asarray(S, dtype=np.float32), "1x16",
                            "per_row" if np.size(S) > 1 else "per_tensor")


def test_tree_sum_order():
    v = np.float32([1e8, 1.0, -1e8, 1.0] + [0.0] * 12)
    # ((1e8 + 1) + (-1e8 + 1)) = (1e8) + (-1e8) = 0 in binary32; a left fold gives 1
    assert Q.tree_sum(v) == 0.0
    assert np.float32(np.float32(np.float32(1e8) + 1) - np.float32(1e8)) + 1 == 1.0


def test_block_exact_at_scale_four_picks_four():
    # S = 1 given: max 4 -> s4 = 1 exactly and every value sits on the grid;
    # s6 = E4M3(4/6) = 0.6875 leaves errors
    row = np.array([4, 3, 2, 1.5, 1, 0.5, 0, -3, -4, 2, 1, 0.5, 3, -2, 1.5, 0], dtype=np.float64)
    c, s, S, take4, e6, e4 = Q.quantize_rowwise(row[None, :], "given", np.float32(1.0), details=True)
    assert take4[0, 0] and e4[0, 0] == 0.0 and e6[0, 0] > 0.0
    assert F.e4m3_value(s)[0, 0] == 1.0
    assert np.array_equal(_dq_rows(c, s, S)[0], row)


def test_block_exact_at_scale_six_picks_six():
    row = np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, 2, 1, 0.5, 3, 4], dtype=np.float64)
    c, s, S, take4, e6, e4 = Q.quantize_rowwise(row[None, :], "given", np.float32(1.0), details=True)
    assert not take4[0, 0] and e6[0, 0] == 0.0 and e4[0, 0] > 0.0
    assert np.array_equal(_dq_rows(c, s, S)[0], row)
    # identical to plain NVFP4 when 6 is chosen
    pc, ps, pS = N.quantize_rowwise(row[None, :], "given", S_given=np.float32(1.0))
    assert np.array_equal(c, pc) and np.array_equal(s, ps)


def test_tie_keeps_six():
    # values in {0, a/4, a/2, a}, a = 12: s6 = 2 and s4 = 3 (both exact E4M3)
    # represent the block exactly, so the errors tie at 0 and 6 is kept
    row = np.array([12, 6, 3, 0, -12, -6, -3, 0, 12, 3, 6, 0, -3, 3, -6, 12], dtype=np.float64)
    c, s, S, take4, e6, e4 = Q.quantize_rowwise(row[None, :], "given", np.float32(1.0), details=True)
    assert e6[0, 0] == 0.0 and e4[0, 0] == 0.0 and not take4[0, 0]
    assert F.e4m3_value(s)[0, 0] == 2.0
    # a planted ">=" rule would store s4 = 3 instead: the bytes differ
    assert F.encode_e4m3_rne(np.array([3.0]))[0] != s[0, 0]
    # all-zero block: both errors 0, code 0 scale
    z = np.zeros((1, 16))
    _, sz, _, tz, _, _ = Q.quantize_rowwise(z, "per_row", details=True)
    assert sz[0, 0] == 0 and not tz[0, 0]


def test_error_bounds_one_eighth_and_one_sixth():
    rs = np.random.default_rng(1)
    x = _bf16(rs.standard_normal((512, 256)))
    c, s, S, take4, _, _ = Q.quantize_rowwise(x, "per_row", details=True)
    dq = _dq_rows(c, s, S).reshape(512, 16, 16)
    xb = x.reshape(512, 16, 16)
    a_b = np.abs(xb).max(axis=-1)
    err = np.abs(dq - xb).max(axis=-1)
    sb = F.e4m3_value(s)
    S_b = np.repeat(S[:, None], 16, axis=1).astype(np.float64)
    # blocks whose chosen scale is exactly a_b / (M S): the page's bounds
    exact4 = take4 & (sb * S_b * 4 == a_b)
    exact6 = ~take4 & (sb * S_b * 6 == a_b)
    assert np.all(err[exact4] <= a_b[exact4] / 8 * (1 + 1e-6))
    assert np.all(err[exact6] <= a_b[exact6] / 6 * (1 + 1e-6))
    # in general the E4M3 rounding of s4 adds at most 1/16 relative, unless s4
    # saturated at 448 (the block's max then lands between 4 and 6 and the
    # choice rests on the sum of squares alone)
    unsat4 = take4 & (s != 0x7E)
    assert np.all(err[unsat4] <= a_b[unsat4] / 8 * (1 + 1 / 16) + 1e-30)
    assert np.any(take4 & (s == 0x7E))
    assert take4.sum() > 0.2 * take4.size and (~take4).sum() > 0.2 * take4.size


def _exact_sse(xb, codes, sb, S):
    sv = Fraction(float(F.e4m3_value(np.uint8(sb))))
    Sv = Fraction(float(np.float32(S)))
    tot = Fraction(0)
    for xv, cv in zip(xb, codes):
        # binary32 dequantized value, then the exact squared error
        d = np.float32(np.float32(np.float32(F.e2m1_value(np.uint8(cv))) * np.float32(sv)) * np.float32(Sv))
        tot += (Fraction(float(xv)) - Fraction(float(d))) ** 2
    return tot


def test_choice_matches_exact_sums_of_squares():
    rs = np.random.default_rng(2)
    x = _bf16(rs.standard_normal((40, 64)) * np.exp(rs.standard_normal((40, 1))))
    c, s, S, take4, e6, e4 = Q.quantize_rowwise(x, "per_row", details=True)
    xb = x.reshape(40, 4, 16)
    checked = 0
    for r in range(40):
        for b in range(4):
            a_b = np.abs(xb[r, b]).max()
            s6, c6, _ = Q.candidate(xb[r, b][None], np.array([a_b]), np.float32(S[r]), 6)
            s4, c4, _ = Q.candidate(xb[r, b][None], np.array([a_b]), np.float32(S[r]), 4)
            E6 = _exact_sse(xb[r, b], c6[0], s6[0], S[r])
            E4 = _exact_sse(xb[r, b], c4[0], s4[0], S[r])
            # binary32 squares and tree sums: relative error below 2^-19 of the larger
            big = max(E6, E4)
            if abs(E6 - E4) > big * Fraction(1, 2 ** 19):
                assert bool(take4[r, b]) == (E4 < E6)
                checked += 1
    assert checked > 100


def test_tile_variant_uses_all_256_values():
    # a 16x16 tile with max 4 and every value on the grid under s4 = 1: picks 4
    rs = np.random.default_rng(3)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4])
    t = rs.choice(grid, (16, 16)) * rs.choice([-1, 1], (16, 16))
    t[0, 0] = 4
    c, s, S, take4, e6, e4 = Q.quantize_tile16(t, "given", np.float32(1.0), details=True)
    assert take4[0, 0] and e4[0, 0] == 0.0
    dq = N.dequantize_f64(c, s, S, "16x16", "per_tensor")
    assert np.array_equal(dq, t)
    # a random tensor: one choice per tile, the error summed over all 256 values
    big = _bf16(rs.standard_normal((64, 48)))
    c2, s2, S2, t2, e62, e42 = Q.quantize_tile16(big, details=True)
    assert t2.shape == (4, 3)
    # tile error equals the row-by-row tree of squares
    xt = big.reshape(4, 16, 3, 16).transpose(0, 2, 1, 3)
    a = np.abs(xt).max(axis=(2, 3))
    s6, c6, d6 = Q.candidate(xt.reshape(4, 3, 256), a, np.full(a.shape, S2[0], np.float32), 6)
    sq = Q.squared_errors(xt.reshape(4, 3, 256), d6).reshape(4, 3, 16, 16)
    assert np.array_equal(Q.tree_sum(Q.tree_sum(sq)), e62)


def test_per_tensor_and_per_row_scales():
    rs = np.random.default_rng(4)
    x = _bf16(rs.standard_normal((32, 128)) * np.exp(rs.standard_normal((32, 1)) * 2))
    c, s, S = Q.quantize_rowwise(x, "per_row")
    assert np.array_equal(S, N.second_scale(np.abs(x).max(axis=1)))
    c2, s2, S2 = Q.quantize_rowwise(x, "per_tensor")
    assert S2.shape == (1,) and S2[0] == N.second_scale(np.abs(x).max())
    # 4/6 never raises the float64 squared error of a block much above plain NVFP4's
    pc, ps, pS = N.quantize_rowwise(x, "per_row")
    e46 = ((_dq_rows(c, s, S) - x) ** 2).reshape(32, 8, 16).sum(-1)
    epl = ((_dq_rows(pc, ps, pS) - x) ** 2).reshape(32, 8, 16).sum(-1)
    assert np.all(e46 <= epl * (1 + 2.0 ** -18) + 1e-300)
    assert np.sum(e46) < np.sum(epl)
