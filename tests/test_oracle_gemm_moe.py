"""Pins of oracle/gemm.py, oracle/moe.py and oracle/layout.py: exact rational
triple loops on tiny inputs, the unit-scale exact special case, brute-force
routing, and planted mistakes (in the oracle's inputs, on the CPU) that the
acceptance check must reject."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import layout as L
from oracle import moe
from oracle import mxfp8 as M
from oracle import nvfp4 as N


def _rand_bf16(shape, seed, std=1.0):
    rs = np.random.default_rng(seed)
    return F.bf16_bits_to_f64(F.bf16_rne(rs.standard_normal(shape) * std))


def test_gemm_f64_matches_exact_triple_loop():
    a = _rand_bf16((5, 64), 0)
    b = _rand_bf16((3, 64), 1)
    c = G.gemm_f64(a, b)
    for i in range(5):
        for j in range(3):
            exact = sum(Fraction(float(a[i, k])) * Fraction(float(b[j, k])) for k in range(64))
            assert abs(Fraction(float(c[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_mxfp8_gemm_reference_is_dequantize_then_matmul():
    x = _rand_bf16((64, 128), 2)
    w = _rand_bf16((32, 128), 3, 0.02)
    cx, sx = M.quantize_rowwise(x)
    cw, sw = M.quantize_rowwise(w)
    ax, bw = M.dequantize_f64(cx, sx), M.dequantize_f64(cw, sw)
    c64 = G.gemm_f64(ax, bw)
    i, j = 7, 11
    exact = sum(Fraction(float(ax[i, k])) * Fraction(float(bw[j, k])) for k in range(128))
    assert abs(Fraction(float(c64[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 48)


def test_unit_scale_products_are_exact_in_any_order():
    """With unit scales and small-integer E4M3 codes (or any E2M1 codes with
    s_b = 1, S = 1) every product is a multiple of 2^-2 of magnitude <= 256, so
    binary32 sums are exact for K <= 2^14: the FP32 path equals float64."""
    rs = np.random.default_rng(4)
    small = np.array([v for v in F.e4m3_value(np.arange(256)) if np.isfinite(v)
                      and abs(v) <= 16 and (4 * v) == int(4 * v)])
    a = rs.choice(small, (32, 4096))
    b = rs.choice(small, (16, 4096))
    assert np.array_equal(G.gemm_f32(a, b).astype(np.float64), G.gemm_f64(a, b))
    e2 = F.e2m1_value(np.arange(16))
    a = rs.choice(e2, (32, 4096))
    b = rs.choice(e2, (16, 4096))
    assert np.array_equal(G.gemm_f32(a, b).astype(np.float64), G.gemm_f64(a, b))


def _nvfp4_operands(seed):
    x = _rand_bf16((96, 256), seed)
    w = _rand_bf16((48, 256), seed + 1, 0.02)
    cx, sx, Sx = N.quantize_rowwise(x, "per_row")
    cw, sw, Sw = N.quantize_tile16(w)
    a64 = N.dequantize_f64(cx, sx, Sx, "1x16", "per_row")
    b64 = N.dequantize_f64(cw, sw, Sw, "16x16", "per_tensor")
    a32 = N.dequantize_f32(cx, sx, Sx, "1x16", "per_row")
    b32 = N.dequantize_f32(cw, sw, Sw, "16x16", "per_tensor")
    return a64, b64, a32, b32


def test_check_accepts_a_correct_result_and_rejects_planted_mistakes():
    a64, b64, a32, b32 = _nvfp4_operands(5)
    good = F.bf16_rne(G.gemm_f64(a64, b64))
    frob, worst, ok = G.check(good, a64, b64, a32, b32)
    assert ok and frob < 4e-3 and worst <= 1.0
    # planted mistakes in what the checker is given
    wrong_t = F.bf16_rne(G.gemm_f64(a64, b64[::-1]))                 # rows of B permuted
    assert not G.check(wrong_t, a64, b64, a32, b32)[2]
    wrong_s = F.bf16_rne(G.gemm_f64(a64 * 2.0, b64))                  # a dropped/doubled scale
    assert not G.check(wrong_s, a64, b64, a32, b32)[2]
    wrong_sign = good.copy()
    wrong_sign[3, 4] ^= 0x8000                                        # one flipped sign
    if F.bf16_bits_to_f64(good[3:4, 4:5])[0, 0] != 0:
        assert not G.check(wrong_sign, a64, b64, a32, b32)[2]


def test_route_topk_bruteforce():
    rs = np.random.default_rng(6)
    logits = rs.standard_normal((50, 16)).astype(np.float32)
    logits[3, 5] = logits[3, 9]                                       # a planted tie
    top = moe.route_topk(logits, 4)
    for t in range(50):
        order = sorted(range(16), key=lambda e: (-float(logits[t, e]), e))[:4]
        assert list(top[t]) == order


def test_group_rows():
    rs = np.random.default_rng(7)
    logits = rs.standard_normal((64, 8)).astype(np.float32)
    top = moe.route_topk(logits, 2)
    row_token, off = moe.group_rows(top, 8)
    assert off[0] == 0 and off[-1] == 128 and np.all(np.diff(off) >= 0)
    pairs = set()
    for g in range(8):
        toks = row_token[off[g]:off[g + 1]]
        assert np.all(np.diff(toks) > 0)
        for t in toks:
            assert g in top[t]
            pairs.add((int(t), g))
    assert len(pairs) == 128


def test_grouped_gemm_matches_per_row():
    rs = np.random.default_rng(8)
    a = rs.standard_normal((20, 32))
    b = rs.standard_normal((3, 6, 32))
    off = np.array([0, 7, 7, 20])
    c = moe.grouped_gemm_f64(a, b, off)
    for r in range(20):
        g = int(np.searchsorted(off, r, side="right") - 1)
        assert np.allclose(c[r], b[g] @ a[r], rtol=1e-13, atol=1e-13)


def test_swiglu_reference():
    """SwiGLU h = silu(g) * u with the gate in the first half of the row.
    Pinned to textbook values of the logistic function sigma(x) = 1 / (1 +
    e^-x) (sigma(1) = 0.7310585786300049, sigma(2) = 0.8807970779778823,
    sigma(3) = 0.9525741268224334), so silu(g) * u = g * sigma(g) * u is known
    without evaluating exp: a swapped gate/up, a flipped exponent sign or a
    missing factor changes the BF16 result."""
    s1, s2, s3 = 0.7310585786300049, 0.8807970779778823, 0.9525741268224334
    #       g:   1,    -2,   3,   0,   2     u:  -1,  0.5,  4,   2,  1
    gu = F.bf16_rne(np.array([[1.0, -2.0, 3.0, 0.0, 2.0, -1.0, 0.5, 4.0, 2.0, 1.0]]))
    want = np.array([[1.0 * s1 * -1.0,              # -0.7310585786...
                      -2.0 * (1.0 - s2) * 0.5,      # -0.1192029220...
                      3.0 * s3 * 4.0,               # 11.430889521...
                      0.0,
                      2.0 * s2 * 1.0]])             # 1.7615941559...
    assert np.array_equal(moe.swiglu_f64(gu, 5), F.bf16_rne(want))
    # the BF16 codes themselves, for the first three
    assert [int(v) for v in moe.swiglu_f64(gu, 5)[0, :3]] == [0xBF3B, 0xBDF4, 0x4137]


def test_mfma_layout_is_a_permutation_and_round_trips():
    rs = np.random.default_rng(9)
    s = rs.integers(0, 255, (64, 8), dtype=np.uint8)
    flat = L.linear_to_mfma(s)
    assert sorted(flat.tolist()) == sorted(s.ravel().tolist())
    assert np.array_equal(L.mfma_to_linear(flat, 64, 8), s)
    offs = sorted(L.mfma_offset(r, b, 8) for r in range(64) for b in range(8))
    assert offs == list(range(64 * 8))
    # the 4 blocks of a row inside one chunk are adjacent bytes
    assert [L.mfma_offset(33, b, 8) for b in range(4, 8)] == [3 * 128 + 4 + i for i in range(4)]


@pytest.mark.parametrize("shape", [(32, 64), (96, 32)])
def test_mxfp8_dual_copies_equal_separate_ones(shape):
    x = _rand_bf16(shape, 10)
    cr, sr = M.quantize_rowwise(x)
    cc, sc = M.quantize_colwise(x)
    assert cr.shape == shape and cc.shape == shape[::-1]
    assert sr.shape == (shape[0], shape[1] // 32) and sc.shape == (shape[1], shape[0] // 32)
