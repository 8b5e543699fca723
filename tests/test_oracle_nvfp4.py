"""Pins of oracle/nvfp4.py: closed-form special cases, the binary32 step
chain checked against exact rational arithmetic, no-overflow bounds,
idempotence, transpose consistency of 16x16 tiles, batch-composition and
gather invariance of per-token scaling, shared gate/up scale, and stochastic
rounding unbiasedness over many seeds."""

from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import nvfp4 as N
from oracle import moe


def _rand_bf16(shape, seed, spread=3.0):
    rs = np.random.default_rng(seed)
    x = rs.standard_normal(shape) * np.exp(rs.standard_normal(shape[:-1] + (1,)) * spread)
    return F.bf16_bits_to_f64(F.bf16_rne(x))


def _round_f32(q):
    """Correctly rounded binary32 of an exact rational (for normal results)."""
    f = np.float32(float(q))
    best = f
    for cand in (np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))):
        if abs(Fraction(float(cand)) - q) < abs(Fraction(float(best)) - q):
            best = cand
    return best


def test_token_max_element_gets_code_6_and_scale_448():
    x = _rand_bf16((64, 256), 0)
    codes, sb, S = N.quantize_rowwise(x, "per_row")
    c = N.unpack_nibbles(codes)
    for r in range(64):
        j = int(np.argmax(np.abs(x[r])))
        assert sb[r, j // 16] == 0x7E
        assert (c[r, j] & 7) == 7 and ((c[r, j] >> 3) & 1) == int(x[r, j] < 0)


def test_scale_chain_against_exact_arithmetic():
    x = _rand_bf16((8, 64), 1)
    codes, sb, S = N.quantize_rowwise(x, "per_row")
    c = N.unpack_nibbles(codes)
    for r in range(8):
        A = max(abs(Fraction(float(v))) for v in x[r])
        s = _round_f32(A / 2688)
        assert s == S[r]
        six_s = _round_f32(6 * Fraction(float(s)))
        for b in range(4):
            blk = x[r, b * 16:(b + 1) * 16]
            ab = max(abs(Fraction(float(v))) for v in blk)
            t = _round_f32(ab / Fraction(float(six_s)))
            # nearest E4M3 value to t, ties to the even code, by search over the grid
            dists = [abs(Fraction(float(g)) - Fraction(float(t))) for g in F.E4M3_GRID]
            best = min(dists)
            cands = [i for i, d in enumerate(dists) if d == best]
            want_sb = [i for i in cands if i % 2 == 0][0] if len(cands) > 1 else cands[0]
            assert sb[r, b] == want_sb
            sbv = Fraction(float(F.E4M3_GRID[want_sb]))
            den = _round_f32(sbv * Fraction(float(s)))
            rr = _round_f32(1 / Fraction(float(den)))
            for k in range(16):
                y = _round_f32(Fraction(float(blk[k])) * Fraction(float(rr)))
                d = [abs(Fraction(float(g)) - abs(Fraction(float(y)))) for g in F.E2M1_GRID]
                m = min(d)
                cc = [i for i, dd in enumerate(d) if dd == m]
                want = [i for i in cc if i % 2 == 0][0] if len(cc) > 1 else cc[0]
                assert (c[r, b * 16 + k] & 7) == want


def test_no_overflow_bounds():
    x = _rand_bf16((256, 512), 2, spread=5.0)
    codes, sb, S = N.quantize_rowwise(x, "per_row")
    A = np.abs(x).max(axis=1)
    ab = np.abs(x).reshape(256, 32, 16).max(-1)
    six_s = (np.float32(6) * S).astype(np.float32)
    t = (ab.astype(np.float32) / six_s[:, None]).astype(np.float32)
    assert np.all(t <= 448 * (1 + 2.0 ** -22))
    assert np.all(sb <= 0x7E)
    assert np.all(S == (A.astype(np.float32) / np.float32(2688)).astype(np.float32))


def test_zero_rows_and_signed_zeros():
    x = np.zeros((3, 32))
    x[1, 3] = -0.0
    x[2, 0] = -2.0
    x[2, 20] = 1.0
    codes, sb, S = N.quantize_rowwise(x, "per_row")
    c = N.unpack_nibbles(codes)
    assert S[0] == 0 and S[1] == 0 and np.all(sb[:2] == 0)
    assert c[1, 3] == 0x8 and c[1, 4] == 0
    assert c[2, 0] == 0xF and sb[2, 0] == 0x7E
    # second block amax 1 with S = 2/2688: t = 224 exactly -> s_b = 224, 1.0 -> code 6 (value 4)? no:
    # y = 1 / (224 * 2/2688) = 6  -> code 7
    assert sb[2, 1] == F.encode_e4m3_rne(np.array([224.0]))[0] and c[2, 20] == 0x7


def test_idempotence_rne():
    x = _rand_bf16((128, 256), 3, spread=1.0)
    for q in (lambda v: N.quantize_rowwise(v, "per_row"),
              lambda v: N.quantize_rowwise(v, "per_tensor")):
        c1, s1, S1 = q(x)
        gs = "per_row" if len(S1) == 128 else "per_tensor"
        d1 = N.dequantize_bf16(c1, s1, S1, "1x16", gs)
        c2, s2, S2 = q(F.bf16_bits_to_f64(d1))
        d2 = N.dequantize_bf16(c2, s2, S2, "1x16", gs)
        assert np.array_equal(d1, d2)
        normal = F.E4M3_GRID[s1] >= 2.0 ** -6
        assert np.array_equal(s1[normal], s2[normal])
        cb1 = N.unpack_nibbles(c1).reshape(128, 16, 16)
        cb2 = N.unpack_nibbles(c2).reshape(128, 16, 16)
        assert np.array_equal(cb1[normal], cb2[normal])


def test_tile16_transpose_consistency():
    x = _rand_bf16((64, 96), 4)
    c, s, S = N.quantize_tile16(x)
    ct, st, St = N.quantize_tile16(np.ascontiguousarray(x.T))
    assert St[0] == S[0]
    assert np.array_equal(st, s.T)
    assert np.array_equal(N.unpack_nibbles(ct), N.unpack_nibbles(c).T)


def test_colwise_equals_rowwise_of_transpose_with_tensor_scale():
    x = _rand_bf16((48, 80), 5)
    c, s, S = N.quantize_colwise(x)
    c2, s2, S2 = N.quantize_rowwise(np.ascontiguousarray(x.T), "per_tensor")
    assert S[0] == S2[0] and np.array_equal(c, c2) and np.array_equal(s, s2)


def test_per_token_batch_composition_and_gather_invariance():
    x = _rand_bf16((40, 128), 6)
    c, s, S = N.quantize_rowwise(x, "per_row")
    for r in (0, 13, 39):
        c1, s1, S1 = N.quantize_rowwise(x[r:r + 1], "per_row")
        assert np.array_equal(c1[0], c[r]) and np.array_equal(s1[0], s[r]) and S1[0] == S[r]
    idx = np.array([5, 5, 0, 39, 12, 7])
    cg, sg, Sg = N.quantize_rowwise(x[idx], "per_row")
    assert np.array_equal(cg, c[idx]) and np.array_equal(sg, s[idx]) and np.array_equal(Sg, S[idx])


def test_gate_up_pair_shares_one_scale():
    rs = np.random.default_rng(7)
    gate = F.bf16_bits_to_f64(F.bf16_rne(rs.standard_normal((32, 64)) * 0.02))
    up = F.bf16_bits_to_f64(F.bf16_rne(rs.standard_normal((32, 64)) * 0.05))
    c, s, S = moe.quantize_expert_weights(np.concatenate([gate, up]))
    A = max(np.abs(gate).max(), np.abs(up).max())
    assert S.shape == (1,) and S[0] == np.float32(np.float32(A) / np.float32(2688))
    # the gate half alone, quantized with the pair's S, gives the same bytes
    cg, sg, _ = N.quantize_rowwise(gate, "given", S_given=S[0])
    assert np.array_equal(cg, c[:32]) and np.array_equal(sg, s[:32])


def test_stochastic_rounding_unbiased_over_seeds():
    x = _rand_bf16((4, 64), 8, spread=0.5)
    exact = None
    acc = np.zeros((4, 64))
    n = 2048
    for seed in range(n):
        c, s, S = N.quantize_rowwise(x, "per_row", rnd="sr", seed=seed)
        acc += N.dequantize_f64(c, s, S, "1x16", "per_row")
        if exact is None:
            # the value each element would have with an infinitely fine grid:
            # x * r * (s_b * S) with the same r, s_b and S as the quantizer uses
            cr, sr, Sr = N.quantize_rowwise(x, "per_row")
            sb = np.repeat(F.e4m3_value(sr), 16, axis=1).astype(np.float32)
            den = (sb * np.repeat(Sr.reshape(4, 1), 64, axis=1)).astype(np.float32)
            r = (np.float32(1) / den).astype(np.float32)
            y = (x.astype(np.float32) * r).astype(np.float32).astype(np.float64)
            step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
            unit = sb.astype(np.float64) * np.repeat(Sr.reshape(4, 1), 64, axis=1).astype(np.float64)
            exact = y * unit
            sigma = step * unit / 2 / np.sqrt(n)
    mean = acc / n
    inside = np.abs(y) <= 6.0          # beyond 6 the code saturates by design
    assert inside.mean() > 0.9
    assert np.all((np.abs(mean - exact) <= 5 * sigma + 1e-30)[inside])
    assert np.all(np.abs(mean[~inside]) == 6 * unit[~inside])


def test_stochastic_rounding_properties():
    x = _rand_bf16((16, 128), 9)
    c0, s0, S0 = N.quantize_rowwise(x, "per_row", rnd="sr", seed=0)
    c0b, _, _ = N.quantize_rowwise(x, "per_row", rnd="sr", seed=0)
    c1, s1, S1 = N.quantize_rowwise(x, "per_row", rnd="sr", seed=1)
    cr, sr, Sr = N.quantize_rowwise(x, "per_row")
    assert np.array_equal(c0, c0b) and not np.array_equal(c0, c1)
    assert np.array_equal(s0, sr) and np.array_equal(S0, Sr)     # scales are RNE either way
    v0 = np.abs(F.e2m1_value(N.unpack_nibbles(c0)))
    vr = np.abs(F.e2m1_value(N.unpack_nibbles(cr)))
    g = list(F.E2M1_GRID)
    idx0 = np.vectorize(g.index)(v0)
    idxr = np.vectorize(g.index)(vr)
    assert np.all(np.abs(idx0 - idxr) <= 1)                      # only neighbours
    # values already on the grid never move
    xg = F.e2m1_value(np.arange(16)).reshape(1, 16) * np.ones((2, 1))
    cg, _, _ = N.quantize_rowwise(np.tile(xg, (1, 2)), "given", S_given=np.float32(2.0 ** -8),
                                  rnd="sr", seed=3)
    cr2, _, _ = N.quantize_rowwise(np.tile(xg, (1, 2)), "given", S_given=np.float32(2.0 ** -8))
    assert np.array_equal(cg, cr2)


def test_dequantize_f32_product_is_exact():
    x = _rand_bf16((32, 64), 10)
    c, s, S = N.quantize_rowwise(x, "per_row")
    v = F.e2m1_value(N.unpack_nibbles(c)) * np.repeat(F.e4m3_value(s), 16, axis=1)
    assert np.array_equal(v.astype(np.float32).astype(np.float64), v)   # c * s_b exact in binary32
    d32 = N.dequantize_f32(c, s, S, "1x16", "per_row")
    assert np.array_equal(d32, (v.astype(np.float32) * S.reshape(-1, 1)).astype(np.float32))


# ---------------------------------------------------------------- tiny scales
# For S < 2^-64 the element chain runs in a frame scaled by 2^64 (s_b * S can
# be subnormal there, and its reciprocal would lose bits or overflow).  Pinned
# by what holds without looking at the frame: a power-of-two scaling of the
# whole input moves S and nothing else (the two-level scale absorbs it), the
# dequantized values stay within half an E2M1 step (in units of s_b * S) of x,
# and zeros stay signed zeros.

def _tiny_rows(seed, rows, cols, log2_amax):
    """Rows whose amax is 2^log2_amax[r] and whose nonzero entries lie within
    2^6 of it (so that a further scaling by 2^-60 stays BF16-normal)."""
    rs = np.random.default_rng(seed)
    mant = rs.uniform(1.0, 2.0, (rows, cols)) * rs.choice([-1.0, 1.0], (rows, cols))
    expo = rs.integers(-6, 0, (rows, cols))
    x = mant * np.exp2(expo) * np.exp2(np.asarray(log2_amax, dtype=np.float64))[:, None]
    x[rs.random((rows, cols)) < 0.05] = 0.0
    return F.bf16_bits_to_f64(F.bf16_rne(x))


def test_power_of_two_scaling_moves_only_the_second_scale():
    """Q(x * 2^-60) == Q(x) in codes and block scales, S scaled by 2^-60, for
    rows whose S crosses from above 2^-64 to below it; per-row and per-tensor,
    1x16, 16x1 and 16x16, RNE and SR."""
    x = _tiny_rows(20, 16, 64, np.linspace(-50, -40, 16))
    xs = x * 2.0 ** -60
    assert np.array_equal(F.bf16_bits_to_f64(F.bf16_rne(xs)), xs)       # the scaling is exact
    for rnd in ("rne", "sr"):
        c0, s0, S0 = N.quantize_rowwise(x, "per_row", rnd=rnd, seed=3)
        c1, s1, S1 = N.quantize_rowwise(xs, "per_row", rnd=rnd, seed=3)
        assert np.all(S0 >= N.TINY_S) and np.all(S1 < N.TINY_S)
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert np.array_equal(S1, (S0 * np.float32(2.0 ** -60)).astype(np.float32))
        for q in (N.quantize_colwise, N.quantize_tile16):
            c0, s0, S0 = q(x, "per_tensor", rnd=rnd, seed=3)
            c1, s1, S1 = q(xs, "per_tensor", rnd=rnd, seed=3)
            assert S1[0] < N.TINY_S <= S0[0]
            assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


# largest half gap between an E2M1 magnitude and its grid neighbours
_HALF_GAP = {0.0: 0.25, 0.5: 0.25, 1.0: 0.25, 1.5: 0.25, 2.0: 0.5, 3.0: 0.5, 4.0: 1.0, 6.0: 1.0}


def test_tiny_rows_dequantize_within_half_a_step():
    """Rows with amax from about 2^-113 (S still a binary32 normal) to 2^-64 and
    blocks down to 2^-24 below their row's amax (so that s_b * S is
    subnormal): |DQ(Q(x)) - x| <= s_b S (half gap + 2^-18) element by element
    wherever |x| <= 7 s_b S (RNE onto the grid), code 6 beyond (saturation),
    zeros encode as signed zeros, and some blocks do take the scaled frame
    with a subnormal s_b * S."""
    rs = np.random.default_rng(21)
    rows, cols = 32, 128
    amax = np.linspace(-112, -65, rows)
    x = _tiny_rows(22, rows, cols, amax)
    # spread the blocks of each row over 24 binades below the row's amax
    shrink = np.exp2(-rs.integers(0, 24, (rows, cols // 16))).repeat(16, axis=1)
    shrink[:, 0] = 1.0
    x = F.bf16_bits_to_f64(F.bf16_rne(x * shrink))
    x[:, 5] = -0.0
    codes, sb, S = N.quantize_rowwise(x, "per_row")
    assert np.all((S > 0) & (S < N.TINY_S)) and np.all(S >= np.float32(2.0 ** -126))
    den = F.e4m3_value(sb).astype(np.float32) * np.repeat(S[:, None], cols // 16, axis=1)
    assert np.any((den > 0) & (den < np.float32(2.0 ** -126)))               # subnormal s_b * S occurs
    c = N.unpack_nibbles(codes)
    v = F.e2m1_value(c)
    unit = np.repeat(F.e4m3_value(sb), 16, axis=1) * S[:, None].astype(np.float64)
    dq = N.dequantize_f64(codes, sb, S, "1x16", "per_row")
    gap = np.vectorize(lambda a: _HALF_GAP[abs(a)])(v)
    live = np.repeat(sb != 0, 16, axis=1)
    assert live.mean() > 0.5
    # past 7 steps the code saturates at 6; that happens only under an E4M3
    # subnormal block scale, whose rounding can leave a_b / (s_b S) well above 6
    over = live & (np.abs(x) > 7.0 * unit)
    assert np.all(np.abs(v[over]) == 6.0) and np.all(np.signbit(v[over]) == np.signbit(x[over]))
    assert np.all(np.repeat(F.e4m3_value(sb), 16, axis=1)[over] < 2.0 ** -6)
    ok = live & ~over
    assert np.all(np.abs(dq - x)[ok] <= (unit * (gap + 2.0 ** -18))[ok])
    # a block whose scale rounds to zero has t = a_b / (6 S) <= 2^-10
    Sx = np.repeat(S[:, None].astype(np.float64), cols, axis=1)
    assert np.all(np.abs(x[~live]) <= 6.0 * Sx[~live] * 2.0 ** -10 * (1 + 2.0 ** -20))
    zero = x == 0
    assert np.array_equal(c[zero] & 7, np.zeros(zero.sum(), dtype=c.dtype))
    assert np.array_equal((c[zero] >> 3) & 1, np.signbit(x[zero]).astype(c.dtype))


def test_smallest_row_of_the_advisor_case():
    """The row [2^-126, 2^-128, 0 x 14]: S = fl(2^-126 / 2688) is subnormal
    and s_b * S = 448 S is below 2^-128, so an unscaled reciprocal is
    infinite.  The block max encodes as 6 under s_b = 448, 2^-128 as 1.5, and
    the zeros as zeros."""
    x = np.zeros((1, 16))
    x[0, 0], x[0, 1] = 2.0 ** -126, 2.0 ** -128
    codes, sb, S = N.quantize_rowwise(x, "per_row")
    assert S[0] < np.float32(2.0 ** -126)                                   # subnormal
    assert int(sb[0, 0]) == 0x7E
    c = N.unpack_nibbles(codes)[0]
    assert c[0] == 7 and c[1] == 3 and np.all(c[2:] == 0)
