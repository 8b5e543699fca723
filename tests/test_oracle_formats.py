"""Pins of the oracle's format code (oracle/formats.py) against things other
than itself: PyTorch's float8 dtypes (a library routine), a threshold-table
formulation of E2M1 rounding, exhaustive enumeration of SR draws, and
PyTorch's float32 -> bfloat16 conversion."""

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert F.E4M3_GRID[-1] == 448.0 and len(F.E4M3_GRID) == 127


def test_e8m0_decode_matches_torch_float8_e8m0fnu():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e8m0_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e2m1_grid_matches_published_value_table():
    # The E2M1 value set written out as a table (not the exponent/mantissa formula).
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.E2M1_GRID) == table
    neg = F.e2m1_value(np.arange(8, 16))
    assert list(-neg) == table and np.all(np.signbit(neg))


def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


def _e4m3_probe_values():
    rs = np.random.default_rng(0)
    bf = _all_bf16_finite().astype(np.float64)
    grid = F.E4M3_GRID
    mids = (grid[1:] + grid[:-1]) / 2
    near = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float64)
    rnd = rs.uniform(0, 464, 200000).astype(np.float32).astype(np.float64)
    tiny = rs.uniform(0, 2.0 ** -6, 50000).astype(np.float32).astype(np.float64)
    v = np.concatenate([bf, near, -near, rnd, -rnd, tiny, -tiny, [0.0, -0.0]])
    return v[np.abs(v) < 464.0]          # torch turns >= 464 into NaN instead of saturating


def test_e4m3_rne_encode_matches_torch():
    v = _e4m3_probe_values()
    ours = F.encode_e4m3_rne(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_above_max():
    v = np.array([464.0, 500.0, 1e30, -1e30, 448.0])
    assert list(F.encode_e4m3_rne(v)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]


def _e2m1_by_thresholds(a):
    """E2M1 RNE written as the decision table of the grid's midpoints, with
    the tie at each midpoint going to the even code."""
    a = np.abs(a)
    out = np.zeros(a.shape, dtype=np.int64)
    out = np.where((a > 0.25) & (a < 0.75), 1, out)
    out = np.where((a >= 0.75) & (a <= 1.25), 2, out)
    out = np.where((a > 1.25) & (a < 1.75), 3, out)
    out = np.where((a >= 1.75) & (a <= 2.5), 4, out)
    out = np.where((a > 2.5) & (a < 3.5), 5, out)
    out = np.where((a >= 3.5) & (a <= 5.0), 6, out)
    out = np.where(a > 5.0, 7, out)
    return out


def test_e2m1_rne_encode_matches_threshold_table():
    rs = np.random.default_rng(1)
    bf = _all_bf16_finite().astype(np.float64)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9))])
    rnd = rs.uniform(0, 8, 500000).astype(np.float32)
    v = np.concatenate([bf, near.astype(np.float64), rnd.astype(np.float64)])
    v = np.concatenate([v, -v])
    codes = F.encode_e2m1_rne(v)
    assert np.array_equal(codes & 7, _e2m1_by_thresholds(v))
    assert np.array_equal((codes >> 3) & 1, np.signbit(v).astype(np.uint8))


def test_e2m1_rne_is_nearest_with_even_ties_bruteforce():
    rs = np.random.default_rng(2)
    v = rs.uniform(0, 6, 20000)
    idx = F.encode_e2m1_rne(v) & 7
    d = np.abs(v[:, None] - F.E2M1_GRID[None, :])
    best = d.min(axis=1)
    assert np.allclose(d[np.arange(len(v)), idx], best, rtol=0, atol=0)


@pytest.mark.parametrize("y", [0.0, 0.1, 0.25, 0.3, 0.5, 0.6, 1.0, 1.1, 1.2, 1.75, 2.2, 2.75,
                               3.0, 3.9, 4.0, 4.5, 5.5, 5.999, 6.0, 6.3])
def test_e2m1_sr_exact_expectation_over_all_draws(y):
    r16 = np.arange(65536)
    for s in (1.0, -1.0):
        v = np.full(65536, s * y)
        codes = F.encode_e2m1_sr(v, r16)
        vals = F.e2m1_value(codes)
        a = min(abs(y), 6.0)
        g = F.E2M1_GRID
        hi = min(np.searchsorted(g, a, side="right"), 7)
        lo = hi - 1
        # only the two neighbours occur
        assert set(np.abs(vals)) <= {g[lo], g[hi]}
        f = (a - g[lo]) / (g[hi] - g[lo]) if a < 6.0 else 0.0
        # the number of draws that round up is ceil(f * 2^16): the rule "up iff u < f"
        n_up = int(np.sum(np.abs(vals) == g[hi])) if a < 6.0 else 0
        assert n_up == int(np.ceil(f * 65536))
        if (f * 65536) == int(f * 65536):
            assert np.mean(vals) == s * a          # exactly unbiased on the 2^-16 grid
        assert np.all(np.signbit(vals) == (s < 0))


def test_bf16_rne_matches_torch_on_float32_inputs():
    rs = np.random.default_rng(3)
    bits = rs.integers(0, 2 ** 32, 400000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    ties = ((np.arange(0, 65536, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    v = np.concatenate([v, ties, np.array([0.0, -0.0], dtype=np.float32)])
    ours = F.bf16_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_rounds_float64_once():
    # a float64 value just above a BF16 midpoint must round up, even though
    # rounding it to float32 first would land exactly on the midpoint.
    mid = 1.0 + 2.0 ** -8
    v = np.array([mid + 2.0 ** -40, mid, mid - 2.0 ** -40])
    out = F.bf16_rne(v)
    assert list(out) == [0x3F81, 0x3F80, 0x3F80]


def test_float32_ops_are_correctly_rounded():
    """The NVFP4 scale chain relies on numpy binary32 ops being IEEE
    correctly rounded: check division and multiplication against exact
    rational arithmetic."""
    from fractions import Fraction
    rs = np.random.default_rng(4)
    a = rs.uniform(1e-30, 1e30, 3000).astype(np.float32)
    b = rs.uniform(1e-3, 1e3, 3000).astype(np.float32)
    q = (a / b).astype(np.float32)
    p = (a * b).astype(np.float32)
    for i in range(len(a)):
        for got, exact in ((q[i], Fraction(float(a[i])) / Fraction(float(b[i]))),
                           (p[i], Fraction(float(a[i])) * Fraction(float(b[i])))):
            g = Fraction(float(got))
            lo = Fraction(float(np.nextafter(got, np.float32(-np.inf))))
            hi = Fraction(float(np.nextafter(got, np.float32(np.inf))))
            assert abs(g - exact) <= abs(lo - exact) and abs(g - exact) <= abs(hi - exact)
