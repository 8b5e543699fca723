"""Element and scale formats, from their closed-form definitions.

The pages only name the formats (MXFP8: E4M3 elements, E8M0 scale; NVFP4: E2M1
elements, E4M3 block scale, FP32 second scale -- "Miles Blackwell RL ...",
section on the two recipes; "Train models faster ... NVFP4", section "NVFP4
format and benefits").  The value grids below are the formats' public
definitions:

* E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities):
  exponent field 0 -> m * 2^-9, otherwise (1 + m/8) * 2^(e-7); 0x7F/0xFF NaN;
  largest finite 448.
* E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN):
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E8M0 (8 exponent bits, bias 127, no sign, no mantissa): 2^(c-127) for
  c = 0..254, 255 = NaN.  The "End-to-End MXFP8 RL on Blackwell" paper, Table 10
  F6, notes that such a scale keeps only the exponent.

Test infrastructure only (see the package docstring).
"""

import numpy as np


# ---------------------------------------------------------------- decoders

def e4m3_value(code):
    """Value of E4M3 code(s) as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e2m1_value(code):
    """Value of E2M1 code(s) (4-bit, sign in bit 3) as float64."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e8m0_value(code):
    """Value of E8M0 code(s) as float64 (NaN for 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


# Magnitude grids, indexed by the magnitude code (codes are monotone in value).
E4M3_GRID = e4m3_value(np.arange(0x7F))     # 0x00 .. 0x7E, 0 .. 448
E2M1_GRID = e2m1_value(np.arange(8))        # 0 .. 6
E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ---------------------------------------------------------------- encoders

def rne_sat_index(mag, grid):
    """Index of the grid point nearest to each non-negative `mag`.

    Ties go to the even index (the code whose last bit is 0); values above the
    largest grid point saturate to it.  Exact in float64: every grid point and
    every midpoint between neighbours is a float64 number.
    """
    a = np.asarray(mag, dtype=np.float64)
    n = len(grid)
    hi = np.searchsorted(grid, a, side="left")          # first grid point >= a
    hi = np.clip(hi, 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= grid[-1], n - 1, idx)
    idx = np.where(a <= 0.0, 0, idx)
    return idx.astype(np.int64)


def encode_e4m3_rne(v):
    """Round-to-nearest-even, saturating E4M3 encode; sign bit = input sign bit."""
    v = np.asarray(v, dtype=np.float64)
    idx = rne_sat_index(np.abs(v), E4M3_GRID)
    return (idx | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def encode_e2m1_rne(v):
    """Round-to-nearest-even, saturating E2M1 encode (4-bit code, sign in bit 3)."""
    v = np.asarray(v, dtype=np.float64)
    idx = rne_sat_index(np.abs(v), E2M1_GRID)
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def encode_e2m1_sr(v, r16):
    """Stochastic-rounding E2M1 encode.

    The NVFP4 recipe rounds gradients stochastically so that small updates are
    not lost on average ("Train models faster ... NVFP4", section "NVFP4
    pretraining recipe"; "NVFP4 RL training", baseline-recipe section).
    With lo <= |v| < hi the neighbouring grid magnitudes and
    f = (|v| - lo) / (hi - lo), the magnitude rounds up iff u < f, where
    u = r16 * 2^-16 and r16 is the element's 16-bit random draw.  |v| >= 6
    gives 6.  The sign is the input's sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    r16 = np.asarray(r16, dtype=np.int64)
    a = np.abs(v)
    g = E2M1_GRID
    hi = np.clip(np.searchsorted(g, a, side="right"), 1, len(g) - 1)  # first grid > a
    lo = hi - 1
    f = (a - g[lo]) / (g[hi] - g[lo])
    u = r16 * 2.0 ** -16
    idx = np.where(u < f, hi, lo)
    idx = np.where(a >= E2M1_MAX, len(g) - 1, idx)
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


# ---------------------------------------------------------------- bfloat16

def bf16_bits_to_f64(bits):
    """BF16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_rne(v):
    """Round real values (given exactly as float64) to BF16, nearest-even.

    BF16 keeps 8 significant bits and the binary32 exponent range; the
    subnormal quantum is 2^-133.  Results beyond the largest finite BF16 round
    to infinity, as IEEE round-to-nearest requires.  Returns uint16 bits.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    qexp = np.maximum(ex - 8, -133)           # quantum exponent
    q = np.rint(np.ldexp(a, -qexp))           # rint is round-half-even
    r = np.ldexp(q, qexp)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(r > bf16_max, np.inf, r)
    r = np.where(np.isnan(a), np.nan, r)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sign = (np.signbit(v).astype(np.uint16) << 15)
    return (bits | sign).astype(np.uint16)


def f32(x):
    """Binary32 view of a value (exact when x is representable)."""
    return np.asarray(x, dtype=np.float32)
