"""MXFP8 quantize / dequantize, step by step.

MXFP8 stores blocks of 32 E4M3 values that share one E8M0 (power-of-two)
scale ("Miles Blackwell RL ...", section on the full RL loop).  The blocks
follow the GEMM's reduction dimension, so forward and backward need differently
oriented copies, each made from the high-precision original ("Miles Blackwell
RL ...", section "Um Quantizador Compartilhado É o Verdadeiro Mecanismo").
A 32x32 tile variant serves weights read both ways.

Scale rule (a reading; the pages give none): the block exponent e is the
smallest integer in [-127, 127] with amax <= 448 * 2^e, so no element of the
block exceeds the E4M3 range after scaling; an all-zero block gets e = -127
(E8M0 code 0x00).  Element code = RNE E4M3 of x * 2^-e, which is exact
scaling, so the only rounding is the E4M3 one.

Array conventions: x is float64 holding BF16 values, shape [rows, cols].
Rowwise (1x32) blocks run along cols; codes [rows, cols] uint8, scales
[rows, cols/32] uint8.  Columnwise (32x1) blocks run along rows and the copy is
stored transposed: codes [cols, rows], scales [cols, rows/32].  32x32 tiles:
codes [rows, cols], scales [rows/32, cols/32].

Test infrastructure only (see the package docstring).
"""

import numpy as np

from .formats import encode_e4m3_rne, e4m3_value, bf16_rne, E4M3_MAX

BLOCK = 32


def block_exponent(amax):
    """Smallest e in [-127, 127] with amax <= 448 * 2^e (amax = 0 -> -127)."""
    a = np.asarray(amax, dtype=np.float64)
    safe = np.where(a > 0, a, 1.0)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # exact corrections: the comparisons below are exact in float64
    for _ in range(3):
        e = np.where(a > E4M3_MAX * np.exp2(e.astype(np.float64)), e + 1, e)
        e = np.where(a <= E4M3_MAX * np.exp2((e - 1).astype(np.float64)), e - 1, e)
    e = np.clip(e, -127, 127)
    return np.where(a > 0, e, -127).astype(np.int64)


def _quantize_blocks(xb):
    """xb: [..., nblocks, 32] float64 -> (codes same shape, e8m0 [..., nblocks])."""
    amax = np.max(np.abs(xb), axis=-1)
    e = block_exponent(amax)
    scaled = xb * np.exp2(-e.astype(np.float64))[..., None]
    assert np.all(np.abs(scaled) <= E4M3_MAX), "MXFP8 block overflow"
    codes = encode_e4m3_rne(scaled)
    return codes, (e + 127).astype(np.uint8)


def quantize_rowwise(x):
    """1x32 blocks along the last (contiguous) dim."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert cols % BLOCK == 0
    codes, sc = _quantize_blocks(x.reshape(rows, cols // BLOCK, BLOCK))
    return codes.reshape(rows, cols), sc


def quantize_colwise(x):
    """32x1 blocks along rows; the copy is stored transposed ([cols, rows])."""
    x = np.asarray(x, dtype=np.float64)
    return quantize_rowwise(np.ascontiguousarray(x.T))


def quantize_tile32(x):
    """One E8M0 scale per 32x32 tile."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % BLOCK == 0 and cols % BLOCK == 0
    t = x.reshape(rows // BLOCK, BLOCK, cols // BLOCK, BLOCK).transpose(0, 2, 1, 3)
    t = t.reshape(rows // BLOCK, cols // BLOCK, BLOCK * BLOCK)
    codes, sc = _quantize_blocks(t)
    codes = codes.reshape(rows // BLOCK, cols // BLOCK, BLOCK, BLOCK).transpose(0, 2, 1, 3)
    return codes.reshape(rows, cols), sc


def scale_per_element(scales, shape, block):
    """Broadcast the E8M0 exponent grid to every element of a [rows, cols] copy."""
    rows, cols = shape
    e = scales.astype(np.int64) - 127
    if block == "1x32":
        return np.repeat(e, BLOCK, axis=1)
    if block == "32x32":
        return np.repeat(np.repeat(e, BLOCK, axis=0), BLOCK, axis=1)
    raise ValueError(block)


def dequantize_f64(codes, scales, block="1x32"):
    """Exact value c * 2^e of every element (float64)."""
    e = scale_per_element(scales, codes.shape, block)
    return e4m3_value(codes) * np.exp2(e.astype(np.float64))


def dequantize_bf16(codes, scales, block="1x32"):
    """DQ(Q(x)) as BF16 bits: RNE of the exact value (exact unless it falls
    below the BF16 subnormal range or beyond its largest finite value)."""
    return bf16_rne(dequantize_f64(codes, scales, block))
