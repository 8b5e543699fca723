"""DeepSeek-style blockwise FP8 with power-of-two scales.

"NVIDIA NeMo RL agora roda treino ... FP8 ponta a ponta" (cafecomtech.com),
section "FP8 nas camadas lineares": the blockwise FP8 recipe quantizes to E4M3
with one scale per [128, 128] weight block and per [1, 128] block of input
activations and of output gradients, the block layout of the DeepSeek-V3
report; "Miles Blackwell RL ..." (remio.ai) describes the same 128x128 /
1x128 design as the Hopper-era FP8 path.  "End-to-End MXFP8 Reinforcement
Learning on Blackwell", Table 1, pairs a learner restricted to power-of-two
scales on Blackwell with a sampler using FP32 scales.

Readings:

1. Scales are powers of two (the scaled MFMA takes E8M0 exponents, as
   Blackwell's blockwise path takes power-of-two scales): the block exponent
   is the MXFP8 rule over the 128 (or 128x128) values of the block -- the
   smallest e in [-127, 127] with amax <= 448 * 2^e, e = -127 for a zero
   block -- stored as an E8M0 byte.  Codes are RNE E4M3 of x * 2^-e.
2. Layouts: 1x128 blocks along the contiguous dimension, codes [rows, cols]
   and scales [rows, cols/128]; the columnwise copy (WGRAD's token-major
   operands) is stored transposed, [cols, rows] with scales [cols, rows/128];
   128x128 tiles: codes [rows, cols], scales [rows/128, cols/128].  A tile's
   scale serves its rows and its columns, so the tile copy of x^T is the same
   codes transposed.
3. FP32 block scales (the other arm of that table, and the DeepSeek-V3
   recipe itself): s = amax / 448 rounded to binary32, codes RNE E4M3 of
   x / s (binary32 division, correctly rounded, clamped to +-448 since the
   rounded quotient of the block maximum may exceed 448 by an ulp).  A zero
   block stores s = 0 and zero codes.  Dequantization is value(c) * s
   (exact in float64; BF16 copies round the binary32 product, as the
   kernels compute it).  A GEMM on such operands is the dequantize-then-
   matmul definition; its kernel scales each 128-wide K block's partial sums
   by s_a * s_b outside the MFMA.

Test infrastructure only (see the package docstring).
"""

import numpy as np

from .formats import encode_e4m3_rne, e4m3_value, bf16_rne, E4M3_MAX
from .mxfp8 import block_exponent

BLOCK = 128


def _quantize_blocks(xb):
    """xb [..., n] float64 -> (codes same shape, E8M0 bytes [...])."""
    amax = np.max(np.abs(xb), axis=-1)
    e = block_exponent(amax)
    scaled = xb * np.exp2(-e.astype(np.float64))[..., None]
    assert np.all(np.abs(scaled) <= E4M3_MAX)
    return encode_e4m3_rne(scaled), (e + 127).astype(np.uint8)


def quantize_rows(x):
    """1x128 blocks along cols."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert cols % BLOCK == 0
    codes, sc = _quantize_blocks(x.reshape(rows, cols // BLOCK, BLOCK))
    return codes.reshape(rows, cols), sc


def quantize_cols(x):
    """128x1 blocks along rows, the copy stored transposed ([cols, rows])."""
    return quantize_rows(np.ascontiguousarray(np.asarray(x, dtype=np.float64).T))


def quantize_tile(x):
    """One scale per 128x128 tile."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % BLOCK == 0 and cols % BLOCK == 0
    t = x.reshape(rows // BLOCK, BLOCK, cols // BLOCK, BLOCK).transpose(0, 2, 1, 3)
    codes, sc = _quantize_blocks(t.reshape(rows // BLOCK, cols // BLOCK, BLOCK * BLOCK))
    codes = codes.reshape(rows // BLOCK, cols // BLOCK, BLOCK, BLOCK).transpose(0, 2, 1, 3)
    return codes.reshape(rows, cols), sc


def scale_per_element(scales, shape, block):
    e = scales.astype(np.int64) - 127
    if block == "1x128":
        return np.repeat(e, BLOCK, axis=1)
    if block == "128x128":
        return np.repeat(np.repeat(e, BLOCK, axis=0), BLOCK, axis=1)
    raise ValueError(block)


def dequantize_f64(codes, scales, block="1x128"):
    """Exact value c * 2^e of every element."""
    e = scale_per_element(scales, codes.shape, block)
    return e4m3_value(codes) * np.exp2(e.astype(np.float64))


def dequantize_bf16(codes, scales, block="1x128"):
    return bf16_rne(dequantize_f64(codes, scales, block))


# ------------------------------------------------------------ FP32 scales

def _quantize_blocks_f32(xb):
    """xb [..., n] float64 (BF16 values) -> (codes, binary32 scales [...])."""
    amax = np.max(np.abs(xb), axis=-1).astype(np.float32)        # exact: BF16 values
    s = amax / np.float32(E4M3_MAX)                                 # binary32, rounded once
    safe = np.where(s == 0, np.float32(1), s)
    q = xb.astype(np.float32) / safe[..., None]                     # binary32 quotient
    q = np.clip(q, -np.float32(E4M3_MAX), np.float32(E4M3_MAX))
    q = np.where((s == 0)[..., None], np.float32(0), q)
    return encode_e4m3_rne(q.astype(np.float64)), s.astype(np.float32)


def quantize_rows_f32(x):
    """1x128 blocks along cols, binary32 scales [rows, cols/128]."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert cols % BLOCK == 0
    codes, sc = _quantize_blocks_f32(x.reshape(rows, cols // BLOCK, BLOCK))
    return codes.reshape(rows, cols), sc


def quantize_cols_f32(x):
    """128x1 blocks along rows, the copy stored transposed ([cols, rows])."""
    return quantize_rows_f32(np.ascontiguousarray(np.asarray(x, dtype=np.float64).T))


def quantize_tile_f32(x):
    """One binary32 scale per 128x128 tile, [rows/128, cols/128]."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % BLOCK == 0 and cols % BLOCK == 0
    t = x.reshape(rows // BLOCK, BLOCK, cols // BLOCK, BLOCK).transpose(0, 2, 1, 3)
    codes, sc = _quantize_blocks_f32(t.reshape(rows // BLOCK, cols // BLOCK, BLOCK * BLOCK))
    codes = codes.reshape(rows // BLOCK, cols // BLOCK, BLOCK, BLOCK).transpose(0, 2, 1, 3)
    return codes.reshape(rows, cols), sc


def scale_f32_per_element(scales, block):
    s = np.asarray(scales, dtype=np.float64)
    if block == "1x128":
        return np.repeat(s, BLOCK, axis=1)
    if block == "128x128":
        return np.repeat(np.repeat(s, BLOCK, axis=0), BLOCK, axis=1)
    raise ValueError(block)


def dequantize_f32s_f64(codes, scales, block="1x128"):
    """Exact value(c) * s of every element."""
    return e4m3_value(codes) * scale_f32_per_element(scales, block)


def dequantize_f32s_bf16(codes, scales, block="1x128"):
    """BF16 copy: the binary32 product value(c) * s, rounded to BF16."""
    p = (e4m3_value(codes).astype(np.float32) * scale_f32_per_element(scales, block).astype(np.float32))
    return bf16_rne(p.astype(np.float64))
