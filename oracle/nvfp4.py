"""NVFP4 quantize / dequantize, step by step in binary32.

NVFP4 stores blocks of 16 E2M1 values, each block with an E4M3 scale, under a
second FP32 scale ("Miles Blackwell RL ...", section on the full RL loop;
"Train models faster ... NVFP4", section "NVFP4 pretraining recipe").  Miles
computes the second scale per token, online from the activation, so that a
token's codes do not depend on its batch neighbours ("Miles Blackwell RL ...",
section "Um Quantizador Compartilhado É o Verdadeiro Mecanismo"; "NVFP4 RL
training", baseline-recipe section).  NVIDIA's pretraining recipe uses a
per-tensor second scale, 16x16 blocks for weights (FPROP and its transposed
DGRAD share the scales) and 1x16 blocks for activations and gradients, with
RNE for weights/activations and stochastic rounding for gradients.

Readings taken where the pages are silent (listed in the design notes):

1. S = fl(A / 2688) with 2688 = 6 * 448; A = max|x| over the token (row) or
   the whole tensor; A = 0 gives S = 0.  S is a decode multiplier.
2. Per block: a_b = max|x| over the block; t = fl(a_b / fl(6 * S));
   s_b = RNE-saturating E4M3 of t (s_b = 0 when S = 0).
3. If s_b = 0 the block's codes are signed zeros.  Otherwise
   r = fl(1 / fl(s_b * S)), y = fl(x * r), code = RNE (or SR) E2M1 of y,
   saturating at 6.  For S < 2^-64 the same steps run in a frame scaled by
   2^64 (x and S times 2^64, both exact), which keeps s_b * S a binary32
   normal for every finite BF16 input; see encode_block_elements.
4. Packing: element 2j in the low nibble, 2j+1 in the high nibble.
5. SR draws come from Philox4x32-10 (see philox.py), 16 bits per element,
   counter from the element's index in the logical input.

Every fl(.) is one binary32 IEEE operation, round-to-nearest-even, subnormals
kept, no fused multiply-add (numpy float32 arithmetic is exactly this).

Array conventions: x float64 holding BF16 values, [rows, cols].  Rowwise 1x16
blocks run along cols: packed codes [rows, cols/2] uint8, block scales
[rows, cols/16] uint8 (E4M3 codes), S per row [rows] or per tensor [1] float32.
Columnwise 16x1 blocks run along rows, the copy stored transposed ([cols, rows]
codes packed along rows); S per tensor.  16x16 tiles: codes [rows, cols/2],
scales [rows/16, cols/16], S per tensor.

Test infrastructure only (see the package docstring).
"""

import numpy as np

from .formats import (encode_e4m3_rne, encode_e2m1_rne, encode_e2m1_sr,
                      e4m3_value, e2m1_value, bf16_rne)
from .philox import element_r16

BLOCK = 16
F32 = np.float32


def second_scale(amax):
    """S = fl(A / 2688) in binary32 (A = 0 gives 0)."""
    return (F32(amax) / F32(2688.0)).astype(F32)


def block_scale(a_b, S):
    """E4M3 block-scale code from the block amax and the second scale S."""
    a_b = np.asarray(a_b, dtype=F32)
    S = np.asarray(S, dtype=F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        six_s = (F32(6.0) * S).astype(F32)
        t = (a_b / six_s).astype(F32)
    t = np.where(S > 0, t, F32(0.0))
    return encode_e4m3_rne(t.astype(np.float64))


TINY_S = np.float32(2.0 ** -64)        # below it, the reciprocal is taken in a scaled frame
FRAME = np.float32(2.0 ** 64)


def encode_block_elements(x, sb_code, S, rnd="rne", r16=None):
    """Element codes of blocks: x [..., 16] float64, sb_code/S broadcast [..., 1].

    y = fl(x * fl(1 / fl(s_b * S))), then RNE (or SR) onto E2M1.  When S is
    below 2^-64 the product s_b * S can fall below binary32's normal range (its
    reciprocal then loses bits or overflows to infinity, and 0 * inf would be
    NaN), so the chain is taken in a frame scaled by the exact power of two
    2^64: y = fl(fl(x * 2^64) * fl(1 / fl(s_b * fl(S * 2^64)))).  Wherever
    s_b * S is a binary32 normal both forms give the same y (every scaling by
    2^64 is exact there), so this only changes blocks whose s_b * S is
    subnormal.  (x * 2^64 exceeds the binary32 range only for |x| >= 2^64
    under a caller-given S < 2^-64; the infinite y then saturates at 6, as
    the exact quotient would.)"""
    sb = e4m3_value(sb_code).astype(F32)
    S = np.asarray(S, dtype=F32)
    frame = np.where(S < TINY_S, FRAME, F32(1.0)).astype(F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        xf = (x.astype(F32) * frame).astype(F32)
        Sf = (S * frame).astype(F32)
        denom = (sb * Sf).astype(F32)
        r = (F32(1.0) / denom).astype(F32)
        y = (xf * r).astype(F32)
    zero_block = (sb == 0) | (S == 0)
    y = np.where(zero_block, np.copysign(F32(0.0), x.astype(F32)), y)
    if rnd == "rne":
        return encode_e2m1_rne(y.astype(np.float64))
    if rnd == "sr":
        return encode_e2m1_sr(y.astype(np.float64), r16)
    raise ValueError(rnd)


def pack_nibbles(codes):
    """[..., 2n] 4-bit codes -> [..., n] bytes, even index in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _rows_1x16(x, S_rows, rnd, r16):
    """Quantize each row of x (1x16 blocks) with per-row second scales S_rows."""
    rows, cols = x.shape
    assert cols % BLOCK == 0
    xb = x.reshape(rows, cols // BLOCK, BLOCK)
    a_b = np.max(np.abs(xb), axis=-1)
    S_b = np.broadcast_to(np.asarray(S_rows, dtype=F32).reshape(-1, 1), a_b.shape)
    sb = block_scale(a_b, S_b)
    rb = None if r16 is None else r16.reshape(rows, cols // BLOCK, BLOCK)
    codes = encode_block_elements(xb, sb[..., None], S_b[..., None], rnd, rb)
    return pack_nibbles(codes.reshape(rows, cols)), sb


def _r16_for(shape, rnd, seed, stream_id, tensor_tag, transposed=False):
    if rnd != "sr":
        return None
    rows, cols = shape                      # shape of the logical input
    r, c = np.meshgrid(np.arange(rows, dtype=np.int64),
                       np.arange(cols, dtype=np.int64), indexing="ij")
    r16 = element_r16(r * cols + c, seed, stream_id, tensor_tag)
    return np.ascontiguousarray(r16.T) if transposed else r16


def quantize_rowwise(x, gscale="per_row", rnd="rne", seed=0, stream_id=0,
                     tensor_tag=0, S_given=None):
    """1x16 blocks along cols.  Returns (packed codes, block scales, S)."""
    x = np.asarray(x, dtype=np.float64)
    if gscale == "per_row":
        S = second_scale(np.max(np.abs(x), axis=1))
        S_rows = S
    elif gscale == "per_tensor":
        S = second_scale(np.max(np.abs(x))).reshape(1)
        S_rows = np.full(x.shape[0], S[0], dtype=F32)
    elif gscale == "given":
        S = np.asarray(S_given, dtype=F32).reshape(1)
        S_rows = np.full(x.shape[0], S[0], dtype=F32)
    else:
        raise ValueError(gscale)
    r16 = _r16_for(x.shape, rnd, seed, stream_id, tensor_tag)
    codes, sb = _rows_1x16(x, S_rows, rnd, r16)
    return codes, sb, S


def quantize_colwise(x, gscale="per_tensor", rnd="rne", seed=0, stream_id=1,
                     tensor_tag=0, S_given=None):
    """16x1 blocks along rows, stored transposed; second scale per tensor.
    Random draws keep the element's index in the logical (untransposed) input."""
    x = np.asarray(x, dtype=np.float64)
    if gscale == "per_tensor":
        S = second_scale(np.max(np.abs(x))).reshape(1)
    elif gscale == "given":
        S = np.asarray(S_given, dtype=F32).reshape(1)
    else:
        raise ValueError("a columnwise copy takes a per-tensor second scale")
    xt = np.ascontiguousarray(x.T)
    r16 = _r16_for(x.shape, rnd, seed, stream_id, tensor_tag, transposed=True)
    codes, sb = _rows_1x16(xt, np.full(xt.shape[0], S[0], dtype=F32), rnd, r16)
    return codes, sb, S


def quantize_tile16(x, gscale="per_tensor", rnd="rne", seed=0, stream_id=0,
                    tensor_tag=0, S_given=None):
    """One E4M3 scale per 16x16 tile, second scale per tensor."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % BLOCK == 0 and cols % BLOCK == 0
    if gscale == "per_tensor":
        S = second_scale(np.max(np.abs(x))).reshape(1)
    elif gscale == "given":
        S = np.asarray(S_given, dtype=F32).reshape(1)
    else:
        raise ValueError("16x16 tiles take a per-tensor second scale")
    t = x.reshape(rows // BLOCK, BLOCK, cols // BLOCK, BLOCK)
    a_b = np.max(np.abs(t), axis=(1, 3))                       # [R, C]
    sb = block_scale(a_b, np.full(a_b.shape, S[0], dtype=F32))
    sb_el = np.repeat(np.repeat(sb, BLOCK, axis=0), BLOCK, axis=1)
    r16 = _r16_for(x.shape, rnd, seed, stream_id, tensor_tag)
    codes = encode_block_elements(x, sb_el, np.full(x.shape, S[0], dtype=F32), rnd, r16)
    return pack_nibbles(codes), sb, S


def scale_per_element(block_scales, S, shape, block, gscale):
    """Broadcast (s_b as float32, S as float32) to every element of the stored copy."""
    rows, cols = shape
    sb = e4m3_value(block_scales).astype(F32)
    if block in ("1x16",):
        sb_el = np.repeat(sb, BLOCK, axis=1)
    elif block == "16x16":
        sb_el = np.repeat(np.repeat(sb, BLOCK, axis=0), BLOCK, axis=1)
    else:
        raise ValueError(block)
    S = np.asarray(S, dtype=F32)
    if gscale == "per_row":
        S_el = np.broadcast_to(S.reshape(rows, 1), shape)
    else:
        S_el = np.full(shape, S.reshape(-1)[0], dtype=F32)
    return sb_el, S_el


def dequantize_f64(packed, block_scales, S, block="1x16", gscale="per_row"):
    """Exact value c * s_b * S of every element (float64)."""
    codes = unpack_nibbles(packed)
    sb_el, S_el = scale_per_element(block_scales, S, codes.shape, block, gscale)
    return e2m1_value(codes) * sb_el.astype(np.float64) * S_el.astype(np.float64)


def dequantize_f32(packed, block_scales, S, block="1x16", gscale="per_row"):
    """fl(fl(c * s_b) * S) in binary32 (c * s_b is exact)."""
    codes = unpack_nibbles(packed)
    sb_el, S_el = scale_per_element(block_scales, S, codes.shape, block, gscale)
    v = (e2m1_value(codes).astype(F32) * sb_el).astype(F32)
    return (v * S_el).astype(F32)


def dequantize_bf16(packed, block_scales, S, block="1x16", gscale="per_row"):
    """DQ(Q(x)) as BF16 bits: BF16 RNE of fl(fl(c * s_b) * S)."""
    return bf16_rne(dequantize_f32(packed, block_scales, S, block, gscale).astype(np.float64))
