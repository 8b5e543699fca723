"""Four-Over-Six (4/6) block scaling for NVFP4 weights and activations.

"NVFP4 RL トレーニング" / "The 4-bitter Lesson" (socker-news), section on
Four-Over-Six for RL weights and activations: with the usual NVFP4 scaling
the block max lands on 6, and values near it fall into the widest gap of the
E2M1 grid (4 to 6), so the worst error is 1/6 of the block's range; scaling
some blocks so that their max lands on 4 instead caps it at 1/8.  Pretraining
applies it to activations, RL to the weights as well; the choice costs extra
computation per block, which the page says must stay cheap.

Readings (the page, garbled in places, fixes neither the choice rule nor the
arithmetic):

1. Two candidates per block, under the same second-level scale S as plain
   NVFP4 (S = fl(A / 2688)):
     M = 6: s6 = E4M3_RNE_sat(fl(a_b / fl(6 S)))   (the plain block scale)
     M = 4: s4 = E4M3_RNE_sat(fl(a_b / fl(4 S)))   (saturating at 448: the
            largest blocks of a tensor cannot reach 4 and keep a larger max)
   Each candidate encodes the block exactly as plain NVFP4 does with its own
   s_b: r = fl(1 / fl(s_b S)), y = fl(x r), RNE onto E2M1, signed zeros when
   s_b = 0.
2. The error of a candidate is the binary32 sum of squared dequantization
   errors: d = fl(fl(value(code) s_b) S) (the dequantizer's order),
   e = fl(x - d), then fl(e e) summed as a pairwise tree in element order
   ((e0 + e1) + (e2 + e3)) + ...; for a 16x16 tile, each row's 16 squares by
   that tree, then the 16 row sums by the same tree in row order.
3. The block takes M = 4 iff its error is strictly smaller; ties (an all-zero
   block, a block both candidates represent exactly) keep M = 6.  The stored
   block scale is the chosen s_b, so dequantization and the GEMMs read a 4/6
   copy like any NVFP4 copy.
4. Rounding is RNE only (weights and activations; gradients keep stochastic
   rounding without 4/6).

Test infrastructure only (see the package docstring).
"""

import numpy as np

from .formats import encode_e4m3_rne, e4m3_value, e2m1_value
from . import nvfp4

BLOCK = 16
F32 = np.float32


def tree_sum(v):
    """Binary32 pairwise sum over the last axis (a power of two), neighbours
    first: ((v0 + v1) + (v2 + v3)) + ..."""
    v = np.asarray(v, dtype=F32)
    while v.shape[-1] > 1:
        v = (v[..., 0::2] + v[..., 1::2]).astype(F32)
    return v[..., 0]


def candidate(xb, a_b, S, M):
    """Scale code, element codes and binary32 dequantized values of candidate
    M (6 or 4) for blocks xb [..., n] with block amax a_b [...] and second
    scale S (broadcast to a_b's shape)."""
    S = np.broadcast_to(np.asarray(S, dtype=F32), a_b.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        mS = (F32(M) * S).astype(F32)
        t = (np.asarray(a_b, dtype=F32) / mS).astype(F32)
    t = np.where(S > 0, t, F32(0.0))
    sb = encode_e4m3_rne(t.astype(np.float64))
    codes = nvfp4.encode_block_elements(xb, sb[..., None], S[..., None], "rne")
    v = e2m1_value(codes).astype(F32)
    d = ((v * e4m3_value(sb).astype(F32)[..., None]).astype(F32) * S[..., None]).astype(F32)
    return sb, codes, d


def squared_errors(xb, d):
    e = (np.asarray(xb, dtype=F32) - d).astype(F32)
    return (e * e).astype(F32)


def _choose(xb, a_b, S, err_of):
    """Both candidates and the per-block choice (True = M 4)."""
    s6, c6, d6 = candidate(xb, a_b, S, 6)
    s4, c4, d4 = candidate(xb, a_b, S, 4)
    e6, e4 = err_of(squared_errors(xb, d6)), err_of(squared_errors(xb, d4))
    take4 = e4 < e6
    return np.where(take4, s4, s6), np.where(take4[..., None], c4, c6), take4, e6, e4


def quantize_rowwise(x, gscale="per_row", S_given=None, details=False):
    """1x16 blocks along cols with the 4/6 choice per block.  Returns (packed
    codes [rows, cols/2], block scales [rows, cols/16], S) as the plain
    rowwise quantizer does; details=True adds (take4, err6, err4)."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert cols % BLOCK == 0
    if gscale == "per_row":
        S = nvfp4.second_scale(np.max(np.abs(x), axis=1))
        S_rows = S
    elif gscale == "per_tensor":
        S = nvfp4.second_scale(np.max(np.abs(x))).reshape(1)
        S_rows = np.full(rows, S[0], dtype=F32)
    elif gscale == "given":
        S = np.asarray(S_given, dtype=F32).reshape(1)
        S_rows = np.full(rows, S[0], dtype=F32)
    else:
        raise ValueError(gscale)
    xb = x.reshape(rows, cols // BLOCK, BLOCK)
    a_b = np.max(np.abs(xb), axis=-1)
    S_b = np.broadcast_to(np.asarray(S_rows, dtype=F32).reshape(-1, 1), a_b.shape)
    sb, codes, take4, e6, e4 = _choose(xb, a_b, S_b, tree_sum)
    out = (nvfp4.pack_nibbles(codes.reshape(rows, cols)), sb.astype(np.uint8), S)
    return out + (take4, e6, e4) if details else out


def quantize_tile16(x, gscale="per_tensor", S_given=None, details=False):
    """16x16 tiles with the 4/6 choice per tile.  Returns (packed codes
    [rows, cols/2], tile scales [rows/16, cols/16], S [1])."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert rows % BLOCK == 0 and cols % BLOCK == 0
    if gscale == "per_tensor":
        S = nvfp4.second_scale(np.max(np.abs(x))).reshape(1)
    elif gscale == "given":
        S = np.asarray(S_given, dtype=F32).reshape(1)
    else:
        raise ValueError("16x16 tiles take a per-tensor second scale")
    # tiles as blocks of 256 values in (tile row, tile column) order
    xt = x.reshape(rows // BLOCK, BLOCK, cols // BLOCK, BLOCK).transpose(0, 2, 1, 3)
    xb = xt.reshape(rows // BLOCK, cols // BLOCK, BLOCK * BLOCK)
    a_b = np.max(np.abs(xb), axis=-1)

    def tile_err(sq):            # row sums by the 16-tree, then the rows by it
        return tree_sum(tree_sum(sq.reshape(sq.shape[:-1] + (BLOCK, BLOCK))))

    sb, codes, take4, e6, e4 = _choose(xb, a_b, np.full(a_b.shape, S[0], dtype=F32), tile_err)
    c = codes.reshape(rows // BLOCK, cols // BLOCK, BLOCK, BLOCK).transpose(0, 2, 1, 3)
    out = (nvfp4.pack_nibbles(c.reshape(rows, cols)), sb.astype(np.uint8), S)
    return out + (take4, e6, e4) if details else out
