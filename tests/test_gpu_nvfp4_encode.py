"""GPU parity of the NVFP4 element encode, exhaustively, and of the quantizers
on inputs whose second scale S is tiny.

* Every BF16 magnitude within 16 binades below a block's maximum (plus zero
  and the smallest subnormal), both signs, under each of the 126 positive
  finite E4M3 block scales and several caller-given S (powers of two, whose
  anchors then give each scale exactly, and one that is not), through the
  rowwise quantizer: codes and scales byte-identical to the oracle, for
  round-to-nearest-even and for stochastic rounding (two seeds).  The same
  with a block maximum past 448 * 6 * S (a saturated block scale, elements
  far beyond 6, including products that overflow binary32).
* Rows, tiles and columns whose S is below 2^-64 (where the element chain
  runs in the scaled frame; "Um Quantizador Compartilhado É o Verdadeiro
  Mecanismo" in "Miles Blackwell RL ..." asks for byte-identical quantizers
  on boundary values), for RNE, stochastic rounding and Four-Over-Six."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import nvfp4 as ON
from oracle import four_over_six as O46
from oracle import rht as OR
from tests.util import requires_gpu, to_dev_bf16, from_dev_bf16, to_np, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def mxq():
    import microscaling_quantization_block_amd as m
    return m


ALL = np.arange(0x7F80, dtype=np.uint32).astype(np.uint16)        # finite BF16 magnitudes
ALLV = F.bf16_bits_to_f64(ALL)


def _blocks_for(anchor_bits):
    """Rows of 16-value blocks: each block leads with the anchor (sign
    alternating) and holds 15 of the magnitudes in [a 2^-16, a] plus 0 and
    the smallest subnormal, each with both signs."""
    a = F.bf16_bits_to_f64(np.array([anchor_bits], dtype=np.uint16))[0]
    keep = ALL[((ALLV >= a * 2.0 ** -16) & (ALLV <= a)) | (ALL <= 1)]
    vals = np.concatenate([keep, keep | 0x8000])
    n = -(-len(vals) // 15)
    body = np.full(n * 15, anchor_bits, dtype=np.uint16)
    body[:len(vals)] = vals
    lead = np.full((n, 1), anchor_bits, dtype=np.uint16)
    lead[1::2] |= 0x8000
    return np.concatenate([lead, body.reshape(n, 15)], axis=1)


def _rows(blocks, per_row=64):
    pad = (-len(blocks)) % per_row
    z = np.zeros((pad, 16), dtype=np.uint16)
    return np.concatenate([blocks, z]).reshape(-1, per_row * 16)


def _check_given(m, x, S, what, rnd="rne", seed=0):
    say(f"nvfp4 element encode {what}: {x.shape[0]}x{x.shape[1]} given S={float(S):.4g} {rnd} seed {seed}")
    Sd = __import__("torch").tensor([float(S)], dtype=__import__("torch").float32, device="cuda")
    c, s, _ = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.GIVEN, gscales=Sd,
                               rnd=m.Round.SR if rnd == "sr" else m.Round.RNE, seed=seed)
    rc, rs, _ = ON.quantize_rowwise(F.bf16_bits_to_f64(x), "given", rnd=rnd, seed=seed, S_given=S)
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(c), rc)
    return rs


@pytest.mark.parametrize("S", [1.0, 2.0 ** -20, 2.0 ** 30, 2.0 ** -70, 2.0 ** -100, 0.0123])
def test_every_bf16_magnitude_under_every_e4m3_block_scale(S):
    """RNE onto E2M1 (the hardware conversion) of every BF16 magnitude that
    can share a block with a given block maximum, under all 126 positive
    finite block scales."""
    m = mxq()
    S = np.float32(S)
    e4 = F.e4m3_value(np.arange(1, 127))
    anchors = F.bf16_rne(e4 * 6.0 * np.float64(S))
    x = _rows(np.concatenate([_blocks_for(a) for a in anchors]))
    rs = _check_given(m, x, S, "all scales")
    if float(S) in (1.0, 2.0 ** -20, 2.0 ** 30, 2.0 ** -70, 2.0 ** -100):
        # power-of-two S: the anchors hit every positive finite scale exactly
        assert set(np.unique(rs).tolist()) >= set(range(1, 127))


@pytest.mark.parametrize("seed", [3, 2 ** 40 + 17])
@pytest.mark.parametrize("S", [1.0, 0.0123, 2.0 ** -70])
def test_every_bf16_magnitude_under_every_e4m3_block_scale_sr(S, seed):
    """Stochastic rounding onto E2M1 (the hardware conversion with the
    magnitude first rounded up to a multiple of 2^-17) of the same inputs:
    every BF16 magnitude that can share a block with a given block maximum,
    under all 126 positive finite block scales.  With S = 0.0123 the
    reciprocals are not powers of two, so y = x * r carries full binary32
    mantissas (the fraction bits below 2^-16 decide the boundary cases);
    2^-70 runs the chain in the scaled frame."""
    m = mxq()
    S = np.float32(S)
    e4 = F.e4m3_value(np.arange(1, 127))
    anchors = F.bf16_rne(e4 * 6.0 * np.float64(S))
    x = _rows(np.concatenate([_blocks_for(a) for a in anchors]))
    _check_given(m, x, S, "all scales", rnd="sr", seed=seed)


@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("S", [1.0, 2.0 ** -70])
def test_saturated_block_scale_and_overflowing_products(S, rnd):
    """Block maxima far past 448 * 6 * S: the scale saturates at 448 and the
    elements at 6, including products x * r beyond the binary32 range."""
    m = mxq()
    S = np.float32(S)
    anchors = F.bf16_rne(np.array([448.0 * 6.0 * 1.5, 448.0 * 6.0 * 2.0 ** 20, 3.0e38]) * np.float64(S))
    anchors = np.concatenate([anchors, np.array([0x7F7F], dtype=np.uint16)])
    x = _rows(np.concatenate([_blocks_for(a) for a in anchors]))
    rs = _check_given(m, x, S, "saturation", rnd=rnd, seed=11)
    assert 0x7E in rs


# ------------------------------------------------------------ tiny S

def _tiny(seed, rows, cols, lo=-112, hi=-65, spread=24):
    """Rows with amax 2^lo .. 2^hi (S = A / 2688 below 2^-64) and 16-value
    blocks spread over `spread` binades below their row's max, so that many
    blocks have a subnormal s_b * S; one zero column, one of negative zeros,
    and the [2^-126, 2^-128, 0 ...] block of the smallest rows."""
    rs = np.random.default_rng(seed)
    mant = rs.uniform(1.0, 2.0, (rows, cols)) * rs.choice([-1.0, 1.0], (rows, cols))
    expo = rs.integers(-6, 1, (rows, cols)).astype(np.float64)
    shrink = rs.integers(0, spread, (rows, cols // 16)).repeat(16, axis=1).astype(np.float64)
    shrink[:, :16] = 0
    x = mant * np.exp2(expo - shrink + np.linspace(lo, hi, rows)[:, None])
    b = F.bf16_rne(x)
    b[:, 3] = 0
    b[:, 7] = 0x8000
    b[0, :16] = 0
    b[0, 0], b[0, 1] = F.bf16_rne(np.array([2.0 ** -126, 2.0 ** -128]))
    return b


@pytest.mark.parametrize("rnd", ["rne", "sr", "4over6"])
@pytest.mark.parametrize("cols", [512, 8208])
def test_tiny_rows(rnd, cols):
    """Per-token rows (the one-wave-per-row kernel, and the two-pass kernel
    for rows past 8192 values)."""
    m = mxq()
    x = _tiny(40, 48, cols)
    v = F.bf16_bits_to_f64(x)
    R = {"rne": m.Round.RNE, "sr": m.Round.SR, "4over6": m.Round.RNE_4OVER6}[rnd]
    say(f"nvfp4 ROW tiny S {x.shape} {rnd}")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW, rnd=R, seed=11)
    if rnd == "4over6":
        rc, rsb, rS = O46.quantize_rowwise(v, "per_row")
    else:
        rc, rsb, rS = ON.quantize_rowwise(v, "per_row", rnd=rnd, seed=11)
    assert np.all(rS < ON.TINY_S)
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(s), rsb)
    assert np.array_equal(to_np(c), rc)
    dq = m.mx_dequantize(m.Format.NVFP4, c, s, x.shape[0], cols, gscales=S, gs=m.GScale.PER_ROW)
    assert np.array_equal(from_dev_bf16(dq), ON.dequantize_bf16(rc, rsb, rS, "1x16", "per_row"))


@pytest.mark.parametrize("rnd", ["rne", "sr", "4over6"])
def test_tiny_tensor_tile16_and_col(rnd):
    """A tensor whose amax is 2^-100 (per-tensor S below 2^-64): 16x16 tiles
    (with the dequantized copy of the fused quantizer), and 16x1 columns with
    and without the Hadamard transform."""
    m = mxq()
    x = _tiny(41, 64, 256, lo=-100, hi=-100, spread=20)
    x[0, 0] = F.bf16_rne(np.array([2.0 ** -100]))[0]
    v = F.bf16_bits_to_f64(x)
    xd = to_dev_bf16(x)
    R = {"rne": m.Round.RNE, "sr": m.Round.SR, "4over6": m.Round.RNE_4OVER6}[rnd]
    say(f"nvfp4 TILE tiny S {x.shape} {rnd}")
    c, s, S = m.nvfp4_quantize(xd, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, rnd=R, seed=12)
    if rnd == "4over6":
        rc, rsb, rS = O46.quantize_tile16(v)
    else:
        rc, rsb, rS = ON.quantize_tile16(v, rnd=rnd, seed=12)
    assert rS[0] < ON.TINY_S
    assert np.array_equal(to_np(S), rS) and np.array_equal(to_np(s), rsb) and np.array_equal(to_np(c), rc)
    if rnd != "sr":
        c2, s2, S2, dq2 = m.nvfp4_quantize_dq(xd, rnd=R)
        assert np.array_equal(to_np(c2), rc) and np.array_equal(to_np(s2), rsb)
        assert np.array_equal(from_dev_bf16(dq2), ON.dequantize_bf16(rc, rsb, rS, "16x16", "per_tensor"))
        return
    say("nvfp4 COL tiny S, plain and with the Hadamard transform, SR")
    c, s, S = m.nvfp4_quantize(xd, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=m.Round.SR, seed=13,
                               stream_id=1)
    rc, rsb, rS = ON.quantize_colwise(v, rnd="sr", seed=13, stream_id=1)
    assert np.array_equal(to_np(S), rS) and np.array_equal(to_np(s), rsb) and np.array_equal(to_np(c), rc)
    c, s, S = m.nvfp4_quantize_rht(xd, 0x5A3C, rnd=m.Round.SR, seed=13, stream_id=1)
    rc, rsb, rS = OR.quantize_colwise_rht(v, 0x5A3C, rnd="sr", seed=13, stream_id=1)
    assert rS[0] < ON.TINY_S
    assert np.array_equal(to_np(S), rS) and np.array_equal(to_np(s), rsb) and np.array_equal(to_np(c), rc)
