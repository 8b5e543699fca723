"""GPU parity of nvfp4_quantize_rht (random Hadamard transform of 16-row
blocks, then the columnwise NVFP4 copy) against oracle/rht.py, byte for byte:
codes, E4M3 block scales and the per-tensor S.  Covers RNE and stochastic
rounding, several sign masks, GIVEN and PER_TENSOR second scales, the MFMA
scale layout, strided input, a ragged column count (not a multiple of the
1024 columns a workgroup covers), more row strips than the amax kernel's
grid, and the config-2 WGRAD inputs at full size.  Then the WGRAD GEMM on two
transformed copies (same mask): parity with the oracle's dequantize-then-
matmul of those copies, and closeness to dY^T X itself, which the orthogonal
transform leaves unchanged."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import layout as L
from oracle import nvfp4 as ON
from oracle import rht as R
import synth
from tests.util import requires_gpu, to_dev_bf16, from_dev_bf16, to_np, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def mxq():
    import microscaling_quantization_block_amd as m
    return m


def _edge_rht(rows, cols, seed, extreme=False):
    """Per-row log-normal magnitudes plus a zero column, a column of negative
    zeros and one of tiny values (near 2^-60, inside the A >= 2^-64
    precondition).  extreme: also values near 2^120 (sixteen of them sum to
    less than the binary32 maximum) and random finite bit patterns below
    2^100, which put most other blocks under the smallest block scale."""
    rs = np.random.default_rng(seed)
    x = rs.standard_normal((rows, cols)) * np.exp(rs.standard_normal((rows, 1)) * 3)
    x[:, 0] = 0.0
    x = F.bf16_rne(x)
    x[:, 1] = 0x8000                                                  # -0 down a column
    if cols > 2:
        x[:, 2] = F.bf16_rne(rs.standard_normal(rows) * 2.0 ** -60)
    if extreme and cols > 4:
        x[5 % rows, 3] = F.bf16_rne(np.array([2.0 ** 120]))[0]
        x[6 % rows, 3] = F.bf16_rne(np.array([-1.5 * 2.0 ** 119]))[0]
        x[:, 4] = (rs.integers(0, 0x7180, rows) | (rs.integers(0, 2, rows) << 15)).astype(np.uint16)
    return x


def _check(m, x, mask, rnd="rne", gs="per_tensor", S_given=None, seed=0, tag=0, layout=0):
    import torch
    v = F.bf16_bits_to_f64(x)
    kw = dict(rnd=m.Round.SR if rnd == "sr" else m.Round.RNE, seed=seed, stream_id=1,
              tensor_tag=tag, layout=layout)
    if gs == "given":
        kw.update(gs=m.GScale.GIVEN, gscales=torch.tensor([S_given], dtype=torch.float32, device="cuda"))
    c, s, S = m.nvfp4_quantize_rht(to_dev_bf16(x), mask, **kw)
    rc, rs, rS = R.quantize_colwise_rht(v, mask, gs, rnd, seed, 1, tag, S_given)
    assert np.array_equal(to_np(S), rS)
    sb = to_np(s).reshape(-1)
    if layout:
        sb = L.mfma_to_linear(sb, *rs.shape)
    assert np.array_equal(sb.reshape(rs.shape), rs)
    assert np.array_equal(to_np(c), rc)
    return c, s, S, rc, rs, rS


@pytest.mark.parametrize("shape,mask,rnd,extreme", [
    ((64, 96), 0x5A3C, "rne", False), ((48, 32), 0x0000, "sr", False),
    ((256, 512), 0xFFFF, "sr", False), ((32, 1040), 0x8001, "rne", False),
    ((512, 2048), 0x1234, "rne", False), ((16, 16), 0x00FF, "sr", False),
    ((64, 96), 0x5A3C, "rne", True), ((48, 32), 0xC001, "sr", True)])
def test_rht_col_matches_oracle(shape, mask, rnd, extreme):
    m = mxq()
    x = _edge_rht(*shape, 41, extreme)
    say(f"nvfp4 RHT COL {shape} mask={mask:#06x} {rnd} extreme={extreme}")
    _check(m, x, mask, rnd, seed=7)


@pytest.mark.parametrize("seed,tag", [(0, 0), (2 ** 40 + 3, 5)])
def test_rht_col_stochastic_rounding_streams(seed, tag):
    m = mxq()
    x = _edge_rht(96, 160, 42)
    say(f"nvfp4 RHT COL SR seed={seed} tag={tag}")
    _check(m, x, 0x3C5A, "sr", seed=seed, tag=tag)


def test_rht_col_given_scale_and_mfma_layout():
    m = mxq()
    x = _edge_rht(128, 64, 43)
    say("nvfp4 RHT COL GIVEN S, LINEAR and MFMA layouts")
    _check(m, x, 0x0F0F, "rne", gs="given", S_given=np.float32(0.0173))
    c, s, S, rc, rs, rS = _check(m, x, 0x0F0F, "sr", seed=3, layout=m.Layout.MFMA)
    # the MFMA-layout copy dequantizes like the linear one
    dq = m.mx_dequantize(m.Format.NVFP4, c, s, 64, 128, gscales=S, gs=m.GScale.PER_TENSOR,
                         layout=m.Layout.MFMA)
    assert np.array_equal(from_dev_bf16(dq), ON.dequantize_bf16(rc, rs, rS, "1x16", "per_tensor"))


def test_plain_col_mfma_layout():
    """The columnwise copy without the transform also places its scales in
    the MFMA layout when asked."""
    m = mxq()
    x = _edge_rht(128, 96, 44)
    say("nvfp4 COL MFMA layout")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), block=m.Block.COL, gs=m.GScale.PER_TENSOR,
                               layout=m.Layout.MFMA)
    rc, rs, rS = ON.quantize_colwise(F.bf16_bits_to_f64(x))
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(L.mfma_to_linear(to_np(s).reshape(-1), *rs.shape).reshape(rs.shape), rs)
    assert np.array_equal(to_np(c), rc)


def test_rht_col_strided_input():
    m = mxq()
    x = _edge_rht(64, 128, 45)
    say("nvfp4 RHT COL strided input (ld 192)")
    big = to_dev_bf16(np.concatenate([x, np.zeros((64, 64), dtype=np.uint16)], axis=1))
    c, s, S = m.nvfp4_quantize_rht(big[:, :128], 0x9669)
    rc, rs, rS = R.quantize_colwise_rht(F.bf16_bits_to_f64(x), 0x9669)
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(c), rc)


def test_rht_amax_grid_walks_many_strips():
    """4096 strips of 16 rows over 64 columns: the amax kernel's grid holds
    at most 2048 workgroups, so each walks two strips."""
    m = mxq()
    x = F.bf16_rne(np.random.default_rng(46).standard_normal((65536, 64)))
    x[65530, 17] = F.bf16_rne(np.array([40.0]))[0]         # the tensor max sits in the last strip
    say("nvfp4 RHT COL 65536x64")
    _check(m, x, 0xA5A5)


def test_rht_config2_wgrad_inputs_full_size():
    m = mxq()
    d = synth.config2()
    say("nvfp4 RHT COL config-2 X 4096x2048 (RNE) and dY 4096x768 (SR)")
    _check(m, d["x"], 0x6B2D, "rne")
    _check(m, d["dy"], 0x6B2D, "sr", seed=11)


def test_rht_wgrad_gemm():
    """dW = dY^T X from two transformed columnwise copies with one mask."""
    m = mxq()
    T, H, I = 512, 256, 160
    x = F.bf16_rne(np.random.default_rng(47).standard_normal((T, H)))
    dy = F.bf16_rne(np.random.default_rng(48).standard_normal((T, I)) * 1e-3)
    x[100, 3] = F.bf16_rne(np.array([30.0]))[0]             # an outlier the transform spreads
    mask = 0x2DB4
    say(f"nvfp4 WGRAD on RHT copies {I}x{H}x{T}")
    cd, sd, Sd = m.nvfp4_quantize_rht(to_dev_bf16(dy), mask, rnd=m.Round.SR, seed=5)
    cx, sx, Sx = m.nvfp4_quantize_rht(to_dev_bf16(x), mask)
    dw = m.mx_gemm(m.Operand(m.Format.NVFP4, cd, sd, Sd, gs=m.GScale.PER_TENSOR),
                   m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_TENSOR), I, H, T)
    a64 = ON.dequantize_f64(to_np(cd), to_np(sd), to_np(Sd), "1x16", "per_tensor")
    a32 = ON.dequantize_f32(to_np(cd), to_np(sd), to_np(Sd), "1x16", "per_tensor")
    b64 = ON.dequantize_f64(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_tensor")
    b32 = ON.dequantize_f32(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_tensor")
    c = from_dev_bf16(dw)
    frob, worst, ok = G.check(c, a64, b64, a32, b32, rtol_frob=1e-2)
    assert ok, f"frobenius {frob:.3e}, worst element ratio {worst:.3f}"
    # the transform cancels in the product: close to the untransformed dY^T X
    # (the oracle's copies give 0.167 here, about what the plain columnwise
    # copies give: Gaussian data has no outliers for the transform to spread)
    exact = F.bf16_bits_to_f64(dy).T @ F.bf16_bits_to_f64(x)
    rel = np.linalg.norm(F.bf16_bits_to_f64(c) - exact) / np.linalg.norm(exact)
    say(f"WGRAD with RHT: relative error to dY^T X {rel:.3f}")
    assert rel < 0.25
