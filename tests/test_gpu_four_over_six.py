"""GPU parity of the Four-Over-Six NVFP4 quantizer (MXQ_ROUND_RNE_4OVER6)
against oracle/four_over_six.py, byte for byte: codes, E4M3 block scales, S.
Covers every rowwise kernel shape (register-resident rows with full and
partial lane coverage, rows longer than 8192 in the two-pass kernel), the
three second-scale modes, the MFMA scale layout, 16x16 tiles with a ragged
column count, the config-2 activations and weight at full size, and the
GEMM on 4/6 copies (the format is plain NVFP4)."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import four_over_six as Q
from oracle import gemm as G
from oracle import layout as L
from oracle import nvfp4 as ON
import synth
from tests.util import requires_gpu, to_dev_bf16, from_dev_bf16, to_np, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def mxq():
    import microscaling_quantization_block_amd as m
    return m


def _edge(rows, cols, seed):
    """Per-row log-normal magnitudes, a zero row, a row of negative zeros, a
    row near 2^-60, and grid-aligned blocks that tie or favour one candidate."""
    rs = np.random.default_rng(seed)
    x = rs.standard_normal((rows, cols)) * np.exp(rs.standard_normal((rows, 1)) * 2)
    if rows > 5:
        x[2] = rs.standard_normal(cols) * 2.0 ** -60
        x[3, :16] = [4, 3, 2, 1.5, 1, 0.5, 0, -3, -4, 2, 1, 0.5, 3, -2, 1.5, 0]      # exact at 4
        x[4, :16] = [12, 6, 3, 0, -12, -6, -3, 0, 12, 3, 6, 0, -3, 3, -6, 12]         # tie
        x[5, :16] = [6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, 2, 1, 0.5, 3, 4]         # exact at 6
    b = F.bf16_rne(x)
    if rows > 1:
        b[0] = 0
        b[1] = 0x8000
    return b


def _check_row(m, x, gs, S_given=None, layout=0):
    import torch
    v = F.bf16_bits_to_f64(x)
    g = {"per_row": m.GScale.PER_ROW, "per_tensor": m.GScale.PER_TENSOR, "given": m.GScale.GIVEN}[gs]
    kw = dict(gs=g, rnd=m.Round.RNE_4OVER6, layout=layout)
    if gs == "given":
        kw["gscales"] = torch.tensor([S_given], dtype=torch.float32, device="cuda")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), **kw)
    rc, rs, rS, take4, _, _ = Q.quantize_rowwise(v, gs, S_given, details=True)
    assert np.array_equal(to_np(S), rS)
    sb = to_np(s).reshape(-1)
    if layout:
        sb = L.mfma_to_linear(sb, *rs.shape)
    assert np.array_equal(sb.reshape(rs.shape), rs)
    assert np.array_equal(to_np(c), rc)
    return c, s, S, rc, rs, rS, take4


@pytest.mark.parametrize("shape", [(64, 1024), (40, 768), (33, 2048), (16, 4096), (9, 8192),
                                   (4, 16384), (7, 16), (2100, 256)])
@pytest.mark.parametrize("gs", ["per_row", "per_tensor"])
def test_row_four_over_six(shape, gs):
    m = mxq()
    x = _edge(*shape, 61)
    say(f"nvfp4 ROW 4/6 {shape} {gs}")
    *_, take4 = _check_row(m, x, gs)
    if shape[0] * shape[1] >= 16384:
        assert 0.1 < take4.mean() < 0.9          # both candidates occur


def test_row_four_over_six_given_scale_and_mfma_layout():
    m = mxq()
    x = _edge(64, 512, 62)
    say("nvfp4 ROW 4/6 GIVEN S and MFMA layout")
    _check_row(m, x, "given", S_given=np.float32(0.0071))
    c, s, S, rc, rs, rS, _ = _check_row(m, x, "per_row", layout=m.Layout.MFMA)
    dq = m.mx_dequantize(m.Format.NVFP4, c, s, 64, 512, gscales=S, gs=m.GScale.PER_ROW,
                         layout=m.Layout.MFMA)
    assert np.array_equal(from_dev_bf16(dq), ON.dequantize_bf16(rc, rs, rS, "1x16", "per_row"))


@pytest.mark.parametrize("shape", [(768, 2048), (48, 80), (64, 1040), (16, 16)])
def test_tile16_four_over_six(shape):
    m = mxq()
    x = F.bf16_rne(np.random.default_rng(63).standard_normal(shape) * 0.02)
    if shape[0] < 100:
        x = _edge(*shape, 63)
    v = F.bf16_bits_to_f64(x)
    say(f"nvfp4 TILE 4/6 {shape}")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), block=m.Block.TILE, gs=m.GScale.PER_TENSOR,
                               rnd=m.Round.RNE_4OVER6)
    rc, rs, rS, take4, _, _ = Q.quantize_tile16(v, details=True)
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(c), rc)
    dq = m.mx_dequantize(m.Format.NVFP4, c, s, shape[0], shape[1], block=m.Block.TILE, gscales=S,
                         gs=m.GScale.PER_TENSOR)
    assert np.array_equal(from_dev_bf16(dq), ON.dequantize_bf16(rc, rs, rS, "16x16", "per_tensor"))
    c2, s2, S2, dq2 = m.nvfp4_quantize_dq(to_dev_bf16(x), rnd=m.Round.RNE_4OVER6)
    assert np.array_equal(to_np(c2), rc) and np.array_equal(to_np(s2), rs)
    assert np.array_equal(from_dev_bf16(dq2), from_dev_bf16(dq))
    if shape == (768, 2048):
        assert take4.any() and not take4.all()           # both candidates occur (3% at 4 here)


def test_config2_full_size_and_fprop_on_four_over_six_copies():
    m = mxq()
    d = synth.config2()
    say("nvfp4 4/6 config-2 X 4096x2048 per-token, W 768x2048 16x16, FPROP")
    cx, sx, Sx, rcx, rsx, rSx, tx = _check_row(m, d["x"], "per_row")
    cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(d["w"]), block=m.Block.TILE, gs=m.GScale.PER_TENSOR,
                                  rnd=m.Round.RNE_4OVER6)
    rcw, rsw, rSw = Q.quantize_tile16(F.bf16_bits_to_f64(d["w"]))
    assert np.array_equal(to_np(sw), rsw) and np.array_equal(to_np(cw), rcw)
    out = m.mx_gemm(m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW),
                    m.Operand(m.Format.NVFP4, cw, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR),
                    4096, 768, 2048)
    a64 = ON.dequantize_f64(rcx, rsx, rSx, "1x16", "per_row")
    a32 = ON.dequantize_f32(rcx, rsx, rSx, "1x16", "per_row")
    b64 = ON.dequantize_f64(rcw, rsw, rSw, "16x16", "per_tensor")
    b32 = ON.dequantize_f32(rcw, rsw, rSw, "16x16", "per_tensor")
    frob, worst, ok = G.check(from_dev_bf16(out), a64, b64, a32, b32, rtol_frob=1e-2)
    assert ok, f"frobenius {frob:.3e}, worst {worst:.3f}"
    # the 4/6 copies are closer to the BF16 inputs than plain NVFP4's
    xv = F.bf16_bits_to_f64(d["x"])
    pc, ps, pS = ON.quantize_rowwise(xv, "per_row")
    e46 = np.sum((a64 - xv) ** 2)
    epl = np.sum((ON.dequantize_f64(pc, ps, pS, "1x16", "per_row") - xv) ** 2)
    say(f"config-2 X: squared error 4/6 / plain = {e46 / epl:.3f}; blocks at 4: {tx.mean():.3f}")
    assert e46 < epl
