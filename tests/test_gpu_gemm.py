"""GPU parity of the block-scaled GEMMs against the oracle's
dequantize-then-matmul: relative Frobenius error <= 1e-2 against float64, and
the element-wise bound |C - C32| <= 2^-8 |C32| + K 2^-23 (|A| |B|) against the
binary32 path; bit-exact equality where every product and sum is exact (unit
scales, small codes).  Operands are quantized by the GPU; the oracle
dequantizes the GPU's own codes (already checked byte-identical to the
oracle's in the quantizer tests) and also requantizes from the BF16 inputs to
confirm they are the same bytes."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import mxfp8 as OM
from oracle import nvfp4 as ON
import synth
from tests.util import requires_gpu, to_dev_bf16, from_dev_bf16, to_np, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def mxq():
    import microscaling_quantization_block_amd as m
    return m


def _bf16(shape, std, seed):
    return F.bf16_rne(np.random.default_rng(seed).standard_normal(shape) * std)


def _assert_gemm(c_dev, a64, b64, a32, b32, rtol=1e-2):
    c = from_dev_bf16(c_dev)
    frob, worst, ok = G.check(c, a64, b64, a32, b32, rtol_frob=rtol)
    assert ok, f"frobenius {frob:.3e}, worst element ratio {worst:.3f}"
    return frob, worst


# ------------------------------------------------------------------ MXFP8

def _mx_row(m, bits):
    c, s = m.mx_quantize(to_dev_bf16(bits))
    return c, s


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (200, 96, 128), (33, 160, 96), (512, 384, 1024)])
def test_mxfp8_fprop(M, N, K):
    m = mxq()
    x = _bf16((M, K), 1.0, 1)
    w = _bf16((N, K), 0.02, 2)
    say(f"mxfp8 FPROP {M}x{N}x{K}")
    cx, sx = _mx_row(m, x)
    cw, sw = _mx_row(m, w)
    A = m.Operand(m.Format.MXFP8, cx, sx)
    B = m.Operand(m.Format.MXFP8, cw, sw)
    out = m.mx_gemm(A, B, M, N, K)
    a64 = OM.dequantize_f64(to_np(cx), to_np(sx))
    b64 = OM.dequantize_f64(to_np(cw), to_np(sw))
    _assert_gemm(out, a64, b64, a64, b64)


def test_mxfp8_config1_gemm():
    m = mxq()
    d = synth.config1()
    say("mxfp8 config-1 GEMM 256x512x256")
    cx, sx = _mx_row(m, d["x"])
    cw, sw = _mx_row(m, d["w"])
    out = m.mx_gemm(m.Operand(m.Format.MXFP8, cx, sx), m.Operand(m.Format.MXFP8, cw, sw), 256, 256, 512)
    rc, rs = OM.quantize_rowwise(F.bf16_bits_to_f64(d["x"]))
    assert np.array_equal(to_np(cx), rc)
    a64 = OM.dequantize_f64(to_np(cx), to_np(sx))
    b64 = OM.dequantize_f64(to_np(cw), to_np(sw))
    _assert_gemm(out, a64, b64, a64, b64)


def test_mxfp8_unit_scale_exact():
    """Codes restricted to small integers with E8M0 scale 1: every product and
    partial sum is exact in binary32, so the BF16 output must equal the BF16
    rounding of the exact result bit for bit."""
    m = mxq()
    import torch
    rs = np.random.default_rng(3)
    ints = np.array([v for v in range(-16, 17)], dtype=np.float64)
    M, N, K = 96, 64, 256
    a = rs.choice(ints, (M, K))
    b = rs.choice(ints, (N, K))
    ca = torch.from_numpy(F.encode_e4m3_rne(a)).cuda()
    cb = torch.from_numpy(F.encode_e4m3_rne(b)).cuda()
    one = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda")
    oneb = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda")
    say("mxfp8 unit-scale exact 96x64x256")
    out = m.mx_gemm(m.Operand(m.Format.MXFP8, ca, one), m.Operand(m.Format.MXFP8, cb, oneb), M, N, K)
    assert np.array_equal(from_dev_bf16(out), F.bf16_rne(a @ b.T))


def test_mxfp8_dgrad_transposed_32x32_weight_and_wgrad():
    """DGRAD dX = dY W with W's 32x32-tile copy read transposed; WGRAD
    dW = dY^T X with both operands' columnwise copies."""
    m = mxq()
    T, H, I = 256, 192, 160
    x = _bf16((T, H), 1.0, 4)
    w = _bf16((I, H), 0.02, 5)           # W [N_f=I, K_f=H]
    dy = _bf16((T, I), 1e-3, 6)
    say("mxfp8 DGRAD (transposed 32x32 W) and WGRAD")
    cw, sw = m.mx_quantize(to_dev_bf16(w), block=m.Block.TILE)
    cdy, sdy, cdyc, sdyc = m.mx_quantize(to_dev_bf16(dy), block=m.Block.DUAL)
    cx, sx, cxc, sxc = m.mx_quantize(to_dev_bf16(x), block=m.Block.DUAL)
    # DGRAD: C[T, H] = sum_i dY[t, i] W[i, h]  (B[n=h, k=i] = W[i, h], stored [K, N])
    B = m.Operand(m.Format.MXFP8, cw, sw, block=m.Block.TILE, transposed=True)
    dx = m.mx_gemm(m.Operand(m.Format.MXFP8, cdy, sdy), B, T, H, I)
    a64 = OM.dequantize_f64(to_np(cdy), to_np(sdy))
    w64 = OM.dequantize_f64(to_np(cw), to_np(sw), "32x32")
    _assert_gemm(dx, a64, w64.T.copy(), a64, w64.T.copy())
    # the quantizer's transposed tile copy, read untransposed, gives the same bits
    _, _, cwt, swt = m.mx_quantize(to_dev_bf16(w), block=m.Block.TILE, transposed_copy=True)
    dx2 = m.mx_gemm(m.Operand(m.Format.MXFP8, cdy, sdy),
                    m.Operand(m.Format.MXFP8, cwt, swt, block=m.Block.TILE), T, H, I)
    assert np.array_equal(from_dev_bf16(dx2), from_dev_bf16(dx))
    # the same tile copy read untransposed serves FPROP
    y = m.mx_gemm(m.Operand(m.Format.MXFP8, cx, sx),
                  m.Operand(m.Format.MXFP8, cw, sw, block=m.Block.TILE), T, I, H)
    x64 = OM.dequantize_f64(to_np(cx), to_np(sx))
    _assert_gemm(y, x64, w64, x64, w64)
    # WGRAD: C[I, H] = sum_t dY[t, i] X[t, h]: A = dY colwise [I, T], B = X colwise [H, T]
    dw = m.mx_gemm(m.Operand(m.Format.MXFP8, cdyc, sdyc), m.Operand(m.Format.MXFP8, cxc, sxc), I, H, T)
    ga = OM.dequantize_f64(to_np(cdyc), to_np(sdyc))
    gb = OM.dequantize_f64(to_np(cxc), to_np(sxc))
    _assert_gemm(dw, ga, gb, ga, gb)


def test_mxfp8_mfma_layout_operands():
    m = mxq()
    M, N, K = 128, 96, 512
    x = _bf16((M, K), 1.0, 7)
    w = _bf16((N if N % 32 == 0 else 128, K), 0.02, 8)
    say("mxfp8 GEMM with MFMA-layout scales")
    cx, sx = m.mx_quantize(to_dev_bf16(x), layout=m.Layout.MFMA)
    cw, sw = m.mx_quantize(to_dev_bf16(w), layout=m.Layout.MFMA)
    out = m.mx_gemm(m.Operand(m.Format.MXFP8, cx, sx, layout=m.Layout.MFMA),
                    m.Operand(m.Format.MXFP8, cw, sw, layout=m.Layout.MFMA), M, N, K)
    rcx, rsx = OM.quantize_rowwise(F.bf16_bits_to_f64(x))
    rcw, rsw = OM.quantize_rowwise(F.bf16_bits_to_f64(w))
    a64, b64 = OM.dequantize_f64(rcx, rsx), OM.dequantize_f64(rcw, rsw)
    _assert_gemm(out, a64, b64, a64, b64)


@pytest.mark.parametrize("M,N,K,a_mfma,b_kind", [
    (600, 416, 384, False, "row"),        # 3 x 2 tiles, ragged M; 6 stages: one unrolled body + 2
    (256, 256, 128, True, "row_mfma"),    # one tile, 2 stages (the tail alone)
    (544, 320, 1024, True, "tile"),       # 32x32 weight scales; 16 stages, no tail
    (1000, 300, 640, False, "row"),       # ragged N (not a multiple of 32); 10 stages
    (768, 352, 768, False, "row_mfma"),   # 12 stages: three unrolled bodies
])
def test_mxfp8_direct_to_lds_kernel(M, N, K, a_mfma, b_kind):
    """Configuration 7 (MXFP8, 256x256 tiles on 4 waves, operands loaded
    straight into LDS) on ragged shapes, with linear and MFMA-layout scales
    and 32x32 weight tiles: matches the oracle and gives the bits of the
    register-staged 256x128 kernel (configuration 5)."""
    m = mxq()
    x = _bf16((M, K), 1.0, 80)
    w = _bf16((N, K), 0.02, 81)
    say(f"mxfp8 direct-to-LDS {M}x{N}x{K} a_mfma={a_mfma} b={b_kind}")
    la = m.Layout.MFMA if a_mfma else m.Layout.LINEAR
    cx, sx = m.mx_quantize(to_dev_bf16(x), layout=la)
    A = m.Operand(m.Format.MXFP8, cx, sx, layout=la)
    rcx, rsx = OM.quantize_rowwise(F.bf16_bits_to_f64(x))
    a64 = OM.dequantize_f64(rcx, rsx)
    if b_kind == "tile":
        cw, sw = m.mx_quantize(to_dev_bf16(w), block=m.Block.TILE)
        B = m.Operand(m.Format.MXFP8, cw, sw, block=m.Block.TILE)
        rcw, rsw = OM.quantize_tile32(F.bf16_bits_to_f64(w))
        b64 = OM.dequantize_f64(rcw, rsw, "32x32")
    else:
        lb = m.Layout.MFMA if b_kind == "row_mfma" else m.Layout.LINEAR
        cw, sw = m.mx_quantize(to_dev_bf16(w), layout=lb)
        B = m.Operand(m.Format.MXFP8, cw, sw, layout=lb)
        rcw, rsw = OM.quantize_rowwise(F.bf16_bits_to_f64(w))
        b64 = OM.dequantize_f64(rcw, rsw)
    try:
        m.mx_gemm_set_tile(7)
        out7 = m.mx_gemm(A, B, M, N, K)
        _assert_gemm(out7, a64, b64, a64, b64)
        m.mx_gemm_set_tile(5)
        out5 = m.mx_gemm(A, B, M, N, K)
    finally:
        m.mx_gemm_set_tile(-1)
    o7, o5 = from_dev_bf16(out7), from_dev_bf16(out5)
    assert np.array_equal(o7, o5), f"{int(np.sum(o7 != o5))} elements differ from the 256x128 kernel"


@pytest.mark.parametrize("M,N,K,a_mfma,b_kind", [
    (4100, 8224, 1024, False, "tile"),    # 17 x 33 tiles (more than one round), ragged M and N; 8 pairs
    (8192, 4160, 1536, False, "row"),     # 32 x 17 tiles, ragged N; 12 pairs, linear scales on both
    (4352, 8448, 2048, True, "row_mfma"), # 17 x 33 tiles; 16 pairs, MFMA-layout scales on both
])
def test_mxfp8_direct_to_lds_kernel_many_tiles(M, N, K, a_mfma, b_kind):
    """Configuration 7 for MXFP8 (the whole-line kernel) over more tiles
    than the CUs, in runs of four tile rows per XCD, with ragged edges and
    every scale layout: matches the oracle and gives the bits of the
    register-staged 256x128 kernel (configuration 5)."""
    m = mxq()
    x = _bf16((M, K), 1.0, 84)
    w = _bf16((N, K), 0.02, 85)
    say(f"mxfp8 direct-to-LDS, many tiles {M}x{N}x{K} a_mfma={a_mfma} b={b_kind}")
    la = m.Layout.MFMA if a_mfma else m.Layout.LINEAR
    cx, sx = m.mx_quantize(to_dev_bf16(x), layout=la)
    A = m.Operand(m.Format.MXFP8, cx, sx, layout=la)
    rcx, rsx = OM.quantize_rowwise(F.bf16_bits_to_f64(x))
    a64 = OM.dequantize_f64(rcx, rsx)
    if b_kind == "tile":
        cw, sw = m.mx_quantize(to_dev_bf16(w), block=m.Block.TILE)
        B = m.Operand(m.Format.MXFP8, cw, sw, block=m.Block.TILE)
        rcw, rsw = OM.quantize_tile32(F.bf16_bits_to_f64(w))
        b64 = OM.dequantize_f64(rcw, rsw, "32x32")
    else:
        lb = m.Layout.MFMA if b_kind == "row_mfma" else m.Layout.LINEAR
        cw, sw = m.mx_quantize(to_dev_bf16(w), layout=lb)
        B = m.Operand(m.Format.MXFP8, cw, sw, layout=lb)
        rcw, rsw = OM.quantize_rowwise(F.bf16_bits_to_f64(w))
        b64 = OM.dequantize_f64(rcw, rsw)
    try:
        m.mx_gemm_set_tile(7)
        out7 = m.mx_gemm(A, B, M, N, K)
        _assert_gemm(out7, a64, b64, a64, b64)
        m.mx_gemm_set_tile(5)
        out5 = m.mx_gemm(A, B, M, N, K)
    finally:
        m.mx_gemm_set_tile(-1)
    o7, o5 = from_dev_bf16(out7), from_dev_bf16(out5)
    assert np.array_equal(o7, o5), f"{int(np.sum(o7 != o5))} elements differ from the 256x128 kernel"


@pytest.mark.parametrize("M,N,K,a_mfma,b_kind", [
    (600, 416, 384, False, "tile"),       # 3 x 2 tiles, ragged M; 3 stages of 128 K
    (256, 256, 128, True, "row_mfma"),    # one tile, one stage
    (544, 320, 1024, True, "tile"),       # 16x16 weight scales; 8 stages
    (1000, 300, 640, False, "row"),       # ragged N; 5 stages
    (768, 352, 1280, False, "row_mfma"),  # 10 stages
])
@pytest.mark.parametrize("tile", [7, 8])
def test_nvfp4_direct_to_lds_kernel(M, N, K, a_mfma, b_kind, tile):
    """Configuration 7 for NVFP4 (256x256 tiles on 4 waves, codes and scale
    words loaded straight into LDS, each wave converting its fragments) on
    ragged shapes, with linear and MFMA-layout scales and 16x16 weight
    tiles: matches the oracle and gives the bits of the ping-pong 256x256
    kernel (configuration 6)."""
    m = mxq()
    x = _bf16((M, K), 1.0, 82)
    w = _bf16((N, K), 0.02, 83)
    say(f"nvfp4 direct-to-LDS tile {tile} {M}x{N}x{K} a_mfma={a_mfma} b={b_kind}")
    la = m.Layout.MFMA if a_mfma else m.Layout.LINEAR
    cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW, layout=la)
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW, layout=la)
    rc, rs, rS = ON.quantize_rowwise(F.bf16_bits_to_f64(x), "per_row")
    a64 = ON.dequantize_f64(rc, rs, rS, "1x16", "per_row")
    a32 = ON.dequantize_f32(rc, rs, rS, "1x16", "per_row")
    if b_kind == "tile":
        cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(w), block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
        B = m.Operand(m.Format.NVFP4, cw, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
        wc, ws, wS = ON.quantize_tile16(F.bf16_bits_to_f64(w))
        bl = "16x16"
    else:
        lb = m.Layout.MFMA if b_kind == "row_mfma" else m.Layout.LINEAR
        cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(w), gs=m.GScale.PER_TENSOR, layout=lb)
        B = m.Operand(m.Format.NVFP4, cw, sw, Sw, gs=m.GScale.PER_TENSOR, layout=lb)
        wc, ws, wS = ON.quantize_rowwise(F.bf16_bits_to_f64(w), "per_tensor")
        bl = "1x16"
    b64 = ON.dequantize_f64(wc, ws, wS, bl, "per_tensor")
    b32 = ON.dequantize_f32(wc, ws, wS, bl, "per_tensor")
    try:
        m.mx_gemm_set_tile(tile)
        out7 = m.mx_gemm(A, B, M, N, K)
        _assert_gemm(out7, a64, b64, a32, b32)
        m.mx_gemm_set_tile(6)
        out6 = m.mx_gemm(A, B, M, N, K)
    finally:
        m.mx_gemm_set_tile(-1)
    o7, o6 = from_dev_bf16(out7), from_dev_bf16(out6)
    assert np.array_equal(o7, o6), f"{int(np.sum(o7 != o6))} elements differ from the ping-pong kernel"


# ------------------------------------------------------------------ NVFP4

def _nv_ops(m, x, w, w_tile=True):
    cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
    if w_tile:
        cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(w), block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
    else:
        cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(w), gs=m.GScale.PER_TENSOR)
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
    B = m.Operand(m.Format.NVFP4, cw, sw, Sw, block=m.Block.TILE if w_tile else m.Block.ROW,
                  gs=m.GScale.PER_TENSOR)
    a64 = ON.dequantize_f64(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
    a32 = ON.dequantize_f32(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
    bl = "16x16" if w_tile else "1x16"
    b64 = ON.dequantize_f64(to_np(cw), to_np(sw), to_np(Sw), bl, "per_tensor")
    b32 = ON.dequantize_f32(to_np(cw), to_np(sw), to_np(Sw), bl, "per_tensor")
    return A, B, (a64, a32, b64, b32), (cw, sw, Sw)


@pytest.mark.parametrize("M,N,K,tile", [(256, 128, 512, True), (100, 48, 96, True), (64, 80, 256, False)])
def test_nvfp4_fprop(M, N, K, tile):
    m = mxq()
    x = F.bf16_rne(np.random.default_rng(9).standard_normal((M, K)) *
                   np.exp(np.random.default_rng(10).standard_normal((M, 1))))
    w = _bf16((N, K), 0.02, 11)
    say(f"nvfp4 FPROP {M}x{N}x{K} tile={tile}")
    A, B, (a64, a32, b64, b32), _ = _nv_ops(m, x, w, tile)
    out = m.mx_gemm(A, B, M, N, K)
    _assert_gemm(out, a64, b64, a32, b32)


def test_nvfp4_config2_fprop_full_size():
    m = mxq()
    d = synth.config2()
    say("nvfp4 config-2 FPROP 4096x768x2048")
    A, B, (a64, a32, b64, b32), _ = _nv_ops(m, d["x"], d["w"], True)
    out = m.mx_gemm(A, B, 4096, 768, 2048)
    frob, worst = _assert_gemm(out, a64, b64, a32, b32)
    say(f"config-2 FPROP frobenius {frob:.3e}, worst {worst:.3f}")


def test_nvfp4_unit_scale_exact():
    m = mxq()
    import torch
    rs = np.random.default_rng(12)
    M, N, K = 64, 96, 512
    ca = rs.integers(0, 16, (M, K)).astype(np.uint8)
    cb = rs.integers(0, 16, (N, K)).astype(np.uint8)
    pa = torch.from_numpy(ON.pack_nibbles(ca)).cuda()
    pb = torch.from_numpy(ON.pack_nibbles(cb)).cuda()
    one_a = torch.full((M, K // 16), 0x38, dtype=torch.uint8, device="cuda")   # E4M3 1.0
    one_b = torch.full((N, K // 16), 0x38, dtype=torch.uint8, device="cuda")
    Sa = torch.ones(M, dtype=torch.float32, device="cuda")
    Sb = torch.ones(1, dtype=torch.float32, device="cuda")
    say("nvfp4 unit-scale exact 64x96x512")
    out = m.mx_gemm(m.Operand(m.Format.NVFP4, pa, one_a, Sa, gs=m.GScale.PER_ROW),
                    m.Operand(m.Format.NVFP4, pb, one_b, Sb, gs=m.GScale.PER_TENSOR), M, N, K)
    exact = F.e2m1_value(ca) @ F.e2m1_value(cb).T
    assert np.array_equal(from_dev_bf16(out), F.bf16_rne(exact))


def test_nvfp4_dgrad_transposed_and_wgrad_with_sr():
    m = mxq()
    T, H, I = 256, 128, 96
    x = _bf16((T, H), 1.0, 13)
    w = _bf16((I, H), 0.02, 14)
    dy = _bf16((T, I), 1e-3, 15)
    say("nvfp4 DGRAD (transposed 16x16 W, SR dY) and WGRAD (columnwise copies)")
    cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(w), block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
    cdy, sdy, Sdy = m.nvfp4_quantize(to_dev_bf16(dy), gs=m.GScale.PER_ROW, rnd=m.Round.SR, seed=0)
    dx = m.mx_gemm(m.Operand(m.Format.NVFP4, cdy, sdy, Sdy, gs=m.GScale.PER_ROW),
                   m.Operand(m.Format.NVFP4, cw, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR,
                             transposed=True), T, H, I)
    a64 = ON.dequantize_f64(to_np(cdy), to_np(sdy), to_np(Sdy), "1x16", "per_row")
    a32 = ON.dequantize_f32(to_np(cdy), to_np(sdy), to_np(Sdy), "1x16", "per_row")
    w64 = ON.dequantize_f64(to_np(cw), to_np(sw), to_np(Sw), "16x16", "per_tensor")
    w32 = ON.dequantize_f32(to_np(cw), to_np(sw), to_np(Sw), "16x16", "per_tensor")
    _assert_gemm(dx, a64, w64.T.copy(), a32, w32.T.copy())
    # WGRAD with columnwise copies (per-tensor S; SR for dY with stream 1)
    cdc, sdc, Sdc = m.nvfp4_quantize(to_dev_bf16(dy), block=m.Block.COL, gs=m.GScale.PER_TENSOR,
                                     rnd=m.Round.SR, seed=0, stream_id=1)
    cxc, sxc, Sxc = m.nvfp4_quantize(to_dev_bf16(x), block=m.Block.COL, gs=m.GScale.PER_TENSOR)
    dw = m.mx_gemm(m.Operand(m.Format.NVFP4, cdc, sdc, Sdc, gs=m.GScale.PER_TENSOR),
                   m.Operand(m.Format.NVFP4, cxc, sxc, Sxc, gs=m.GScale.PER_TENSOR), I, H, T)
    ga64 = ON.dequantize_f64(to_np(cdc), to_np(sdc), to_np(Sdc), "1x16", "per_tensor")
    ga32 = ON.dequantize_f32(to_np(cdc), to_np(sdc), to_np(Sdc), "1x16", "per_tensor")
    gb64 = ON.dequantize_f64(to_np(cxc), to_np(sxc), to_np(Sxc), "1x16", "per_tensor")
    gb32 = ON.dequantize_f32(to_np(cxc), to_np(sxc), to_np(Sxc), "1x16", "per_tensor")
    _assert_gemm(dw, ga64, gb64, ga32, gb32)


# ------------------------------------------------------------------ BF16 (dequantized backward)

def test_dequantized_backward_dgrad_config2():
    """dX = dY * DQ(Q(W)): the BF16 operand is the library's own dequantized
    16x16 weight (bit-equal to the oracle's), read transposed."""
    m = mxq()
    d = synth.config2()
    say("dequantized-backward DGRAD config-2 4096x2048x768")
    cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(d["w"]), block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
    wdq = m.mx_dequantize(m.Format.NVFP4, cw, sw, 768, 2048, block=m.Block.TILE, gscales=Sw,
                          gs=m.GScale.PER_TENSOR)
    ref_dq = ON.dequantize_bf16(to_np(cw), to_np(sw), to_np(Sw), "16x16", "per_tensor")
    assert np.array_equal(from_dev_bf16(wdq), ref_dq)
    dyd = to_dev_bf16(d["dy"])
    dx = m.mx_gemm(m.Operand(m.Format.BF16, dyd, block=m.Block.NONE),
                   m.Operand(m.Format.BF16, wdq, block=m.Block.NONE, transposed=True), 4096, 2048, 768)
    a = F.bf16_bits_to_f64(d["dy"])
    b = F.bf16_bits_to_f64(ref_dq).T.copy()
    _assert_gemm(dx, a, b, a, b)


def test_bf16_gemm_ragged_both_orientations():
    m = mxq()
    M, N, K = 70, 56, 72
    a = _bf16((M, K), 1.0, 16)
    b = _bf16((N, K), 1.0, 17)
    say("bf16 GEMM ragged")
    out = m.mx_gemm(m.Operand(m.Format.BF16, to_dev_bf16(a), block=m.Block.NONE),
                    m.Operand(m.Format.BF16, to_dev_bf16(b), block=m.Block.NONE), M, N, K)
    av, bv = F.bf16_bits_to_f64(a), F.bf16_bits_to_f64(b)
    _assert_gemm(out, av, bv, av, bv)
    bt = np.ascontiguousarray(b.T)                 # stored [K, N]
    out2 = m.mx_gemm(m.Operand(m.Format.BF16, to_dev_bf16(a), block=m.Block.NONE),
                     m.Operand(m.Format.BF16, to_dev_bf16(bt), block=m.Block.NONE, transposed=True),
                     M, N, K)
    assert np.array_equal(from_dev_bf16(out2), from_dev_bf16(out))


def test_gemm_is_deterministic():
    m = mxq()
    x = _bf16((512, 1024), 1.0, 18)
    w = _bf16((256, 1024), 0.02, 19)
    say("GEMM determinism")
    A, B, _, _ = _nv_ops(m, x, w, True)
    o1 = from_dev_bf16(m.mx_gemm(A, B, 512, 256, 1024))
    o2 = from_dev_bf16(m.mx_gemm(A, B, 512, 256, 1024))
    assert np.array_equal(o1, o2)


def _path_operands(m, path, bt, x, w):
    """A (rowwise x) and B (w [N, K]; stored [K, N] and read transposed when
    bt) on the GPU for one path, with the oracle's float64 / binary32
    dequantized copies of both as [M, K] and [N, K]."""
    wt = np.ascontiguousarray(w.T)                   # stored [K, N] for the transposed case
    if path == "mxfp8":
        cx, sx = m.mx_quantize(to_dev_bf16(x))
        a64 = OM.dequantize_f64(to_np(cx), to_np(sx))
        A = m.Operand(m.Format.MXFP8, cx, sx)
        if bt:
            cw, sw = m.mx_quantize(to_dev_bf16(wt), block=m.Block.TILE)
            B = m.Operand(m.Format.MXFP8, cw, sw, block=m.Block.TILE, transposed=True)
            b64 = OM.dequantize_f64(to_np(cw), to_np(sw), "32x32").T.copy()
        else:
            cw, sw = m.mx_quantize(to_dev_bf16(w))
            B = m.Operand(m.Format.MXFP8, cw, sw)
            b64 = OM.dequantize_f64(to_np(cw), to_np(sw))
        a32, b32 = a64, b64
    elif path == "nvfp4":
        cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
        A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
        a64 = ON.dequantize_f64(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
        a32 = ON.dequantize_f32(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
        src = wt if bt else w
        cw, sw, Sw = m.nvfp4_quantize(to_dev_bf16(src), block=m.Block.TILE, gs=m.GScale.PER_TENSOR)
        B = m.Operand(m.Format.NVFP4, cw, sw, Sw, block=m.Block.TILE, gs=m.GScale.PER_TENSOR, transposed=bt)
        b64 = ON.dequantize_f64(to_np(cw), to_np(sw), to_np(Sw), "16x16", "per_tensor")
        b32 = ON.dequantize_f32(to_np(cw), to_np(sw), to_np(Sw), "16x16", "per_tensor")
        if bt:
            b64, b32 = b64.T.copy(), b32.T.copy()
    else:
        A = m.Operand(m.Format.BF16, to_dev_bf16(x), block=m.Block.NONE)
        B = m.Operand(m.Format.BF16, to_dev_bf16(wt if bt else w), block=m.Block.NONE, transposed=bt)
        a64 = a32 = F.bf16_bits_to_f64(x)
        b64 = b32 = F.bf16_bits_to_f64(w)
    return A, B, (a64, a32, b64, b32)


@pytest.mark.parametrize("path", ["mxfp8", "nvfp4", "bf16"])
@pytest.mark.parametrize("bt", [False, True])
@pytest.mark.parametrize("K", [256, 288])
def test_gemm_large_tile_variants(path, bt, K):
    """M = N = 4096 selects the largest tiles (256x256, or 256x128 for MXFP8);
    checked on 256 sampled rows spread over every m-tile, all columns.  K = 288
    ends on half a stage (and, for MXFP8, a scale count that is not a multiple
    of four words), so the loaders' ragged-K paths run on these tiles too."""
    m = mxq()
    M, N = 4096, 4096
    x = _bf16((M, K), 1.0, 40)
    w = _bf16((N, K), 0.02, 41)
    say(f"large-tile GEMM {path} bt={bt} {M}x{N}x{K}")
    rows = np.sort(np.random.default_rng(42).choice(M, 256, replace=False))
    A, B, (a64, a32, b64, b32) = _path_operands(m, path, bt, x, w)
    out = from_dev_bf16(m.mx_gemm(A, B, M, N, K))
    frob, worst, ok = G.check(out[rows], a64[rows], b64, a32[rows], b32)
    assert ok, f"frobenius {frob:.3e}, worst {worst:.3f}"


@pytest.mark.parametrize("path", ["mxfp8", "nvfp4", "bf16"])
@pytest.mark.parametrize("bt", [False, True])
@pytest.mark.parametrize("K", [320, 384])
def test_every_tile_configuration_gives_the_same_bits(path, bt, K):
    """All nine workgroup tiles (forced with mx_gemm_set_tile) on one ragged
    problem: the measured default is checked against the oracle, and every
    forced tile must return the same BF16 bits (each output element sums its
    K products in the same order whatever the tile)."""
    m = mxq()
    M, N = 600, 416                                  # ragged M; N, K multiples of the 32x32 tiles
    x = _bf16((M, K), 1.0, 60)
    w = _bf16((N, K), 0.02, 61)
    A, B, (a64, a32, b64, b32) = _path_operands(m, path, bt, x, w)
    say(f"tile sweep {path} bt={bt} {M}x{N}x{K}")
    ref = m.mx_gemm(A, B, M, N, K)
    _assert_gemm(ref, a64, b64, a32, b32)
    ref = from_dev_bf16(ref)
    try:
        for t in range(9):
            m.mx_gemm_set_tile(t)
            out = from_dev_bf16(m.mx_gemm(A, B, M, N, K))
            assert np.array_equal(out, ref), f"tile {t}: {int(np.sum(out != ref))} elements differ"
    finally:
        m.mx_gemm_set_tile(-1)


@pytest.mark.parametrize("path", ["mxfp8", "nvfp4", "bf16"])
def test_every_tile_configuration_grouped(path):
    """The grouped launch (three experts, one of them empty, gathered A rows)
    under every forced tile returns the default's bits, and the default
    matches the oracle expert by expert."""
    import torch
    m = mxq()
    T, N, K, E = 300, 160, 256, 3
    off = np.array([0, 230, 230, 410], dtype=np.int32)
    M = int(off[-1])
    idx = np.random.default_rng(70).integers(0, T, M).astype(np.int32)
    x = _bf16((T, K), 1.0, 71)
    w = _bf16((E * N, K), 0.02, 72)
    say(f"grouped tile sweep {path} M={M} N={N} K={K} E={E}")
    if path == "mxfp8":
        cx, sx = m.mx_quantize(to_dev_bf16(x))
        A = m.Operand(m.Format.MXFP8, cx, sx)
        a64 = a32 = OM.dequantize_f64(to_np(cx), to_np(sx))
        cw, sw = m.mx_quantize(to_dev_bf16(w))
        B = m.Operand(m.Format.MXFP8, cw, sw)
        b64 = b32 = OM.dequantize_f64(to_np(cw), to_np(sw))
    elif path == "nvfp4":
        cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
        A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
        a64 = ON.dequantize_f64(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
        a32 = ON.dequantize_f32(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
        # one per-tensor S per expert: the grouped GEMM reads S[g] for group g
        cw = torch.empty((E * N, K // 2), dtype=torch.uint8, device="cuda")
        sw = torch.empty((E * N, K // 16), dtype=torch.uint8, device="cuda")
        Sw = torch.empty(E, dtype=torch.float32, device="cuda")
        wd = to_dev_bf16(w)
        for e in range(E):
            r = slice(e * N, (e + 1) * N)
            m.nvfp4_quantize(wd[r], gs=m.GScale.PER_TENSOR, codes=cw[r], block_scales=sw[r],
                             gscales=Sw[e:e + 1])
        B = m.Operand(m.Format.NVFP4, cw, sw, Sw, gs=m.GScale.PER_TENSOR)
        b64 = np.concatenate([ON.dequantize_f64(to_np(cw[e * N:(e + 1) * N]), to_np(sw[e * N:(e + 1) * N]),
                                                to_np(Sw[e:e + 1]), "1x16", "per_tensor") for e in range(E)])
        b32 = np.concatenate([ON.dequantize_f32(to_np(cw[e * N:(e + 1) * N]), to_np(sw[e * N:(e + 1) * N]),
                                                to_np(Sw[e:e + 1]), "1x16", "per_tensor") for e in range(E)])
    else:
        A = m.Operand(m.Format.BF16, to_dev_bf16(x), block=m.Block.NONE)
        B = m.Operand(m.Format.BF16, to_dev_bf16(w), block=m.Block.NONE)
        a64 = a32 = F.bf16_bits_to_f64(x)
        b64 = b32 = F.bf16_bits_to_f64(w)
    off_d = torch.from_numpy(off).cuda()
    idx_d = torch.from_numpy(idx).cuda()
    run = lambda: from_dev_bf16(m.mx_gemm(A, B, M, N, K, group_row_offsets=off_d,
                                          a_row_index=idx_d, a_rows=T))
    ref = run()
    for g in range(E):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            rows = idx[lo:hi]
            frob, worst, ok = G.check(ref[lo:hi], a64[rows], b64[g * N:(g + 1) * N],
                                      a32[rows], b32[g * N:(g + 1) * N])
            assert ok, f"expert {g}: frobenius {frob:.3e}, worst {worst:.3f}"
    try:
        for t in range(9):
            m.mx_gemm_set_tile(t)
            out = run()
            assert np.array_equal(out, ref), f"tile {t}: {int(np.sum(out != ref))} elements differ"
    finally:
        m.mx_gemm_set_tile(-1)


def test_grouped_many_groups_and_empty_ones():
    """600 groups (three chunks of the device-side group scan) with 0..40 rows
    each, a third of them empty, gathered A rows: every group matches the
    oracle, under the measured tile and under forced 128- and 256-row tiles."""
    import torch
    m = mxq()
    E, N, K, T = 600, 64, 64, 500
    rng = np.random.default_rng(80)
    rows = rng.integers(0, 41, E)
    rows[rng.random(E) < 0.33] = 0
    off = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    M = int(off[-1])
    idx = rng.integers(0, T, M).astype(np.int32)
    x = _bf16((T, K), 1.0, 81)
    w = _bf16((E * N, K), 0.05, 82)
    say(f"grouped GEMM with {E} groups, M={M}")
    A = m.Operand(m.Format.BF16, to_dev_bf16(x), block=m.Block.NONE)
    B = m.Operand(m.Format.BF16, to_dev_bf16(w), block=m.Block.NONE)
    off_d = torch.from_numpy(off).cuda()
    idx_d = torch.from_numpy(idx).cuda()
    x64, w64 = F.bf16_bits_to_f64(x), F.bf16_bits_to_f64(w)
    run = lambda: from_dev_bf16(m.mx_gemm(A, B, M, N, K, group_row_offsets=off_d,
                                          a_row_index=idx_d, a_rows=T))
    ref = run()
    for g in range(E):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            a = x64[idx[lo:hi]]
            b = w64[g * N:(g + 1) * N]
            frob, worst, ok = G.check(ref[lo:hi], a, b, a, b)
            assert ok, f"group {g}: frobenius {frob:.3e}, worst {worst:.3f}"
    try:
        for t in (1, 6):
            m.mx_gemm_set_tile(t)
            assert np.array_equal(run(), ref), f"tile {t}"
    finally:
        m.mx_gemm_set_tile(-1)


@pytest.mark.parametrize("M,N,K", [(256, 192, 512), (96, 160, 320)])
def test_nvfp4_gemm_mfma_scale_layout_same_bits(M, N, K):
    """NVFP4 FPROP with both operands' block scales in the MFMA layout returns
    the bits of the LINEAR-layout call (same codes, scales only moved); the
    LINEAR call is checked against the oracle.  Both the measured tile and a
    forced 256x256 tile run."""
    m = mxq()
    x = _bf16((M, K), 1.0, 90)
    w = _bf16((N, K), 0.02, 91)
    say(f"nvfp4 GEMM MFMA scale layout {M}x{N}x{K}")
    xd, wd = to_dev_bf16(x), to_dev_bf16(w)
    cx, sx, Sx = m.nvfp4_quantize(xd, gs=m.GScale.PER_ROW)
    cw, sw, Sw = m.nvfp4_quantize(wd, gs=m.GScale.PER_TENSOR)
    cxm, sxm, Sxm = m.nvfp4_quantize(xd, gs=m.GScale.PER_ROW, layout=m.Layout.MFMA)
    cwm, swm, Swm = m.nvfp4_quantize(wd, gs=m.GScale.PER_TENSOR, layout=m.Layout.MFMA)
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
    B = m.Operand(m.Format.NVFP4, cw, sw, Sw, gs=m.GScale.PER_TENSOR)
    Am = m.Operand(m.Format.NVFP4, cxm, sxm, Sxm, gs=m.GScale.PER_ROW, layout=m.Layout.MFMA)
    Bm = m.Operand(m.Format.NVFP4, cwm, swm, Swm, gs=m.GScale.PER_TENSOR, layout=m.Layout.MFMA)
    ref = m.mx_gemm(A, B, M, N, K)
    a64 = ON.dequantize_f64(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
    a32 = ON.dequantize_f32(to_np(cx), to_np(sx), to_np(Sx), "1x16", "per_row")
    b64 = ON.dequantize_f64(to_np(cw), to_np(sw), to_np(Sw), "1x16", "per_tensor")
    b32 = ON.dequantize_f32(to_np(cw), to_np(sw), to_np(Sw), "1x16", "per_tensor")
    _assert_gemm(ref, a64, b64, a32, b32)
    ref = from_dev_bf16(ref)
    assert np.array_equal(from_dev_bf16(m.mx_gemm(Am, Bm, M, N, K)), ref)
    try:
        m.mx_gemm_set_tile(6)
        assert np.array_equal(from_dev_bf16(m.mx_gemm(Am, Bm, M, N, K)), ref)
    finally:
        m.mx_gemm_set_tile(-1)


@pytest.mark.parametrize("path,K", [("mxfp8", 8192), ("nvfp4", 16384), ("bf16", 4096)])
@pytest.mark.parametrize("bt", [False, True])
def test_grouped_tile_order_with_a_ragged_last_run(path, K, bt):
    """A dense GEMM whose B (8 MB) exceeds an XCD's L2 and whose rows hold at
    most 64 tiles takes the grouped tile order: runs of 8 tile rows (128-row
    tiles) or 4 (256-row tiles) walked column by column.  M = 1100 gives 9 or
    5 tile rows, so the last run is ragged.  The default tile is compared whole
    with the oracle, and every forced tile must give the same bits."""
    m = mxq()
    M, N = 1100, 1024
    x = _bf16((M, K), 1.0, 70)
    w = _bf16((N, K), 0.02, 71)
    A, B, (a64, a32, b64, b32) = _path_operands(m, path, bt, x, w)
    say(f"grouped tile order {path} bt={bt} {M}x{N}x{K}")
    ref = m.mx_gemm(A, B, M, N, K)
    _assert_gemm(ref, a64, b64, a32, b32)
    ref = from_dev_bf16(ref)
    try:
        for t in range(9):
            m.mx_gemm_set_tile(t)
            out = from_dev_bf16(m.mx_gemm(A, B, M, N, K))
            assert np.array_equal(out, ref), f"tile {t}: {int(np.sum(out != ref))} elements differ"
    finally:
        m.mx_gemm_set_tile(-1)
