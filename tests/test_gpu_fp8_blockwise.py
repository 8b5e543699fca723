"""GPU parity of blockwise FP8 (1x128 / 128x1 / 128x128 blocks, power-of-two
scales) against oracle/fp8_blockwise.py: the quantizer byte for byte (codes
and E8M0 scales, every block kind, the TILE's transposed copy, DUAL), the
dequantizer bit for bit, and the GEMMs (FPROP, DGRAD with the weight read
transposed or through its transposed copy, WGRAD on the columnwise copies)
within the GEMM bounds of the oracle's dequantize-then-matmul; exact equality
with unit scales and small codes; every tile configuration the same bits."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import fp8_blockwise as OB
from oracle import gemm as G
from tests.util import requires_gpu, to_dev_bf16, from_dev_bf16, to_np, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def mxq():
    import microscaling_quantization_block_amd as m
    return m


def _edge(rows, cols, seed):
    """Per-row log-normal magnitudes, a zero row, negative zeros, BF16
    subnormals, the largest BF16 and random finite bit patterns."""
    rs = np.random.default_rng(seed)
    x = F.bf16_rne(rs.standard_normal((rows, cols)) * np.exp(rs.standard_normal((rows, 1)) * 3))
    x[0] = 0
    if rows > 1:
        x[1] = 0x8000
    if rows > 2:
        x[2] = rs.integers(1, 0x80, cols).astype(np.uint16)
    if rows > 3:
        x[3, 5] = 0x7F7F
        x[3, 6] = 0xFF7F
    if rows > 4:
        x[4] = (rs.integers(0, 0x7F80, cols) | (rs.integers(0, 2, cols) << 15)).astype(np.uint16)
    return x


def _v(bits):
    return F.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("shape", [(64, 512), (37, 384), (5, 128), (1000, 1024)])
def test_rows_1x128(shape):
    m = mxq()
    x = _edge(*shape, 71)
    say(f"fp8bw ROW {shape}")
    c, s = m.fp8bw_quantize(to_dev_bf16(x))
    rc, rs = OB.quantize_rows(_v(x))
    assert np.array_equal(to_np(s), rs) and np.array_equal(to_np(c), rc)
    dq = m.mx_dequantize(m.Format.FP8_B128, c, s, *shape)
    assert np.array_equal(from_dev_bf16(dq), OB.dequantize_bf16(rc, rs))


@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (384, 256), (1024, 640)])
def test_col_tile_dual(shape):
    m = mxq()
    x = _edge(*shape, 72)
    v = _v(x)
    xd = to_dev_bf16(x)
    say(f"fp8bw COL/TILE/DUAL {shape}")
    c, s = m.fp8bw_quantize(xd, block=m.Block.COL)
    rc, rs = OB.quantize_cols(v)
    assert np.array_equal(to_np(s), rs) and np.array_equal(to_np(c), rc)
    c, s = m.fp8bw_quantize(xd, block=m.Block.TILE)
    tc, ts = OB.quantize_tile(v)
    assert np.array_equal(to_np(s), ts) and np.array_equal(to_np(c), tc)
    dq = m.mx_dequantize(m.Format.FP8_B128, c, s, *shape, block=m.Block.TILE)
    assert np.array_equal(from_dev_bf16(dq), OB.dequantize_bf16(tc, ts, "128x128"))
    c, s, ct, st = m.fp8bw_quantize(xd, block=m.Block.TILE, transposed_copy=True)
    tct, tst = OB.quantize_tile(np.ascontiguousarray(v.T))
    assert np.array_equal(to_np(c), tc) and np.array_equal(to_np(s), ts)
    assert np.array_equal(to_np(ct), tct) and np.array_equal(to_np(st), tst)
    c, s, cc, sc = m.fp8bw_quantize(xd, block=m.Block.DUAL)
    r1, s1 = OB.quantize_rows(v)
    assert np.array_equal(to_np(c), r1) and np.array_equal(to_np(s), s1)
    assert np.array_equal(to_np(cc), rc) and np.array_equal(to_np(sc), rs)


def _op(m, c, s, tile=False, transposed=False):
    return m.Operand(m.Format.FP8_B128, c, s, block=m.Block.TILE if tile else m.Block.ROW,
                     transposed=transposed)


def _check(out, a64, b64):
    frob, worst, ok = G.check(from_dev_bf16(out), a64, b64, a64, b64, rtol_frob=1e-2)
    assert ok, f"frobenius {frob:.3e}, worst element ratio {worst:.3f}"


def test_fprop_dgrad_wgrad():
    m = mxq()
    T, H, I = 512, 384, 256
    rs = np.random.default_rng(73)
    x = F.bf16_rne(rs.standard_normal((T, H)) * np.exp(rs.standard_normal((T, 1))))
    w = F.bf16_rne(rs.standard_normal((I, H)) * 0.02)
    dy = F.bf16_rne(rs.standard_normal((T, I)) * 1e-3)
    say(f"fp8bw FPROP / DGRAD / WGRAD T={T} H={H} I={I}")
    cx, sx, cxc, sxc = m.fp8bw_quantize(to_dev_bf16(x), block=m.Block.DUAL)
    cw, sw, cwt, swt = m.fp8bw_quantize(to_dev_bf16(w), block=m.Block.TILE, transposed_copy=True)
    cd, sd, cdc, sdc = m.fp8bw_quantize(to_dev_bf16(dy), block=m.Block.DUAL)
    X64 = OB.dequantize_f64(*OB.quantize_rows(_v(x)))
    W64 = OB.dequantize_f64(*OB.quantize_tile(_v(w)), "128x128")
    D64 = OB.dequantize_f64(*OB.quantize_rows(_v(dy)))
    # FPROP Y = X W^T
    _check(m.mx_gemm(_op(m, cx, sx), _op(m, cw, sw, tile=True), T, I, H), X64, W64)
    # DGRAD dX = dY W: W read transposed, and its transposed copy read as is
    Wt = np.ascontiguousarray(W64.T)
    d1 = m.mx_gemm(_op(m, cd, sd), _op(m, cw, sw, tile=True, transposed=True), T, H, I)
    _check(d1, D64, Wt)
    d2 = m.mx_gemm(_op(m, cd, sd), _op(m, cwt, swt, tile=True), T, H, I)
    assert np.array_equal(from_dev_bf16(d1), from_dev_bf16(d2))
    # WGRAD dW = dY^T X on the columnwise copies
    DC = OB.dequantize_f64(*OB.quantize_cols(_v(dy)))
    XC = OB.dequantize_f64(*OB.quantize_cols(_v(x)))
    _check(m.mx_gemm(_op(m, cdc, sdc), _op(m, cxc, sxc), I, H, T), DC, XC)


def test_unit_scale_exact_and_tiles_same_bits():
    m = mxq()
    import torch
    rs = np.random.default_rng(74)
    M, N, K = 384, 256, 1024
    # codes of small integers (|v| <= 16) with unit scales: every product and
    # sum is exact, so C equals bf16(exact)
    ints = np.arange(-16, 17)
    av, bv = rs.choice(ints, (M, K)).astype(np.float64), rs.choice(ints, (N, K)).astype(np.float64)
    ca, cb = F.encode_e4m3_rne(av), F.encode_e4m3_rne(bv)
    one_a = torch.full((M, K // 128), 127, dtype=torch.uint8, device="cuda")
    one_b = torch.full((N // 128, K // 128), 127, dtype=torch.uint8, device="cuda")
    say("fp8bw unit-scale exact 384x256x1024, every tile")
    A = _op(m, torch.from_numpy(ca).cuda(), one_a)
    B = _op(m, torch.from_numpy(cb).cuda(), one_b, tile=True)
    exact = F.bf16_rne(av @ bv.T)
    outs = []
    try:
        for t in range(-1, 9):
            m.mx_gemm_set_tile(t)
            outs.append(from_dev_bf16(m.mx_gemm(A, B, M, N, K)))
    finally:
        m.mx_gemm_set_tile(-1)
    for o in outs:
        assert np.array_equal(o, exact)
    # random operands: every tile configuration gives the same bits
    x = F.bf16_rne(rs.standard_normal((M, K)))
    w = F.bf16_rne(rs.standard_normal((N, K)) * 0.05)
    cx, sx = m.fp8bw_quantize(to_dev_bf16(x))
    cw, sw = m.fp8bw_quantize(to_dev_bf16(w), block=m.Block.TILE)
    ref = None
    try:
        for t in range(-1, 9):
            m.mx_gemm_set_tile(t)
            o = from_dev_bf16(m.mx_gemm(_op(m, cx, sx), _op(m, cw, sw, tile=True), M, N, K))
            ref = o if ref is None else ref
            assert np.array_equal(o, ref), f"tile {t}"
    finally:
        m.mx_gemm_set_tile(-1)
    _check_arr = G.check(ref, OB.dequantize_f64(*OB.quantize_rows(_v(x))),
                         OB.dequantize_f64(*OB.quantize_tile(_v(w)), "128x128"),
                         OB.dequantize_f64(*OB.quantize_rows(_v(x))),
                         OB.dequantize_f64(*OB.quantize_tile(_v(w)), "128x128"))
    assert _check_arr[2]


# ------------------------------------------------------------ binary32 scales

@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (1024, 640)])
def test_f32_scales_every_block_kind(shape):
    m = mxq()
    x = _edge(*shape, 75)
    v = _v(x)
    xd = to_dev_bf16(x)
    say(f"fp8bw f32 ROW/COL/TILE/DUAL {shape}")
    c, s = m.fp8bw_quantize_f32(xd)
    rc, rs = OB.quantize_rows_f32(v)
    assert to_np(s).dtype == np.float32
    assert np.array_equal(to_np(s).view(np.uint32), rs.view(np.uint32)) and np.array_equal(to_np(c), rc)
    dq = m.mx_dequantize(m.Format.FP8_B128_F32, c, s, *shape)
    assert np.array_equal(from_dev_bf16(dq), OB.dequantize_f32s_bf16(rc, rs))
    c, s = m.fp8bw_quantize_f32(xd, block=m.Block.COL)
    cc, cs = OB.quantize_cols_f32(v)
    assert np.array_equal(to_np(s).view(np.uint32), cs.view(np.uint32)) and np.array_equal(to_np(c), cc)
    c, s, ct, st = m.fp8bw_quantize_f32(xd, block=m.Block.TILE, transposed_copy=True)
    tc, ts = OB.quantize_tile_f32(v)
    assert np.array_equal(to_np(s).view(np.uint32), ts.view(np.uint32)) and np.array_equal(to_np(c), tc)
    assert np.array_equal(to_np(ct), tc.T) and np.array_equal(to_np(st), ts.T)
    dq = m.mx_dequantize(m.Format.FP8_B128_F32, c, s, *shape, block=m.Block.TILE)
    assert np.array_equal(from_dev_bf16(dq), OB.dequantize_f32s_bf16(tc, ts, "128x128"))
    c, s, c2, s2 = m.fp8bw_quantize_f32(xd, block=m.Block.DUAL)
    assert np.array_equal(to_np(c), rc) and np.array_equal(to_np(s).view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(to_np(c2), cc) and np.array_equal(to_np(s2).view(np.uint32), cs.view(np.uint32))


def test_f32_scales_tiny_and_huge_blocks():
    """Blocks whose binary32 scale is subnormal (BF16 subnormal maxima) or
    near the top of the range, rows of any count (ROW)."""
    m = mxq()
    rs_ = np.random.default_rng(76)
    x = F.bf16_rne(rs_.standard_normal((37, 512)))
    x[:, :128] = rs_.integers(1, 0x80, (37, 128)).astype(np.uint16) | (rs_.integers(0, 2, (37, 128)) << 15).astype(np.uint16)
    x[:, 128:256] = F.bf16_rne(rs_.standard_normal((37, 128)) * 2.0 ** 120)
    x[:, 256:384] = F.bf16_rne(rs_.standard_normal((37, 128)) * 2.0 ** -125)
    say("fp8bw f32 ROW 37x512 subnormal and huge blocks")
    c, s = m.fp8bw_quantize_f32(to_dev_bf16(x))
    rc, rsc = OB.quantize_rows_f32(_v(x))
    assert np.array_equal(to_np(s).view(np.uint32), rsc.view(np.uint32))
    assert np.array_equal(to_np(c), rc)


def _opf(m, c, s, tile=False):
    return m.Operand(m.Format.FP8_B128_F32, c, s, block=m.Block.TILE if tile else m.Block.ROW)


def test_f32_scales_fprop_dgrad_wgrad():
    m = mxq()
    T, H, I = 512, 384, 256
    rs = np.random.default_rng(77)
    x = F.bf16_rne(rs.standard_normal((T, H)) * np.exp(rs.standard_normal((T, 1))))
    w = F.bf16_rne(rs.standard_normal((I, H)) * 0.02)
    dy = F.bf16_rne(rs.standard_normal((T, I)) * 1e-3)
    say(f"fp8bw f32 FPROP / DGRAD / WGRAD T={T} H={H} I={I}")
    cx, sx, cxc, sxc = m.fp8bw_quantize_f32(to_dev_bf16(x), block=m.Block.DUAL)
    cw, sw, cwt, swt = m.fp8bw_quantize_f32(to_dev_bf16(w), block=m.Block.TILE, transposed_copy=True)
    cd, sd, cdc, sdc = m.fp8bw_quantize_f32(to_dev_bf16(dy), block=m.Block.DUAL)
    X64 = OB.dequantize_f32s_f64(*OB.quantize_rows_f32(_v(x)))
    W64 = OB.dequantize_f32s_f64(*OB.quantize_tile_f32(_v(w)), "128x128")
    D64 = OB.dequantize_f32s_f64(*OB.quantize_rows_f32(_v(dy)))
    _check(m.mx_gemm(_opf(m, cx, sx), _opf(m, cw, sw, tile=True), T, I, H), X64, W64)
    _check(m.mx_gemm(_opf(m, cd, sd), _opf(m, cwt, swt, tile=True), T, H, I), D64, np.ascontiguousarray(W64.T))
    DC = OB.dequantize_f32s_f64(*OB.quantize_cols_f32(_v(dy)))
    XC = OB.dequantize_f32s_f64(*OB.quantize_cols_f32(_v(x)))
    _check(m.mx_gemm(_opf(m, cdc, sdc), _opf(m, cxc, sxc), I, H, T), DC, XC)


@pytest.mark.parametrize("M,N,K,tile_b", [(384, 256, 1024, True), (600, 416, 384, False),
                                          (130, 1, 128, False), (1, 128, 256, True),
                                          (4100, 2048, 256, True), (4096, 2050, 128, False)])
def test_f32_scales_exact_block_scaling(M, N, K, tile_b):
    """Small-integer codes with scales from {0.5, 0.75, 1, 1.25, 1.5, 2}
    per (row, K block) and per (tile, K block): every partial sum, scale
    product and accumulation is exact in binary32, so C equals the BF16
    rounding of the exact result: a wrong block index anywhere shows.
    Ragged M and N run through the tails of the tiles; the last two shapes
    take several rounds of tiles over the CUs."""
    import torch
    m = mxq()
    rs = np.random.default_rng(78 + M)
    ints = np.arange(-16, 17)
    av, bv = rs.choice(ints, (M, K)).astype(np.float64), rs.choice(ints, (N, K)).astype(np.float64)
    grid = np.array([0.5, 0.75, 1.0, 1.25, 1.5, 2.0])
    sa = rs.choice(grid, (M, K // 128)).astype(np.float32)
    sb = rs.choice(grid, ((N // 128) if tile_b else N, K // 128)).astype(np.float32)
    say(f"fp8bw f32 exact {M}x{N}x{K} tile_b={tile_b}")
    A = _opf(m, torch.from_numpy(F.encode_e4m3_rne(av)).cuda(), torch.from_numpy(sa).cuda())
    B = _opf(m, torch.from_numpy(F.encode_e4m3_rne(bv)).cuda(), torch.from_numpy(sb).cuda(), tile=tile_b)
    a64 = OB.dequantize_f32s_f64(F.encode_e4m3_rne(av), sa)
    b64 = OB.dequantize_f32s_f64(F.encode_e4m3_rne(bv), sb, "128x128" if tile_b else "1x128")
    out = from_dev_bf16(m.mx_gemm(A, B, M, N, K))
    assert np.array_equal(out, F.bf16_rne(a64 @ b64.T))


def test_f32_scales_strided_buffers():
    """Binary32-scale quantizer on a column slice of a wider BF16 tensor,
    writing into a wider code buffer; the GEMM reading row-padded operands and
    writing a column slice of a wider output (ld > cols everywhere)."""
    import torch
    m = mxq()
    rs = np.random.default_rng(79)
    R, C, W = 256, 384, 640
    full = F.bf16_rne(rs.standard_normal((R, W)) * 3)
    xd = to_dev_bf16(full)[:, 128:128 + C]
    say("fp8bw f32 strided 256x384 (ld 640) into ld 512, GEMM into a slice of ld 700")
    codes = torch.zeros((R, 512), dtype=torch.uint8, device="cuda")[:, :C]
    c, s = m.fp8bw_quantize_f32(xd, codes=codes)
    rc, rsc = OB.quantize_rows_f32(F.bf16_bits_to_f64(full[:, 128:128 + C]))
    assert np.array_equal(to_np(c), rc) and np.array_equal(to_np(s).view(np.uint32), rsc.view(np.uint32))
    wv = F.bf16_rne(rs.standard_normal((256, C)) * 0.05)
    cw, sw = m.fp8bw_quantize_f32(to_dev_bf16(wv), block=m.Block.TILE)
    out = torch.zeros((R, 700), dtype=torch.bfloat16, device="cuda")
    view = out[:, 40:40 + 256]
    m.mx_gemm(_opf(m, c, s), _opf(m, cw, sw, tile=True), R, 256, C, out=view)
    got = from_dev_bf16(view.contiguous())
    _check(view.contiguous(), OB.dequantize_f32s_f64(rc, rsc),
           OB.dequantize_f32s_f64(*OB.quantize_tile_f32(F.bf16_bits_to_f64(wv)), "128x128"))
    rest = from_dev_bf16(out)
    assert np.all(rest[:, :40] == 0) and np.all(rest[:, 296:] == 0)      # nothing outside the slice
    assert got.shape == (R, 256)


@pytest.mark.parametrize("M,N,K,b_tile", [(600, 256, 384, True), (300, 384, 640, False), (512, 512, 1152, True)])
def test_fp8bw_direct_to_lds_kernel(M, N, K, b_tile):
    """Blockwise FP8 on configuration 7 (the direct-to-LDS 256x256 kernel):
    K = 128 x odd puts a row's scale byte at every position of its word;
    ragged M and N; 128x128 weight tiles or 1x128 rows.  Same bits as the
    256x128 kernel (configuration 5), within the GEMM bound of the oracle."""
    m = mxq()
    rs = np.random.default_rng(75)
    x = F.bf16_rne(rs.standard_normal((M, K)))
    w = F.bf16_rne(rs.standard_normal((N, K)) * 0.05)
    say(f"fp8bw direct-to-LDS {M}x{N}x{K} b_tile={b_tile}")
    cx, sx = m.fp8bw_quantize(to_dev_bf16(x))
    if b_tile:
        cw, sw = m.fp8bw_quantize(to_dev_bf16(w), block=m.Block.TILE)
        b64 = OB.dequantize_f64(*OB.quantize_tile(_v(w)), "128x128")
    else:
        cw, sw = m.fp8bw_quantize(to_dev_bf16(w))
        b64 = OB.dequantize_f64(*OB.quantize_rows(_v(w)))
    a64 = OB.dequantize_f64(*OB.quantize_rows(_v(x)))
    outs = {}
    try:
        for t in (7, 5):
            m.mx_gemm_set_tile(t)
            outs[t] = from_dev_bf16(m.mx_gemm(_op(m, cx, sx), _op(m, cw, sw, tile=b_tile), M, N, K))
    finally:
        m.mx_gemm_set_tile(-1)
    assert np.array_equal(outs[7], outs[5]), f"{int(np.sum(outs[7] != outs[5]))} elements differ"
    assert G.check(outs[7], a64, b64, a64, b64)[2]
