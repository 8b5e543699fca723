"""GPU parity of the quantizers and dequantizers against the oracle: codes and
scales must be byte-identical (and DQ outputs bit-identical) on the same seeded
inputs.  Shapes: the configurations' own tensors where the oracle finishes in
seconds, ragged shapes, and edge-value tensors (zeros, signed zeros, outliers,
subnormals, the largest BF16)."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import layout as L
from oracle import mxfp8 as OM
from oracle import nvfp4 as ON
import synth
from tests.util import requires_gpu, to_dev_bf16, from_dev_bf16, to_np, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def mxq():
    import microscaling_quantization_block_amd as m
    return m


def _edge_bf16(rows, cols, seed, nvfp4=False):
    """Seeded values plus edge rows: zeros, negative zeros, tiny values (BF16
    subnormals for MXFP8; for NVFP4 values near 2^-60, inside its stated
    precondition A >= 2^-64), the largest BF16, and random bit patterns."""
    rs = np.random.default_rng(seed)
    x = rs.standard_normal((rows, cols)) * np.exp(rs.standard_normal((rows, 1)) * 3)
    x = F.bf16_rne(x)
    x[0, :] = 0                                            # zero row
    x[1, :] = 0x8000                                       # negative zeros
    if rows > 2:
        if nvfp4:
            x[2, :] = F.bf16_rne(rs.standard_normal(cols) * 2.0 ** -60)
        else:
            x[2, :] = rs.integers(1, 0x80, cols).astype(np.uint16)      # BF16 subnormals
    if rows > 3:
        x[3, 5] = 0x7F7F                                  # largest finite BF16
        x[3, 6] = 0xFF7F
    if rows > 4:
        x[4, :] = (rs.integers(0, 0x7F80, cols) | (rs.integers(0, 2, cols) << 15)).astype(np.uint16)
    return x


def _vals(bits):
    return F.bf16_bits_to_f64(bits)


# ------------------------------------------------------------------ MXFP8

@pytest.mark.parametrize("shape,seed", [((256, 512), 1), ((37, 96), 2), ((5, 32), 3), ((64, 2048), 4)])
def test_mxfp8_row_matches_oracle(shape, seed):
    m = mxq()
    x = _edge_bf16(*shape, seed) if shape[0] >= 5 else F.bf16_rne(np.random.default_rng(seed).standard_normal(shape))
    say(f"mxfp8 ROW {shape}")
    codes, scales = m.mx_quantize(to_dev_bf16(x))
    rc, rs = OM.quantize_rowwise(_vals(x))
    assert np.array_equal(to_np(codes), rc)
    assert np.array_equal(to_np(scales), rs)


def test_mxfp8_config1_with_outliers_and_dequant():
    m = mxq()
    x = synth.config1()["x"]
    say("mxfp8 config-1 X 256x512 quantize + dequantize")
    xd = to_dev_bf16(x)
    codes, scales = m.mx_quantize(xd)
    rc, rs = OM.quantize_rowwise(_vals(x))
    assert np.array_equal(to_np(codes), rc) and np.array_equal(to_np(scales), rs)
    dq = m.mx_dequantize(m.Format.MXFP8, codes, scales, 256, 512)
    assert np.array_equal(from_dev_bf16(dq), OM.dequantize_bf16(rc, rs))


def test_mxfp8_every_bf16_value_under_every_exponent():
    """All finite BF16 values as block members under all block exponents
    e = -127..119: each block's first element is 2^(e+8), fixing e, and the
    other 31 are BF16 values no larger in magnitude."""
    m = mxq()
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mags = F.bf16_bits_to_f64(allb)
    finite = np.isfinite(mags)
    blocks = []
    for e in range(-127, 120):
        lead = F.bf16_rne(np.array([2.0 ** (e + 8)]))[0]
        keep = allb[finite & (np.abs(mags) <= 2.0 ** (e + 8))]
        n = -(-len(keep) // 31)
        body = np.zeros(n * 31, dtype=np.uint16)
        body[:len(keep)] = keep
        blk = np.concatenate([np.full((n, 1), lead, dtype=np.uint16), body.reshape(n, 31)], axis=1)
        blocks.append(blk)
    x = np.concatenate(blocks)
    pad = (-len(x)) % 8
    x = np.concatenate([x, np.zeros((pad, 32), dtype=np.uint16)]).reshape(-1, 256)
    rows = x.shape[0]
    say(f"mxfp8 exhaustive element encode, {rows}x256")
    codes, scales = m.mx_quantize(to_dev_bf16(x))
    rc, rs = OM.quantize_rowwise(_vals(x))
    assert np.array_equal(to_np(scales), rs)
    assert np.array_equal(to_np(codes), rc)
    dq = m.mx_dequantize(m.Format.MXFP8, codes, scales, rows, 256)
    assert np.array_equal(from_dev_bf16(dq), OM.dequantize_bf16(rc, rs))


@pytest.mark.parametrize("shape", [(64, 96), (96, 512), (32, 32), (256, 288), (160, 416), (384, 1024)])
def test_mxfp8_col_tile_dual(shape):
    m = mxq()
    x = _edge_bf16(*shape, 11)
    v = _vals(x)
    xd = to_dev_bf16(x)
    say(f"mxfp8 COL/TILE/DUAL {shape}")
    c, s = m.mx_quantize(xd, block=m.Block.COL)
    rc, rs = OM.quantize_colwise(v)
    assert np.array_equal(to_np(c), rc) and np.array_equal(to_np(s), rs)
    c, s = m.mx_quantize(xd, block=m.Block.TILE)
    tc, ts = OM.quantize_tile32(v)
    assert np.array_equal(to_np(c), tc) and np.array_equal(to_np(s), ts)
    c, s, cc, sc = m.mx_quantize(xd, block=m.Block.DUAL)
    r1, s1 = OM.quantize_rowwise(v)
    assert np.array_equal(to_np(c), r1) and np.array_equal(to_np(s), s1)
    assert np.array_equal(to_np(cc), rc) and np.array_equal(to_np(sc), rs)
    dq = m.mx_dequantize(m.Format.MXFP8, c, s, shape[0], shape[1])
    assert np.array_equal(from_dev_bf16(dq), OM.dequantize_bf16(r1, s1))
    dqt = m.mx_dequantize(m.Format.MXFP8, *m.mx_quantize(xd, block=m.Block.TILE), shape[0], shape[1],
                          block=m.Block.TILE)
    assert np.array_equal(from_dev_bf16(dqt), OM.dequantize_bf16(tc, ts, "32x32"))
    # TILE with its transposed copy: the oracle's 32x32 quantization of x^T
    c, s, ct, st = m.mx_quantize(xd, block=m.Block.TILE, transposed_copy=True)
    tct, tst = OM.quantize_tile32(np.ascontiguousarray(v.T))
    assert np.array_equal(to_np(c), tc) and np.array_equal(to_np(s), ts)
    assert np.array_equal(to_np(ct), tct) and np.array_equal(to_np(st), tst)


def test_mxfp8_mfma_scale_layout_and_strided_input():
    m = mxq()
    import torch
    x = _edge_bf16(128, 256, 12)
    big = torch.zeros((128, 320), dtype=torch.bfloat16, device="cuda")
    big[:, :256] = to_dev_bf16(x)
    xs = big[:, :256]                                  # ld_x = 320
    say("mxfp8 MFMA layout, strided input")
    c, s = m.mx_quantize(xs, layout=m.Layout.MFMA)
    rc, rs = OM.quantize_rowwise(_vals(x))
    assert np.array_equal(to_np(c), rc)
    assert np.array_equal(to_np(s).reshape(-1), L.linear_to_mfma(rs))
    c, s, cc, sc = m.mx_quantize(xs, block=m.Block.DUAL, layout=m.Layout.MFMA)
    cr, sr = OM.quantize_colwise(_vals(x))
    assert np.array_equal(to_np(sc).reshape(-1), L.linear_to_mfma(sr))
    dq = m.mx_dequantize(m.Format.MXFP8, c, s, 128, 256, layout=m.Layout.MFMA)
    assert np.array_equal(from_dev_bf16(dq), OM.dequantize_bf16(rc, rs))


# ------------------------------------------------------------------ NVFP4

def _nv_check_row(m, x, gs, rnd="rne", seed=0, layout=0, S_given=None, tag=0):
    v = _vals(x)
    import torch
    kw = dict(gs=gs, rnd=m.Round.SR if rnd == "sr" else m.Round.RNE, seed=seed, tensor_tag=tag,
              layout=layout)
    if gs == m.GScale.GIVEN:
        kw["gscales"] = torch.tensor([S_given], dtype=torch.float32, device="cuda")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), **kw)
    og = {m.GScale.PER_ROW: "per_row", m.GScale.PER_TENSOR: "per_tensor", m.GScale.GIVEN: "given"}[gs]
    rc, rs, rS = ON.quantize_rowwise(v, og, rnd=rnd, seed=seed, stream_id=0, tensor_tag=tag,
                                     S_given=S_given)
    assert np.array_equal(to_np(S), rS)
    sb = to_np(s).reshape(-1) if layout == 0 else L.mfma_to_linear(to_np(s).reshape(-1), *rs.shape)
    assert np.array_equal(sb.reshape(rs.shape), rs)
    assert np.array_equal(to_np(c), rc)
    return c, s, S, rc, rs, rS


@pytest.mark.parametrize("shape", [(64, 2048), (33, 48), (7, 16), (16, 768), (4, 8192), (2, 16384)])
def test_nvfp4_row_per_token(shape):
    m = mxq()
    x = _edge_bf16(*shape, 21, nvfp4=True) if shape[0] >= 5 else F.bf16_rne(np.random.default_rng(5).standard_normal(shape) * 3)
    say(f"nvfp4 ROW per-row {shape}")
    c, s, S, rc, rs, rS = _nv_check_row(m, x, m.GScale.PER_ROW)
    dq = m.mx_dequantize(m.Format.NVFP4, c, s, shape[0], shape[1], gscales=S, gs=m.GScale.PER_ROW)
    assert np.array_equal(from_dev_bf16(dq), ON.dequantize_bf16(rc, rs, rS, "1x16", "per_row"))


def test_nvfp4_config2_activations_full_size():
    m = mxq()
    x = synth.config2()["x"]
    say("nvfp4 config-2 X 4096x2048 per-token")
    _nv_check_row(m, x, m.GScale.PER_ROW)


@pytest.mark.parametrize("shape", [(5000, 2048), (20000, 512), (2100, 8208)])
@pytest.mark.parametrize("gs", ["per_row", "per_tensor"])
def test_nvfp4_row_many_rows_sampled(shape, gs):
    """A row per wave; more rows than the grid's 8192 waves (each wave walks
    two or three rows); and rows longer than 8192 (the two-pass kernel).  Rows
    are independent given S, so the oracle runs on sampled rows: per row, or
    with the tensor's S (the exact binary32 amax / 2688) given."""
    m = mxq()
    R, C = shape
    x = F.bf16_rne(np.random.default_rng(31).standard_normal(shape) *
                   np.exp(np.random.default_rng(32).standard_normal((R, 1))))
    say(f"nvfp4 ROW {gs} {shape} sampled rows")
    g = m.GScale.PER_ROW if gs == "per_row" else m.GScale.PER_TENSOR
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), gs=g)
    rows = sorted({0, 1, 2047, 2048, 2049, 4095, 4096, 8191, 8192, 8193, 16383, 16384, 16385,
                   R - 2, R - 1} & set(range(R)))
    v = _vals(x[rows])
    if gs == "per_row":
        rc, rs, rS = ON.quantize_rowwise(v, "per_row")
        assert np.array_equal(to_np(S)[rows], rS)
    else:
        S_t = np.float32(np.float32(np.abs(_vals(x)).max()) / np.float32(2688.0))
        assert to_np(S)[0] == S_t
        rc, rs, rS = ON.quantize_rowwise(v, "given", S_given=S_t)
    assert np.array_equal(to_np(s)[rows], rs)
    assert np.array_equal(to_np(c)[rows], rc)


@pytest.mark.parametrize("gs", ["per_tensor", "given"])
def test_nvfp4_row_tensor_scale(gs):
    m = mxq()
    x = _edge_bf16(48, 256, 22, nvfp4=True)
    g = m.GScale.PER_TENSOR if gs == "per_tensor" else m.GScale.GIVEN
    say(f"nvfp4 ROW {gs}")
    _nv_check_row(m, x, g, S_given=np.float32(0.0123) if gs == "given" else None)


@pytest.mark.parametrize("seed,tag", [(0, 0), (12345, 7), (2 ** 40 + 3, 1)])
def test_nvfp4_row_stochastic_rounding(seed, tag):
    m = mxq()
    x = _edge_bf16(40, 512, 23, nvfp4=True)
    say(f"nvfp4 ROW SR seed={seed}")
    _nv_check_row(m, x, m.GScale.PER_ROW, rnd="sr", seed=seed, tag=tag)


@pytest.mark.parametrize("seed", [0, 7, 2 ** 33 + 5])
def test_nvfp4_sr_encoder_every_bf16_value(seed):
    """Every BF16 magnitude in [0, 6], both signs, through the stochastic
    encoder: each 16-value block leads with 6 and S = 1 is given, so s_b = 1,
    r = 1 and y = x exactly; the draws differ per element and per seed."""
    m = mxq()
    import torch
    mags = np.arange(0, 0x40C1, dtype=np.uint16)                    # BF16 0 .. 6.0
    vals = np.concatenate([mags, mags | 0x8000])
    rows = -(-len(vals) // 15)
    x = np.full(rows * 15, 0x3F80, dtype=np.uint16)                 # pad with 1.0
    x[:len(vals)] = vals
    x = x.reshape(rows, 15)
    six = np.full((rows, 1), 0x40C0, dtype=np.uint16)
    x = np.concatenate([six, x], axis=1)                             # [rows, 16]
    say(f"nvfp4 SR encoder, every BF16 value in [0, 6], seed {seed}")
    _nv_check_row(m, x, m.GScale.GIVEN, rnd="sr", seed=seed, S_given=np.float32(1.0))


def test_nvfp4_row_mfma_layout():
    m = mxq()
    x = _edge_bf16(64, 256, 24, nvfp4=True)
    say("nvfp4 ROW MFMA layout")
    c, s, S, rc, rs, rS = _nv_check_row(m, x, m.GScale.PER_ROW, layout=m.Layout.MFMA)
    dq = m.mx_dequantize(m.Format.NVFP4, c, s, 64, 256, gscales=S, gs=m.GScale.PER_ROW,
                         layout=m.Layout.MFMA)
    assert np.array_equal(from_dev_bf16(dq), ON.dequantize_bf16(rc, rs, rS, "1x16", "per_row"))


@pytest.mark.parametrize("shape,rnd", [((768, 2048), "rne"), ((48, 80), "rne"), ((64, 96), "sr")])
def test_nvfp4_tile16(shape, rnd):
    m = mxq()
    x = F.bf16_rne(np.random.default_rng(25).standard_normal(shape) * 0.02)
    if shape[0] < 100:
        x = _edge_bf16(*shape, 25, nvfp4=True)
    v = _vals(x)
    say(f"nvfp4 TILE {shape} {rnd}")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), block=m.Block.TILE, gs=m.GScale.PER_TENSOR,
                               rnd=m.Round.SR if rnd == "sr" else m.Round.RNE, seed=9)
    rc, rs, rS = ON.quantize_tile16(v, rnd=rnd, seed=9)
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(c), rc)
    dq = m.mx_dequantize(m.Format.NVFP4, c, s, shape[0], shape[1], block=m.Block.TILE, gscales=S,
                         gs=m.GScale.PER_TENSOR)
    assert np.array_equal(from_dev_bf16(dq), ON.dequantize_bf16(rc, rs, rS, "16x16", "per_tensor"))
    if rnd == "rne":
        # the same copy and its dequantized BF16 copy in one pass
        c2, s2, S2, dq2 = m.nvfp4_quantize_dq(to_dev_bf16(x))
        assert np.array_equal(to_np(c2), rc) and np.array_equal(to_np(s2), rs) and np.array_equal(to_np(S2), rS)
        assert np.array_equal(from_dev_bf16(dq2), from_dev_bf16(dq))


@pytest.mark.parametrize("shape,rnd", [((64, 96), "rne"), ((48, 32), "sr"), ((256, 512), "sr")])
def test_nvfp4_col(shape, rnd):
    m = mxq()
    x = _edge_bf16(*shape, 26, nvfp4=True)
    v = _vals(x)
    say(f"nvfp4 COL {shape} {rnd}")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), block=m.Block.COL, gs=m.GScale.PER_TENSOR,
                               rnd=m.Round.SR if rnd == "sr" else m.Round.RNE, seed=5, stream_id=1)
    rc, rs, rS = ON.quantize_colwise(v, rnd=rnd, seed=5, stream_id=1)
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(c), rc)


def test_quantizers_are_deterministic():
    m = mxq()
    x = to_dev_bf16(_edge_bf16(128, 1024, 27, nvfp4=True))
    say("determinism: run twice")
    a = [to_np(t) for t in m.nvfp4_quantize(x, rnd=m.Round.SR, seed=3)]
    b = [to_np(t) for t in m.nvfp4_quantize(x, rnd=m.Round.SR, seed=3)]
    assert all(np.array_equal(p, q) for p, q in zip(a, b))
    a = [to_np(t) for t in m.mx_quantize(x, block=m.Block.DUAL)]
    b = [to_np(t) for t in m.mx_quantize(x, block=m.Block.DUAL)]
    assert all(np.array_equal(p, q) for p, q in zip(a, b))


def test_swiglu_close_to_reference():
    m = mxq()
    from oracle import moe
    rs = np.random.default_rng(28)
    gu = F.bf16_rne(rs.standard_normal((64, 2 * 96)) * 2)
    say("swiglu 64x96")
    h = from_dev_bf16(m.mx_swiglu(to_dev_bf16(gu), 96))
    ref = moe.swiglu_f64(gu, 96)
    a, b = F.bf16_bits_to_f64(h), F.bf16_bits_to_f64(ref)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-30)


@pytest.mark.parametrize("cols", [8208, 16384, 20000, 32768, 32784])
@pytest.mark.parametrize("rnd", ["rne", "sr", "4over6"])
def test_nvfp4_long_rows(cols, rnd):
    """Rows past 8192 values: one workgroup per row with the row in registers
    (up to 16384 values with 8 chunks per thread, up to 32768 with 16, chunk
    counts that do not fill the last pass), and the two-pass kernel beyond."""
    m = mxq()
    from oracle import four_over_six as O46
    x = _edge_bf16(6, cols, 33, nvfp4=True)
    v = _vals(x)
    R = {"rne": m.Round.RNE, "sr": m.Round.SR, "4over6": m.Round.RNE_4OVER6}[rnd]
    say(f"nvfp4 ROW long rows 6x{cols} {rnd}")
    c, s, S = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW, rnd=R, seed=4)
    if rnd == "4over6":
        rc, rs, rS = O46.quantize_rowwise(v, "per_row")
    else:
        rc, rs, rS = ON.quantize_rowwise(v, "per_row", rnd=rnd, seed=4)
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(c), rc)


@pytest.mark.parametrize("shape,rnd", [((768, 2048), "rne"), ((48, 80), "rne"), ((64, 96), "sr"),
                                       ((96, 1040), "4over6"), ((4096, 14336), "rne")])
def test_nvfp4_tile16_with_transposed_copy(shape, rnd):
    """The 16x16 copy and, from the same pass, the transposed copy: equal to
    the oracle's 16x16 quantization of x^T (the codes and the tile scales
    transposed), with the plain copy unchanged."""
    m = mxq()
    from oracle import four_over_six as O46
    x = F.bf16_rne(np.random.default_rng(34).standard_normal(shape) * 0.02)
    if shape[0] < 100:
        x = _edge_bf16(*shape, 34, nvfp4=True)
    v = _vals(x)
    R = {"rne": m.Round.RNE, "sr": m.Round.SR, "4over6": m.Round.RNE_4OVER6}[rnd]
    say(f"nvfp4 TILE with transposed copy {shape} {rnd}")
    c, s, ct, st, S = m.nvfp4_quantize_tile_t(to_dev_bf16(x), rnd=R, seed=6)
    if rnd == "4over6":
        rc, rs, rS = O46.quantize_tile16(v)
        tc, ts, tS = O46.quantize_tile16(np.ascontiguousarray(v.T))
    else:
        rc, rs, rS = ON.quantize_tile16(v, rnd=rnd, seed=6)
        tc, ts, tS = ON.unpack_nibbles(rc).T, rs.T, rS          # the copy of x^T: transposed codes
        tc = ON.pack_nibbles(np.ascontiguousarray(tc))
        if rnd == "rne":
            oc, os_, oS = ON.quantize_tile16(np.ascontiguousarray(v.T))
            assert np.array_equal(oc, tc) and np.array_equal(os_, ts) and np.array_equal(oS, tS)
    assert np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(s), rs) and np.array_equal(to_np(c), rc)
    assert np.array_equal(to_np(st), ts) and np.array_equal(to_np(ct), tc)


@pytest.mark.parametrize("shape", [(48, 256), (64, 2048), (32, 8208), (16, 32784), (96, 1024)])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_nvfp4_rowcol_equals_the_two_copies(shape, rnd):
    """nvfp4_quantize_rowcol gives exactly the ROW per-token copy (stream 0)
    and the COL per-tensor copy (stream 1) of separate calls, whichever row
    kernel runs (one wave per row, one workgroup per row, two passes), and
    both copies equal the oracle's; the MFMA scale layout as well."""
    m = mxq()
    x = _edge_bf16(*shape, 35, nvfp4=True)
    v = _vals(x)
    xd = to_dev_bf16(x)
    R = m.Round.SR if rnd == "sr" else m.Round.RNE
    lays = [m.Layout.LINEAR] + ([m.Layout.MFMA] if shape[0] % 64 == 0 and shape[1] % 64 == 0 else [])
    for lay in lays:
        say(f"nvfp4 rowcol {shape} {rnd} layout {int(lay)}")
        c, s, S, cc, sc, Sc = m.nvfp4_quantize_rowcol(xd, rnd=R, seed=8, layout=lay)
        c1, s1, S1 = m.nvfp4_quantize(xd, gs=m.GScale.PER_ROW, rnd=R, seed=8, stream_id=0, layout=lay)
        c2, s2, S2 = m.nvfp4_quantize(xd, block=m.Block.COL, gs=m.GScale.PER_TENSOR, rnd=R, seed=8, stream_id=1,
                                      layout=lay)
        for a, b in ((c, c1), (s, s1), (S, S1), (cc, c2), (sc, s2), (Sc, S2)):
            assert np.array_equal(to_np(a), to_np(b))
    rc, rs, rS = ON.quantize_rowwise(v, "per_row", rnd=rnd, seed=8, stream_id=0)
    cc_, cs_, cS_ = ON.quantize_colwise(v, rnd=rnd, seed=8, stream_id=1)
    c, s, S, cc, sc, Sc = m.nvfp4_quantize_rowcol(xd, rnd=R, seed=8)
    assert np.array_equal(to_np(c), rc) and np.array_equal(to_np(s), rs) and np.array_equal(to_np(S), rS)
    assert np.array_equal(to_np(cc), cc_) and np.array_equal(to_np(sc), cs_) and np.array_equal(to_np(Sc), cS_)
