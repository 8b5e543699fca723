"""GPU parity of the MoE expert path (grouped GEMMs with a row gather, joint
gate/up scale, SwiGLU, per-token requantization) against the oracle.  Each
bit-exact check feeds the oracle the GPU's own input to that stage (SwiGLU's
exp is not bit-reproducible between CPU and GPU); GEMM stages use the GEMM
tolerance."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from oracle import moe
from oracle import nvfp4 as ON
import synth
from tests.util import requires_gpu, to_dev_bf16, from_dev_bf16, to_np, say

pytestmark = [pytest.mark.gpu, requires_gpu]


def mxq():
    import microscaling_quantization_block_amd as m
    return m


def quantize_experts(m, w_bits, layout=None):
    """Per-expert NVFP4 1x16 copies with one per-tensor S each (for W_gu that
    S spans the gate/up pair), scales in `layout` (default LINEAR)."""
    import torch
    E, N, K = w_bits.shape
    codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((E, N, K // 16), dtype=torch.uint8, device="cuda")
    gs = torch.empty(E, dtype=torch.float32, device="cuda")
    wd = to_dev_bf16(w_bits.reshape(E * N, K)).view(E, N, K)
    for e in range(E):
        m.nvfp4_quantize(wd[e], gs=m.GScale.PER_TENSOR, codes=codes[e], block_scales=scales[e],
                         gscales=gs[e:e + 1], layout=m.Layout.LINEAR if layout is None else layout)
    return codes, scales, gs


def _grouped_check(out, a_rows64, a_rows32, w64, w32, off):
    c = from_dev_bf16(out)
    M = c.shape[0]
    c64 = moe.grouped_gemm_f64(a_rows64, w64, off)
    c32 = np.zeros_like(c64, dtype=np.float32)
    ap = np.zeros_like(c64)
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            c32[lo:hi] = G.gemm_f32(a_rows32[lo:hi], w32[g])
            ap[lo:hi] = G.abs_product(a_rows64[lo:hi], w64[g])
    K = a_rows64.shape[1]
    frob = G.rel_frobenius(c, c64)
    bound = G.elementwise_bound(c32, ap, K)
    diff = np.abs(F.bf16_bits_to_f64(c) - c32.astype(np.float64))
    assert frob <= 1e-2 and np.all(diff <= bound), (frob, float(np.max(diff / np.maximum(bound, 1e-300))))
    return frob


def run_moe_layer(m, d, check=True):
    import torch
    x, logits = d["x"], d["logits"]
    T, H = x.shape
    E, N2, _ = d["w_gu"].shape
    I = N2 // 2
    top = moe.route_topk(logits, d["topk"])
    row_token, off = moe.group_rows(top, E)
    M = len(row_token)
    # per-token Q(X) once; rows gathered by index inside the GEMM
    cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
    cgu, sgu, Sgu = quantize_experts(m, d["w_gu"])
    cdn, sdn, Sdn = quantize_experts(m, d["w_dn"])
    off_d = torch.from_numpy(off).cuda()
    idx_d = torch.from_numpy(row_token).cuda()
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
    Bgu = m.Operand(m.Format.NVFP4, cgu.view(E * N2, H // 2), sgu, Sgu, gs=m.GScale.PER_TENSOR)
    gu = m.mx_gemm(A, Bgu, M, N2, H, group_row_offsets=off_d, a_row_index=idx_d, a_rows=T)
    h = m.mx_swiglu(gu, I)
    if I % 64 == 0 and H % 64 == 0:
        # the gate_up GEMM with the SwiGLU in its epilogue gives the same bits
        hf = m.mx_gemm_swiglu(A, Bgu, M, I, H, group_row_offsets=off_d, a_row_index=idx_d, a_rows=T)
        assert np.array_equal(from_dev_bf16(hf), from_dev_bf16(h))
    ch, sh, Sh = m.nvfp4_quantize(h, gs=m.GScale.PER_ROW)
    Bdn = m.Operand(m.Format.NVFP4, cdn.view(E * H, I // 2), sdn, Sdn, gs=m.GScale.PER_TENSOR)
    y = m.mx_gemm(m.Operand(m.Format.NVFP4, ch, sh, Sh, gs=m.GScale.PER_ROW), Bdn, M, H, I,
                  group_row_offsets=off_d)
    if not check:
        return y
    # ---- stage checks
    rc, rs, rS = ON.quantize_rowwise(F.bf16_bits_to_f64(x), "per_row")
    assert np.array_equal(to_np(cx), rc) and np.array_equal(to_np(sx), rs)
    ax64 = ON.dequantize_f64(rc, rs, rS, "1x16", "per_row")[row_token]
    ax32 = ON.dequantize_f32(rc, rs, rS, "1x16", "per_row")[row_token]
    wgu64 = np.stack([ON.dequantize_f64(to_np(cgu[e]), to_np(sgu[e]), to_np(Sgu[e:e + 1]), "1x16", "per_tensor") for e in range(E)])
    wgu32 = np.stack([ON.dequantize_f32(to_np(cgu[e]), to_np(sgu[e]), to_np(Sgu[e:e + 1]), "1x16", "per_tensor") for e in range(E)])
    # joint gate/up scale: S over the whole [gate; up] pair of each expert
    for e in range(0, E, max(1, E // 4)):
        A_e = np.abs(F.bf16_bits_to_f64(d["w_gu"][e])).max()
        assert to_np(Sgu)[e] == np.float32(np.float32(A_e) / np.float32(2688))
    _grouped_check(gu, ax64, ax32, wgu64, wgu32, off)
    # SwiGLU within a few BF16 ulps of the float64 reference on the GPU's gate_up
    gu_bits = from_dev_bf16(gu)
    h_bits = from_dev_bf16(h)
    ref_h = F.bf16_bits_to_f64(moe.swiglu_f64(gu_bits, I))
    assert np.all(np.abs(F.bf16_bits_to_f64(h_bits) - ref_h) <= 2.0 ** -7 * np.abs(ref_h) + 1e-30)
    # per-token Q(H) bit-exact on the GPU's own H
    hc, hs, hS = ON.quantize_rowwise(F.bf16_bits_to_f64(h_bits), "per_row")
    assert np.array_equal(to_np(ch), hc) and np.array_equal(to_np(sh), hs) and np.array_equal(to_np(Sh), hS)
    ah64 = ON.dequantize_f64(hc, hs, hS, "1x16", "per_row")
    ah32 = ON.dequantize_f32(hc, hs, hS, "1x16", "per_row")
    wdn64 = np.stack([ON.dequantize_f64(to_np(cdn[e]), to_np(sdn[e]), to_np(Sdn[e:e + 1]), "1x16", "per_tensor") for e in range(E)])
    wdn32 = np.stack([ON.dequantize_f32(to_np(cdn[e]), to_np(sdn[e]), to_np(Sdn[e:e + 1]), "1x16", "per_tensor") for e in range(E)])
    _grouped_check(y, ah64, ah32, wdn64, wdn32, off)
    return y


def test_moe_small():
    m = mxq()
    d = synth.config3(tokens=256, hidden=256, experts=8, inter=64, topk=2, seed=31)
    say("moe small T=256 H=256 E=8 I=64 top-2")
    run_moe_layer(m, d)


def test_moe_empty_and_uneven_groups():
    """Some experts receive no rows, others many (skewed logits)."""
    m = mxq()
    d = synth.config3(tokens=128, hidden=128, experts=16, inter=32, topk=2, seed=32)
    d["logits"][:, :4] += 3.0          # experts 0..3 take most tokens; several get none
    say("moe skewed routing with empty groups")
    run_moe_layer(m, d)


def test_moe_gather_equals_pre_gathered():
    """Quantize-then-gather inside the GEMM equals gathering the BF16 rows
    first and quantizing them (per-token scales are batch-invariant)."""
    m = mxq()
    import torch
    rs = np.random.default_rng(33)
    x = F.bf16_rne(rs.standard_normal((64, 128)))
    w = F.bf16_rne(rs.standard_normal((1, 64, 128)) * 0.02)
    idx = rs.integers(0, 64, 96).astype(np.int32)
    off = np.array([0, 96], dtype=np.int32)
    say("moe gather invariance")
    cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
    cw, sw, Sw = quantize_experts(m, w)
    B = m.Operand(m.Format.NVFP4, cw.view(64, 64), sw, Sw, gs=m.GScale.PER_TENSOR)
    y1 = m.mx_gemm(m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW), B, 96, 64, 128,
                   group_row_offsets=torch.from_numpy(off).cuda(),
                   a_row_index=torch.from_numpy(idx).cuda(), a_rows=64)
    cg, sg, Sg = m.nvfp4_quantize(to_dev_bf16(x[idx]), gs=m.GScale.PER_ROW)
    y2 = m.mx_gemm(m.Operand(m.Format.NVFP4, cg, sg, Sg, gs=m.GScale.PER_ROW), B, 96, 64, 128,
                   group_row_offsets=torch.from_numpy(off).cuda())
    assert np.array_equal(from_dev_bf16(y1), from_dev_bf16(y2))


@pytest.mark.parametrize("I,dense", [(128, False), (192, False), (64, True), (320, True)])
def test_fused_swiglu_every_tile(I, dense):
    """mx_gemm_swiglu equals mx_swiglu(mx_gemm(...)) bit for bit under every
    workgroup tile: grouped with a gather (an empty group included) or dense;
    2I = 384 and 640 leave waves of the last tile past N."""
    import torch
    m = mxq()
    rs = np.random.default_rng(33)
    H, T = 256, 192
    E = 1 if dense else 5
    w = F.bf16_rne(rs.standard_normal((E, 2 * I, H)) * 0.05)
    x = F.bf16_rne(rs.standard_normal((T, H)))
    cw, sw, Sw = quantize_experts(m, w)
    cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
    B = m.Operand(m.Format.NVFP4, cw.view(E * 2 * I, H // 2), sw, Sw, gs=m.GScale.PER_TENSOR)
    if dense:
        kw, M = {}, T
    else:
        M = 300
        off = np.array([0, 70, 70, 171, 260, 300], dtype=np.int32)     # group 1 empty
        idx = rs.integers(0, T, M).astype(np.int32)
        kw = dict(group_row_offsets=torch.from_numpy(off).cuda(), a_row_index=torch.from_numpy(idx).cuda(),
                  a_rows=T)
    say(f"fused SwiGLU I={I} dense={dense}")
    try:
        for t in range(-1, 9):
            m.mx_gemm_set_tile(t)
            gu = m.mx_gemm(A, B, M, 2 * I, H, **kw)
            ref = from_dev_bf16(m.mx_swiglu(gu, I))
            got = from_dev_bf16(m.mx_gemm_swiglu(A, B, M, I, H, **kw))
            assert np.array_equal(got, ref), f"tile {t}"
    finally:
        m.mx_gemm_set_tile(-1)
    # and close to the float64 SwiGLU of the GPU's own gate_up (as for mx_swiglu)
    ref64 = F.bf16_bits_to_f64(moe.swiglu_f64(from_dev_bf16(gu), I))
    assert np.all(np.abs(F.bf16_bits_to_f64(got) - ref64) <= 2.0 ** -7 * np.abs(ref64) + 1e-30)


@pytest.mark.parametrize("I,K,dense,layout,tiny,b_mfma", [
    (768, 256, False, "linear", False, False),   # the config-3 width, grouped, a gather, an empty group
    (512, 320, True, "linear", False, False),    # dense, ragged M, five 64-K stages
    (256, 128, False, "mfma", False, False),     # MFMA scale layout of the Q(H) copy
    (768, 2048, False, "linear", False, True),   # the config-3 K; the weights' scales in the MFMA layout
    (256, 192, True, "linear", True, False),     # token scales below 2^-64 (the scaled frame)
])
def test_fused_swiglu_requant(I, K, dense, layout, tiny, b_mfma):
    """mx_gemm_swiglu_nvfp4 writes the bytes nvfp4_quantize(H, per-token S,
    1x16, RNE) writes for H = mx_gemm_swiglu(...), and H itself; the
    quantization of its H also equals the oracle's."""
    import torch
    m = mxq()
    rs = np.random.default_rng(37 + I + K)
    T = 160
    E = 1 if dense else 6
    w = F.bf16_rne(rs.standard_normal((E, 2 * I, K)) * 0.05)
    x = F.bf16_rne(rs.standard_normal((T, K)) * (2.0 ** -30 if tiny else 1.0))
    x[5] = 0                                                          # a token whose H row is zero
    blay = m.Layout.MFMA if b_mfma else m.Layout.LINEAR
    cw, sw, Sw = quantize_experts(m, w, blay)
    cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
    B = m.Operand(m.Format.NVFP4, cw.view(E * 2 * I, K // 2), sw, Sw, gs=m.GScale.PER_TENSOR, layout=blay)
    if dense:
        kw, M = {}, (T if layout == "mfma" else T - 3)
    else:
        M = 320 if layout == "mfma" else 300
        off = np.array([0, 64, 64, 150, 200, 263, M], dtype=np.int32)    # group 1 empty
        idx = rs.integers(0, T, M).astype(np.int32)
        idx[:3] = 5
        kw = dict(group_row_offsets=torch.from_numpy(off).cuda(), a_row_index=torch.from_numpy(idx).cuda(),
                  a_rows=T)
    lay = m.Layout.MFMA if layout == "mfma" else m.Layout.LINEAR
    say(f"fused SwiGLU + Q(H) I={I} K={K} dense={dense} layout={layout} tiny={tiny} b_mfma={b_mfma} M={M}")
    h_ref = m.mx_gemm_swiglu(A, B, M, I, K, **kw)
    cr, sr, Sr = m.nvfp4_quantize(h_ref, gs=m.GScale.PER_ROW, layout=lay)
    c, s, S, h = m.mx_gemm_swiglu_nvfp4(A, B, M, I, K, layout=lay, with_h=True, **kw)
    assert np.array_equal(from_dev_bf16(h), from_dev_bf16(h_ref))
    assert np.array_equal(to_np(S), to_np(Sr))
    assert np.array_equal(to_np(s).reshape(-1), to_np(sr).reshape(-1))
    assert np.array_equal(to_np(c), to_np(cr))
    # without H the same bytes
    c2, s2, S2 = m.mx_gemm_swiglu_nvfp4(A, B, M, I, K, layout=lay, **kw)
    assert np.array_equal(to_np(c2), to_np(c)) and np.array_equal(to_np(s2), to_np(s))
    assert np.array_equal(to_np(S2), to_np(S))
    if tiny:
        assert np.all(to_np(S)[to_np(S) > 0] < 2.0 ** -64)
    if layout == "linear":
        hc, hs, hS = ON.quantize_rowwise(F.bf16_bits_to_f64(from_dev_bf16(h)), "per_row")
        assert np.array_equal(to_np(c), hc)
        assert np.array_equal(to_np(s).reshape(M, I // 16), hs)
        assert np.array_equal(to_np(S), hS)


def test_fused_swiglu_requant_rejects_other_widths():
    import torch
    m = mxq()
    rs = np.random.default_rng(41)
    x = F.bf16_rne(rs.standard_normal((64, 128)))
    w = F.bf16_rne(rs.standard_normal((1, 2 * 320, 128)) * 0.05)
    cw, sw, Sw = quantize_experts(m, w)
    cx, sx, Sx = m.nvfp4_quantize(to_dev_bf16(x), gs=m.GScale.PER_ROW)
    A = m.Operand(m.Format.NVFP4, cx, sx, Sx, gs=m.GScale.PER_ROW)
    B = m.Operand(m.Format.NVFP4, cw.view(640, 64), sw, Sw, gs=m.GScale.PER_TENSOR)
    with pytest.raises(m.MXQError):
        m.mx_gemm_swiglu_nvfp4(A, B, 64, 320, 128)
