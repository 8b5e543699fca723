"""The C ABI without a GPU: the library loads, exports every function that
include/mxq.h declares, and rejects invalid arguments on the host with the
documented status before anything is launched (no compute call is made)."""

import ctypes
import os
import re

import pytest

from tests.util import ROOT

HEADER = os.path.join(ROOT, "include", "mxq.h")


def _lib():
    import microscaling_quantization_block_amd as m
    # tests/test_host_sanitizers.py reruns this file against a host-only
    # build of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
    sanitized = os.environ.get("MXQ_TEST_SANITIZED_LIBRARY")
    if sanitized:
        m.library_path = sanitized
    if not os.path.exists(m.library_path):
        pytest.skip("libmxq.so not built (run __graft_entry__.build())")
    return m, m.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ("mx_quantize", "nvfp4_quantize", "nvfp4_quantize_dq", "nvfp4_quantize_tile_t",
                 "nvfp4_quantize_rht", "nvfp4_quantize_rowcol", "fp8bw_quantize",
                 "fp8bw_quantize_f32", "mx_dequantize",
                 "mx_gemm", "mx_gemm_swiglu", "mx_gemm_swiglu_nvfp4",
                 "mx_swiglu", "mxq_status_str", "mxq_last_error", "mxq_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    _, L = _lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    _, L = _lib()
    assert L.mxq_version() == 1
    for s in range(6):
        assert L.mxq_status_str(s)
    assert b"unknown" in L.mxq_status_str(99)


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p(0x10008)


def _err(L):
    return L.mxq_last_error().decode()


def test_mx_quantize_rejects_bad_arguments():
    m, L = _lib()
    B, Lay = m.Block, m.Layout
    assert L.mx_quantize(None, 32, 64, 64, B.ROW, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 1
    assert L.mx_quantize(FAKE, 32, 48, 48, B.ROW, Lay.LINEAR, FAKE, 48, FAKE, None, 0, None, None) == 2
    assert "cols % 32" in _err(L)
    assert L.mx_quantize(FAKE, 40, 64, 64, B.COL, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 2
    assert L.mx_quantize(FAKE_ODD, 32, 64, 64, B.ROW, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 3
    assert L.mx_quantize(FAKE, 32, 64, 64, B.TILE, Lay.MFMA, FAKE, 64, FAKE, None, 0, None, None) == 4
    assert L.mx_quantize(FAKE, 32, 64, 64, B.DUAL, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 1
    assert L.mx_quantize(FAKE, -1, 64, 64, B.ROW, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 1
    assert L.mx_quantize(FAKE, 32, 64, 32, B.ROW, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 1
    assert L.mx_quantize(FAKE, 32, 64, 64, 9, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 1
    # empty input: nothing to do, nothing launched
    assert L.mx_quantize(FAKE, 0, 64, 64, B.ROW, Lay.LINEAR, FAKE, 64, FAKE, None, 0, None, None) == 0


def test_nvfp4_quantize_rejects_bad_arguments():
    m, L = _lib()
    B, G, R, Lay = m.Block, m.GScale, m.Round, m.Layout
    call = lambda *a: L.nvfp4_quantize(*a)
    assert call(FAKE, 16, 24, 24, B.ROW, G.PER_ROW, R.RNE, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE, FAKE, None) == 2
    assert call(FAKE, 16, 32, 32, B.COL, G.PER_ROW, R.RNE, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE, FAKE, None) == 4
    assert "per-row" in _err(L)
    assert call(FAKE, 16, 32, 32, B.TILE, G.PER_ROW, R.RNE, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE, FAKE, None) == 4
    assert call(FAKE, 16, 32, 32, B.DUAL, G.PER_TENSOR, R.RNE, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE, FAKE, None) == 4
    assert call(FAKE, 24, 32, 32, B.TILE, G.PER_TENSOR, R.RNE, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE, FAKE, None) == 2
    assert call(FAKE, 16, 32, 32, B.ROW, G.PER_ROW, R.RNE, 0, 0, 0, Lay.LINEAR, FAKE, 20, FAKE, FAKE, None) == 3
    assert call(FAKE, 16, 32, 32, B.ROW, G.PER_ROW, R.RNE, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE, None, None) == 1
    assert call(FAKE, 16, 32, 32, B.ROW, G.PER_ROW, 7, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE, FAKE, None) == 1
    # Four-Over-Six: ROW and TILE only
    assert call(FAKE, 16, 32, 32, B.COL, G.PER_TENSOR, R.RNE_4OVER6, 0, 0, 0, Lay.LINEAR, FAKE, 16, FAKE,
                FAKE, None) == 4
    assert "Four-Over-Six" in _err(L)


def test_nvfp4_quantize_dq_rejects_bad_arguments():
    m, L = _lib()
    G, R = m.GScale, m.Round
    call = lambda gs, rnd=R.RNE, dq=FAKE, ld_dq=32, rows=32, x=FAKE: \
        L.nvfp4_quantize_dq(x, rows, 32, 32, gs, rnd, FAKE, 16, FAKE, FAKE, dq, ld_dq, None)
    assert call(G.PER_TENSOR, rnd=R.SR) == 4
    assert call(G.PER_ROW) == 4                       # a tiled copy takes a per-tensor scale
    assert call(G.PER_TENSOR, dq=None) == 1
    assert call(G.PER_TENSOR, ld_dq=16) == 1
    assert call(G.PER_TENSOR, dq=FAKE_ODD) == 3
    assert call(G.PER_TENSOR, rows=24) == 2
    assert call(G.PER_TENSOR, x=FAKE_ODD) == 3


def test_nvfp4_quantize_tile_t_rejects_bad_arguments():
    m, L = _lib()
    G, R = m.GScale, m.Round
    call = lambda gs=G.PER_TENSOR, ct=FAKE, ldt=16, st=FAKE, rows=32, cols=32, x=FAKE: \
        L.nvfp4_quantize_tile_t(x, rows, cols, cols, gs, R.RNE, 0, 0, 0, FAKE, 16, FAKE, ct, ldt, st, FAKE, None)
    assert call(ct=None) == 1
    assert call(st=None) == 1
    assert call(ldt=8) == 1                            # shorter than rows / 2
    assert call(ldt=20) == 3                           # not a multiple of 8
    assert call(ct=ctypes.c_void_p(0x10004)) == 3      # not 8-byte aligned
    assert call(gs=G.PER_ROW) == 4                    # a tiled copy takes a per-tensor scale
    assert call(rows=24) == 2
    assert call(rows=0) == 0 and call(rows=0, ct=None) == 0


def test_nvfp4_quantize_rowcol_rejects_bad_arguments():
    m, L = _lib()
    R, Lay = m.Round, m.Layout
    G1, G2 = ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000)
    call = lambda rows=32, cols=32, rnd=R.RNE, lay=Lay.LINEAR, ldc=16, ldcc=16, g=G1, gc=G2, x=FAKE, cc=FAKE: \
        L.nvfp4_quantize_rowcol(x, rows, cols, cols, rnd, 0, 0, lay, FAKE, ldc, FAKE, g, cc, ldcc, FAKE, gc, None)
    assert call(rnd=R.RNE_4OVER6) == 4
    assert call(rnd=7) == 1
    assert call(lay=5) == 1
    assert call(cc=None) == 1 and call(gc=None) == 1
    assert call(rows=24) == 2 and call(cols=40) == 2
    assert call(lay=Lay.MFMA) == 2                    # MFMA layout of both copies: multiples of 64
    assert call(ldcc=8) == 1                           # shorter than rows / 2
    assert call(x=FAKE_ODD) == 3 and call(ldcc=20) == 3
    assert call(gc=G1) == 1                            # the tensor scale must not alias the row scales
    assert call(rows=0) == 0


def test_nvfp4_quantize_rht_rejects_bad_arguments():
    m, L = _lib()
    G, R, Lay = m.GScale, m.Round, m.Layout
    call = lambda rows, cols, mask, gs, rnd=R.RNE, lay=Lay.LINEAR, ldc=16, x=FAKE, g=FAKE: \
        L.nvfp4_quantize_rht(x, rows, cols, cols, mask, gs, rnd, 0, 1, 0, lay, FAKE, ldc, FAKE, g, None)
    assert call(32, 32, 0x10000, G.PER_TENSOR) == 1
    assert "sign_mask" in _err(L)
    assert call(32, 32, 0x1234, G.PER_ROW) == 4
    assert call(32, 32, 0x1234, G.NONE) == 1
    assert call(24, 32, 0x1234, G.PER_TENSOR) == 2
    assert call(32, 24, 0x1234, G.PER_TENSOR) == 2
    assert call(32, 32, 0x1234, G.PER_TENSOR, rnd=5) == 1
    assert call(32, 32, 0x1234, G.PER_TENSOR, rnd=R.RNE_4OVER6) == 4
    assert call(32, 32, 0x1234, G.PER_TENSOR, lay=Lay.MFMA) == 2          # rows % 64
    assert call(32, 32, 0x1234, G.PER_TENSOR, ldc=8) == 1                 # ld_codes < rows/2
    assert call(32, 32, 0x1234, G.PER_TENSOR, x=FAKE_ODD) == 3
    assert call(32, 32, 0x1234, G.PER_TENSOR, g=None) == 1
    assert call(0, 32, 0x1234, G.PER_TENSOR) == 0                         # empty: nothing launched


def test_fp8bw_quantize_rejects_bad_arguments():
    m, L = _lib()
    B = m.Block
    call = lambda x, rows, cols, ld, blk, cc=None: L.fp8bw_quantize(x, rows, cols, ld, blk, FAKE, cols, FAKE,
                                                                   cc, rows, FAKE if cc else None, None)
    assert call(FAKE, 128, 96, 96, B.ROW) == 2                    # cols % 128
    assert "cols % 128" in _err(L)
    assert call(FAKE, 96, 128, 128, B.COL) == 2                   # rows % 128 for COL
    assert call(FAKE, 128, 128, 128, B.DUAL) == 1                 # DUAL needs the second copy
    assert call(FAKE_ODD, 128, 128, 128, B.ROW) == 3
    assert call(None, 128, 128, 128, B.ROW) == 1
    assert call(FAKE, 128, 128, 128, 9) == 1
    assert call(FAKE, 0, 128, 128, B.ROW) == 0


def test_fp8bw_quantize_f32_rejects_bad_arguments():
    m, L = _lib()
    B = m.Block
    odd4 = ctypes.c_void_p(0x10002)                 # not 4-byte aligned
    call = lambda rows, cols, blk, sc=FAKE, cc=None, scc=None: L.fp8bw_quantize_f32(
        FAKE, rows, cols, cols, blk, FAKE, cols if blk != B.COL else rows, sc, cc, rows, scc, None)
    assert call(128, 96, B.ROW) == 2 and "fp8bw_quantize_f32" in _err(L)
    assert call(96, 128, B.TILE) == 2
    assert call(128, 128, B.ROW, sc=odd4) == 3 and "4-byte" in _err(L)
    assert call(128, 128, B.DUAL, cc=FAKE, scc=odd4) == 3
    assert call(128, 128, B.DUAL) == 1                # DUAL needs the second copy
    assert call(128, 128, B.ROW, sc=None) == 1
    assert call(0, 128, B.ROW) == 0


def test_mx_gemm_rejects_bad_arguments():
    m, L = _lib()
    F, B, G = m.Format, m.Block, m.GScale
    Op = m._Operand

    def op(fmt, block=B.ROW, gs=G.NONE, ld=64, transposed=0, scales=FAKE.value, gsc=FAKE.value):
        return Op(fmt, FAKE.value, scales, gsc, block, gs, 0, ld, transposed)

    def gemm(a, b, M=32, N=32, K=64):
        return L.mx_gemm(ctypes.byref(a), ctypes.byref(b), M, N, K, M, FAKE, N, 0, None, None, None)

    assert gemm(op(F.MXFP8), op(F.NVFP4, gs=G.PER_TENSOR)) == 4          # mixed formats
    assert "formats differ" in _err(L)
    assert gemm(op(F.MXFP8), op(F.MXFP8), K=48) == 2                    # K % 32
    assert gemm(op(F.NVFP4, gs=G.PER_ROW), op(F.NVFP4, gs=G.PER_ROW)) == 4   # per-row S on B
    assert gemm(op(F.MXFP8), op(F.MXFP8, transposed=1)) == 4            # transposed needs TILE
    assert gemm(op(F.MXFP8, transposed=1), op(F.MXFP8)) == 4            # A transposed
    assert gemm(op(F.MXFP8, block=B.TILE), op(F.MXFP8)) == 4            # tile A
    assert gemm(op(F.MXFP8), op(F.MXFP8, scales=None)) == 1
    assert gemm(op(F.NVFP4, gs=G.PER_ROW, gsc=None), op(F.NVFP4, gs=G.PER_TENSOR)) == 1
    assert gemm(op(F.MXFP8, ld=40), op(F.MXFP8)) == 3
    assert gemm(op(F.BF16, block=B.NONE), op(F.BF16, block=B.NONE, ld=36)) == 3
    assert gemm(op(F.MXFP8), op(F.MXFP8, block=B.TILE, transposed=1), N=48) == 2
    # empty GEMM: no launch
    assert gemm(op(F.MXFP8), op(F.MXFP8), M=0) == 0
    # blockwise FP8: K % 128, linear scales
    assert gemm(op(F.FP8_B128), op(F.FP8_B128, block=B.TILE), K=64) == 2
    # blockwise FP8 with binary32 scales: dense, as stored, aligned scales
    f32 = lambda **k: op(F.FP8_B128_F32, ld=128, **k)
    assert gemm(f32(), f32(), K=64) == 2                                 # K % 128
    assert gemm(f32(), op(F.FP8_B128, ld=128), K=128) == 4              # mixed formats
    assert gemm(f32(), f32(transposed=1), K=128) == 4                   # read as stored
    assert gemm(f32(), f32(block=B.TILE), K=128) == 2                   # TILE needs N % 128
    assert gemm(f32(), f32(scales=0x10002), K=128) == 3                 # scale alignment
    assert gemm(f32(), f32(scales=None), K=128) == 1
    assert gemm(f32(gs=G.PER_TENSOR), f32(), K=128) == 4
    assert L.mx_gemm(ctypes.byref(f32()), ctypes.byref(f32()), 32, 32, 128, 32, FAKE, 32, 1, FAKE,
                     None, None) == 4                                    # grouped
    assert "dense" in _err(L)

    def fused(a, b, M=32, inter=64, K=64, ldh=64):
        return L.mx_gemm_swiglu(ctypes.byref(a), ctypes.byref(b), M, inter, K, M, FAKE, ldh, 0, None, None,
                                None)

    nv = lambda gs, **k: op(F.NVFP4, gs=gs, **k)
    assert fused(op(F.MXFP8), op(F.MXFP8)) == 4                            # NVFP4 only
    assert "NVFP4" in _err(L)
    assert fused(nv(G.PER_ROW), nv(G.PER_TENSOR), inter=96, ldh=96) == 2   # inter % 64
    assert fused(nv(G.PER_ROW), nv(G.PER_TENSOR, block=B.TILE, transposed=1)) == 4
    assert fused(nv(G.PER_ROW), nv(G.PER_TENSOR), ldh=32) == 1             # ldh < inter
    assert fused(nv(G.PER_ROW), nv(G.PER_TENSOR), inter=0) == 0            # nothing to do
    assert fused(nv(G.PER_ROW), nv(G.PER_TENSOR), inter=-64) == 1

    def fused_q(a, b, M=32, inter=256, K=64, codes=FAKE, ld_codes=128, scales=FAKE, layout=0, gsc=FAKE,
                h=None, ldh=0):
        return L.mx_gemm_swiglu_nvfp4(ctypes.byref(a), ctypes.byref(b), M, inter, K, M, codes, ld_codes, scales,
                                      layout, gsc, h, ldh, 0, None, None, None)

    A, Bw = nv(G.PER_ROW), nv(G.PER_TENSOR)
    assert fused_q(op(F.MXFP8), op(F.MXFP8)) == 4                          # NVFP4 only
    assert fused_q(A, Bw, inter=320, ld_codes=160) == 4                    # inter in {256, 512, 768}
    assert "256, 512 or 768" in _err(L)
    assert fused_q(A, Bw, codes=None) == 1                                 # outputs required
    assert fused_q(A, Bw, scales=None) == 1
    assert fused_q(A, Bw, gsc=None) == 1
    assert fused_q(A, Bw, ld_codes=64) == 1                                # row of codes: inter / 2 bytes
    assert fused_q(A, Bw, ld_codes=136) == 3                               # 16-byte rows
    assert fused_q(A, Bw, layout=1, M=48) == 2                             # MFMA layout: M % 32
    assert fused_q(A, Bw, layout=7) == 1
    assert fused_q(A, Bw, h=FAKE, ldh=260) == 3                            # h rows 16-byte aligned
    assert fused_q(A, Bw, K=96) == 2                                       # K % 64
    assert fused_q(A, Bw, M=0) == 0                                        # nothing to do


def test_dequantize_and_swiglu_reject_bad_arguments():
    m, L = _lib()
    F, B, G, Lay = m.Format, m.Block, m.GScale, m.Layout
    assert L.mx_dequantize(F.MXFP8, FAKE, 64, FAKE, None, 32, 64, B.COL, G.NONE, Lay.LINEAR, FAKE, 64, None) == 4
    assert L.mx_dequantize(F.NVFP4, FAKE, 32, FAKE, None, 32, 64, B.ROW, G.PER_ROW, Lay.LINEAR, FAKE, 64, None) == 1
    assert L.mx_dequantize(F.MXFP8, FAKE, 64, FAKE, None, 32, 64, B.ROW, G.PER_ROW, Lay.LINEAR, FAKE, 64, None) == 4
    assert L.mx_dequantize(F.BF16, FAKE, 64, FAKE, None, 32, 64, B.ROW, G.NONE, Lay.LINEAR, FAKE, 64, None) == 1
    assert L.mx_dequantize(F.FP8_B128_F32, FAKE, 128, ctypes.c_void_p(0x10002), None, 32, 128, B.ROW,
                           G.NONE, Lay.LINEAR, FAKE, 128, None) == 3     # binary32 scale alignment
    assert L.mx_dequantize(F.FP8_B128_F32, FAKE, 128, FAKE, None, 32, 96, B.ROW, G.NONE, Lay.LINEAR,
                           FAKE, 128, None) == 2
    assert L.mx_swiglu(FAKE, 4, 12, 24, FAKE, 12, None) == 2
    assert L.mx_swiglu(FAKE_ODD, 4, 16, 32, FAKE, 16, None) == 3


def test_gemm_set_tile_range():
    m, L = _lib()
    assert L.mx_gemm_set_tile(9) == 1 and "outside" in _err(L)
    assert L.mx_gemm_set_tile(-2) == 1
    assert L.mx_gemm_set_tile(-1) == 0                # the default; no device work
