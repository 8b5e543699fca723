"""Python binding of libmxq, the MI355X (gfx950) microscaling quantization
library.  Argument marshalling only: every step of the hot path runs in the
library's HIP kernels.  PyTorch supplies device memory and the current stream.

The names and arguments follow the C ABI in include/mxq.h:
    mx_quantize, nvfp4_quantize, mx_dequantize, mx_gemm, mx_swiglu,
    mx_gemm_set_tile
Outputs the caller does not pass are allocated here with torch (the library
itself never allocates).  Every call is asynchronous on the current stream.

There is no fallback: if libmxq.so is missing or a call fails, this raises.
"""

import ctypes
import enum
import os

import torch

__all__ = ["Format", "Block", "GScale", "Round", "Layout", "Operand", "MXQError",
           "mx_quantize", "nvfp4_quantize", "nvfp4_quantize_dq", "nvfp4_quantize_tile_t", "nvfp4_quantize_rht",
           "nvfp4_quantize_rowcol", "fp8bw_quantize",
           "fp8bw_quantize_f32",
           "mx_dequantize", "mx_gemm", "mx_gemm_swiglu", "mx_gemm_swiglu_nvfp4",
           "mx_swiglu", "mx_gemm_set_tile", "library_path", "lib"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmxq.so")


class Format(enum.IntEnum):
    MXFP8 = 0
    NVFP4 = 1
    BF16 = 2
    FP8_B128 = 3
    FP8_B128_F32 = 4


class Block(enum.IntEnum):
    ROW = 0
    COL = 1
    TILE = 2
    DUAL = 3
    NONE = 4


class GScale(enum.IntEnum):
    NONE = 0
    PER_ROW = 1
    PER_TENSOR = 2
    GIVEN = 3


class Round(enum.IntEnum):
    RNE = 0
    SR = 1
    RNE_4OVER6 = 2


class Layout(enum.IntEnum):
    LINEAR = 0
    MFMA = 1


class MXQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class _Operand(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("gscales", ctypes.c_void_p), ("block", ctypes.c_int), ("gs", ctypes.c_int),
                ("layout", ctypes.c_int), ("ld", ctypes.c_int64), ("transposed", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libmxq (ctypes).  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(f"{library_path} is missing: build it with "
                          "`python -m microscaling_quantization_block_amd.build`")
    L = ctypes.CDLL(library_path)
    i64, u64, u32, vp, ci = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    L.mx_quantize.argtypes = [vp, i64, i64, i64, ci, ci, vp, i64, vp, vp, i64, vp, vp]
    L.fp8bw_quantize.argtypes = [vp, i64, i64, i64, ci, vp, i64, vp, vp, i64, vp, vp]
    L.fp8bw_quantize_f32.argtypes = [vp, i64, i64, i64, ci, vp, i64, vp, vp, i64, vp, vp]
    L.nvfp4_quantize.argtypes = [vp, i64, i64, i64, ci, ci, ci, u64, u32, u32, ci, vp, i64, vp, vp, vp]
    L.nvfp4_quantize_dq.argtypes = [vp, i64, i64, i64, ci, ci, vp, i64, vp, vp, vp, i64, vp]
    L.nvfp4_quantize_tile_t.argtypes = [vp, i64, i64, i64, ci, ci, u64, u32, u32, vp, i64, vp, vp, i64, vp,
                                        vp, vp]
    L.nvfp4_quantize_rowcol.argtypes = [vp, i64, i64, i64, ci, u64, u32, ci, vp, i64, vp, vp, vp, i64, vp, vp,
                                        vp]
    L.nvfp4_quantize_rht.argtypes = [vp, i64, i64, i64, u32, ci, ci, u64, u32, u32, ci, vp, i64, vp,
                                     vp, vp]
    L.mx_dequantize.argtypes = [ci, vp, i64, vp, vp, i64, i64, ci, ci, ci, vp, i64, vp]
    L.mx_gemm.argtypes = [ctypes.POINTER(_Operand), ctypes.POINTER(_Operand), i64, i64, i64, i64,
                          vp, i64, ctypes.c_int32, vp, vp, vp]
    L.mx_gemm_swiglu.argtypes = [ctypes.POINTER(_Operand), ctypes.POINTER(_Operand), i64, i64, i64, i64,
                          vp, i64, ctypes.c_int32, vp, vp, vp]
    L.mx_gemm_swiglu_nvfp4.argtypes = [ctypes.POINTER(_Operand), ctypes.POINTER(_Operand), i64, i64, i64, i64,
                                       vp, i64, vp, ctypes.c_int32, vp, vp, i64, ctypes.c_int32, vp, vp, vp]
    L.mx_swiglu.argtypes = [vp, i64, i64, i64, vp, i64, vp]
    L.mx_gemm_set_tile.argtypes = [ctypes.c_int32]
    for f in ("mx_quantize", "nvfp4_quantize", "nvfp4_quantize_dq", "nvfp4_quantize_tile_t", "nvfp4_quantize_rht",
           "nvfp4_quantize_rowcol", "fp8bw_quantize",
              "fp8bw_quantize_f32",
              "mx_dequantize", "mx_gemm", "mx_gemm_swiglu", "mx_gemm_swiglu_nvfp4", "mx_swiglu",
              "mx_gemm_set_tile"):
        getattr(L, f).restype = ci
    L.mxq_last_error.restype = ctypes.c_char_p
    L.mxq_status_str.restype = ctypes.c_char_p
    L.mxq_status_str.argtypes = [ci]
    L.mxq_version.restype = ci
    _lib = L
    return L


def _check(status):
    if status != 0:
        L = lib()
        raise MXQError(status, L.mxq_last_error().decode() or L.mxq_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_2d(x, dtype, name):
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or x.dtype != dtype or not x.is_cuda:
        raise TypeError(f"{name} must be a 2-D {dtype} CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError(f"{name} must be row-major (unit column stride)")


def _u8(shape, device):
    return torch.empty(shape, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- quantizers

def mx_quantize(x, block=Block.ROW, layout=Layout.LINEAR, codes=None, scales=None,
                codes_col=None, scales_col=None, transposed_copy=False, stream=None):
    """MXFP8 quantization of a BF16 matrix.  Returns (codes, scales) or, for
    DUAL and for TILE with transposed_copy, (codes, scales, codes_col,
    scales_col); TILE's transposed copy is the 32x32 quantization of x^T."""
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    block = Block(block)
    if block == Block.COL:
        codes = _u8((cols, rows), dev) if codes is None else codes
        scales = _u8((cols, max(rows // 32, 0)), dev) if scales is None else scales
    elif block == Block.TILE:
        codes = _u8((rows, cols), dev) if codes is None else codes
        scales = _u8((max(rows // 32, 0), cols // 32), dev) if scales is None else scales
    else:
        codes = _u8((rows, cols), dev) if codes is None else codes
        scales = _u8((rows, cols // 32), dev) if scales is None else scales
    if block == Block.DUAL:
        codes_col = _u8((cols, rows), dev) if codes_col is None else codes_col
        scales_col = _u8((cols, max(rows // 32, 0)), dev) if scales_col is None else scales_col
    elif block == Block.TILE and transposed_copy:
        codes_col = _u8((cols, rows), dev) if codes_col is None else codes_col
        scales_col = _u8((cols // 32, max(rows // 32, 0)), dev) if scales_col is None else scales_col
    else:
        codes_col = scales_col = None
    ldc = codes.stride(0)
    ldcc = codes_col.stride(0) if codes_col is not None else 0
    _check(lib().mx_quantize(_ptr(x), rows, cols, x.stride(0), int(block), int(layout), _ptr(codes),
                             ldc, _ptr(scales), _ptr(codes_col), ldcc, _ptr(scales_col), _stream(stream)))
    if codes_col is not None:
        return codes, scales, codes_col, scales_col
    return codes, scales


def _fp8bw(fn, sdt, x, block, codes, scales, codes_col, scales_col, transposed_copy, stream):
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    block = Block(block)
    u8 = lambda shape: _u8(shape, dev)
    sc = lambda shape: torch.empty(shape, dtype=sdt, device=dev)
    if block == Block.COL:
        codes = u8((cols, rows)) if codes is None else codes
        scales = sc((cols, rows // 128)) if scales is None else scales
    elif block == Block.TILE:
        codes = u8((rows, cols)) if codes is None else codes
        scales = sc((rows // 128, cols // 128)) if scales is None else scales
    else:
        codes = u8((rows, cols)) if codes is None else codes
        scales = sc((rows, cols // 128)) if scales is None else scales
    if block == Block.DUAL:
        codes_col = u8((cols, rows)) if codes_col is None else codes_col
        scales_col = sc((cols, rows // 128)) if scales_col is None else scales_col
    elif block == Block.TILE and transposed_copy:
        codes_col = u8((cols, rows)) if codes_col is None else codes_col
        scales_col = sc((cols // 128, rows // 128)) if scales_col is None else scales_col
    else:
        codes_col = scales_col = None
    ldcc = codes_col.stride(0) if codes_col is not None else 0
    _check(fn(_ptr(x), rows, cols, x.stride(0), int(block), _ptr(codes), codes.stride(0),
              _ptr(scales), _ptr(codes_col), ldcc, _ptr(scales_col), _stream(stream)))
    if codes_col is not None:
        return codes, scales, codes_col, scales_col
    return codes, scales


def fp8bw_quantize(x, block=Block.ROW, codes=None, scales=None, codes_col=None, scales_col=None,
                   transposed_copy=False, stream=None):
    """Blockwise FP8 (1x128 / 128x1 / 128x128 blocks, power-of-two scales).
    Returns (codes, scales) or, for DUAL and for TILE with transposed_copy,
    (codes, scales, codes_col, scales_col).  GEMM operands use
    Format.FP8_B128."""
    return _fp8bw(lib().fp8bw_quantize, torch.uint8, x, block, codes, scales, codes_col,
                  scales_col, transposed_copy, stream)


def fp8bw_quantize_f32(x, block=Block.ROW, codes=None, scales=None, codes_col=None,
                       scales_col=None, transposed_copy=False, stream=None):
    """Blockwise FP8 with binary32 block scales (float32 tensors of the
    shapes fp8bw_quantize gives its byte scales).  GEMM operands use
    Format.FP8_B128_F32."""
    return _fp8bw(lib().fp8bw_quantize_f32, torch.float32, x, block, codes, scales, codes_col,
                  scales_col, transposed_copy, stream)


def nvfp4_quantize(x, block=Block.ROW, gs=GScale.PER_ROW, rnd=Round.RNE, seed=0, stream_id=0,
                   tensor_tag=0, layout=Layout.LINEAR, codes=None, block_scales=None,
                   gscales=None, stream=None):
    """NVFP4 quantization.  Returns (packed codes, E4M3 block scales, FP32 S).
    For gs=GIVEN pass `gscales` holding S (a 1-element float32 CUDA tensor)."""
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    block, gs = Block(block), GScale(gs)
    if block == Block.COL:
        codes = _u8((cols, rows // 2), dev) if codes is None else codes
        block_scales = _u8((cols, rows // 16), dev) if block_scales is None else block_scales
    elif block == Block.TILE:
        codes = _u8((rows, cols // 2), dev) if codes is None else codes
        block_scales = _u8((rows // 16, cols // 16), dev) if block_scales is None else block_scales
    else:
        codes = _u8((rows, cols // 2), dev) if codes is None else codes
        block_scales = _u8((rows, cols // 16), dev) if block_scales is None else block_scales
    if gscales is None:
        if gs == GScale.GIVEN:
            raise ValueError("gs=GIVEN needs gscales")
        gscales = torch.empty(rows if gs == GScale.PER_ROW else 1, dtype=torch.float32, device=dev)
    _check(lib().nvfp4_quantize(_ptr(x), rows, cols, x.stride(0), int(block), int(gs), int(rnd),
                                int(seed), int(stream_id), int(tensor_tag), int(layout), _ptr(codes),
                                codes.stride(0), _ptr(block_scales), _ptr(gscales), _stream(stream)))
    return codes, block_scales, gscales


def nvfp4_quantize_dq(x, gs=GScale.PER_TENSOR, rnd=Round.RNE, codes=None, block_scales=None,
                      gscales=None, dq=None, stream=None):
    """16x16 NVFP4 weight copy plus its dequantized BF16 copy in one pass.
    Returns (codes, block scales, S, dq)."""
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    gs = GScale(gs)
    codes = _u8((rows, cols // 2), dev) if codes is None else codes
    block_scales = _u8((rows // 16, cols // 16), dev) if block_scales is None else block_scales
    if gscales is None:
        if gs == GScale.GIVEN:
            raise ValueError("gs=GIVEN needs gscales")
        gscales = torch.empty(1, dtype=torch.float32, device=dev)
    dq = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev) if dq is None else dq
    _check(lib().nvfp4_quantize_dq(_ptr(x), rows, cols, x.stride(0), int(gs), int(rnd), _ptr(codes),
                                   codes.stride(0), _ptr(block_scales), _ptr(gscales), _ptr(dq),
                                   dq.stride(0), _stream(stream)))
    return codes, block_scales, gscales, dq


def nvfp4_quantize_rowcol(x, rnd=Round.RNE, seed=0, tensor_tag=0, layout=Layout.LINEAR, codes=None,
                          block_scales=None, gscales=None, codes_col=None, block_scales_col=None,
                          gscale_col=None, stream=None):
    """The rowwise per-token copy and the columnwise per-tensor copy of x in
    two passes (SR draws: stream 0 rowwise, 1 columnwise).  Returns (codes,
    block scales, S [rows], codes_col [cols, rows/2], block scales_col, S_col [1])."""
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    codes = _u8((rows, cols // 2), dev) if codes is None else codes
    block_scales = _u8((rows, cols // 16), dev) if block_scales is None else block_scales
    gscales = torch.empty(rows, dtype=torch.float32, device=dev) if gscales is None else gscales
    codes_col = _u8((cols, rows // 2), dev) if codes_col is None else codes_col
    block_scales_col = _u8((cols, rows // 16), dev) if block_scales_col is None else block_scales_col
    gscale_col = torch.empty(1, dtype=torch.float32, device=dev) if gscale_col is None else gscale_col
    _check(lib().nvfp4_quantize_rowcol(_ptr(x), rows, cols, x.stride(0), int(rnd), int(seed), int(tensor_tag),
                                       int(layout), _ptr(codes), codes.stride(0), _ptr(block_scales),
                                       _ptr(gscales), _ptr(codes_col), codes_col.stride(0),
                                       _ptr(block_scales_col), _ptr(gscale_col), _stream(stream)))
    return codes, block_scales, gscales, codes_col, block_scales_col, gscale_col


def nvfp4_quantize_tile_t(x, gs=GScale.PER_TENSOR, rnd=Round.RNE, seed=0, stream_id=0, tensor_tag=0,
                          codes=None, block_scales=None, codes_t=None, block_scales_t=None, gscales=None,
                          stream=None):
    """16x16 NVFP4 copy of x and its transposed copy (the 16x16 copy of x^T)
    in one pass.  Returns (codes, block scales, codes_t [cols, rows/2],
    block_scales_t [cols/16, rows/16], S)."""
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    gs = GScale(gs)
    codes = _u8((rows, cols // 2), dev) if codes is None else codes
    block_scales = _u8((rows // 16, cols // 16), dev) if block_scales is None else block_scales
    codes_t = _u8((cols, rows // 2), dev) if codes_t is None else codes_t
    block_scales_t = _u8((cols // 16, rows // 16), dev) if block_scales_t is None else block_scales_t
    if gscales is None:
        if gs == GScale.GIVEN:
            raise ValueError("gs=GIVEN needs gscales")
        gscales = torch.empty(1, dtype=torch.float32, device=dev)
    _check(lib().nvfp4_quantize_tile_t(_ptr(x), rows, cols, x.stride(0), int(gs), int(rnd), int(seed),
                                       int(stream_id), int(tensor_tag), _ptr(codes), codes.stride(0),
                                       _ptr(block_scales), _ptr(codes_t), codes_t.stride(0),
                                       _ptr(block_scales_t), _ptr(gscales), _stream(stream)))
    return codes, block_scales, codes_t, block_scales_t, gscales


def nvfp4_quantize_rht(x, sign_mask, gs=GScale.PER_TENSOR, rnd=Round.RNE, seed=0, stream_id=1,
                       tensor_tag=0, layout=Layout.LINEAR, codes=None, block_scales=None,
                       gscales=None, stream=None):
    """Columnwise NVFP4 copy of the random Hadamard transform of x (16-row
    blocks, signs from the 16-bit sign_mask).  Returns (packed codes [cols,
    rows/2], E4M3 block scales [cols, rows/16], FP32 S [1]), like
    nvfp4_quantize with block=COL."""
    _check_2d(x, torch.bfloat16, "x")
    rows, cols = x.shape
    dev = x.device
    gs = GScale(gs)
    codes = _u8((cols, rows // 2), dev) if codes is None else codes
    block_scales = _u8((cols, rows // 16), dev) if block_scales is None else block_scales
    if gscales is None:
        if gs == GScale.GIVEN:
            raise ValueError("gs=GIVEN needs gscales")
        gscales = torch.empty(1, dtype=torch.float32, device=dev)
    _check(lib().nvfp4_quantize_rht(_ptr(x), rows, cols, x.stride(0), int(sign_mask), int(gs),
                                    int(rnd), int(seed), int(stream_id), int(tensor_tag),
                                    int(layout), _ptr(codes), codes.stride(0), _ptr(block_scales),
                                    _ptr(gscales), _stream(stream)))
    return codes, block_scales, gscales


def mx_dequantize(fmt, codes, scales, rows, cols, block=Block.ROW, gscales=None, gs=GScale.NONE,
                  layout=Layout.LINEAR, out=None, stream=None):
    """DQ(Q(x)) of one stored copy ([rows, cols] as stored) to BF16."""
    fmt = Format(fmt)
    dev = codes.device
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev) if out is None else out
    _check(lib().mx_dequantize(int(fmt), _ptr(codes), codes.stride(0), _ptr(scales), _ptr(gscales),
                               rows, cols, int(block), int(gs), int(layout), _ptr(out),
                               out.stride(0), _stream(stream)))
    return out


class Operand:
    """A GEMM operand: a stored quantized copy (or BF16 tensor) plus its format.
    `ld` defaults to the row stride of `data` in elements."""

    def __init__(self, fmt, data, scales=None, gscales=None, block=Block.ROW, gs=GScale.NONE,
                 layout=Layout.LINEAR, ld=None, transposed=False):
        self.fmt, self.data, self.scales, self.gscales = Format(fmt), data, scales, gscales
        self.block, self.gs, self.layout = Block(block), GScale(gs), Layout(layout)
        if ld is None:
            ld = data.stride(-2) * (2 if self.fmt == Format.NVFP4 else 1)
        self.ld, self.transposed = int(ld), bool(transposed)

    def _c(self):
        return _Operand(int(self.fmt), self.data.data_ptr(),
                        0 if self.scales is None else self.scales.data_ptr(),
                        0 if self.gscales is None else self.gscales.data_ptr(),
                        int(self.block), int(self.gs), int(self.layout), self.ld,
                        1 if self.transposed else 0)


def _check_gemm_args(a, b, M, ncols, out, group_row_offsets, a_row_index, num_groups_expected=None):
    """Host-side checks of what the library reads on the device without
    validating: the group offsets, the gather index, the output and the
    second-scale tensors (the C ABI checks formats, shapes and alignment)."""
    for name, op in (("a", a), ("b", b)):
        if not isinstance(op, Operand):
            raise TypeError(f"{name} must be an Operand")
        if not (isinstance(op.data, torch.Tensor) and op.data.is_cuda):
            raise TypeError(f"{name}.data must be a CUDA tensor")
        if op.gscales is not None and (op.gscales.dtype != torch.float32 or not op.gscales.is_cuda
                                       or not op.gscales.is_contiguous()):
            raise TypeError(f"{name}.gscales must be a contiguous float32 CUDA tensor")
    if out is not None:
        if not (isinstance(out, torch.Tensor) and out.is_cuda and out.dtype == torch.bfloat16 and out.dim() == 2):
            raise TypeError("out must be a 2-D bfloat16 CUDA tensor")
        if out.shape[0] < M or out.shape[1] < ncols or out.stride(1) != 1:
            raise ValueError(f"out must hold [{M}, {ncols}] with unit column stride, got {tuple(out.shape)} "
                             f"strides {out.stride()}")
    if group_row_offsets is not None:
        g = group_row_offsets
        if not (isinstance(g, torch.Tensor) and g.is_cuda and g.dtype == torch.int32 and g.dim() == 1
                and g.is_contiguous()):
            raise TypeError("group_row_offsets must be a contiguous 1-D int32 CUDA tensor")
        if g.numel() < 2:
            raise ValueError("group_row_offsets needs num_groups + 1 >= 2 entries")
        if b.gscales is not None and b.gscales.numel() < g.numel() - 1:
            raise ValueError("b.gscales needs one scale per group")
    if a_row_index is not None:
        i = a_row_index
        if not (isinstance(i, torch.Tensor) and i.is_cuda and i.dtype == torch.int32 and i.dim() == 1
                and i.is_contiguous()):
            raise TypeError("a_row_index must be a contiguous 1-D int32 CUDA tensor")
        if i.numel() != M:
            raise ValueError(f"a_row_index must have M = {M} entries, got {i.numel()}")


def mx_gemm(a, b, M, N, K, out=None, group_row_offsets=None, a_row_index=None, a_rows=None,
            stream=None):
    """C[M, N] = sum_k A[m, k] B[n, k] in BF16 (FP32 accumulation).  Grouped
    (MoE) launches take int32 group_row_offsets [num_groups + 1] and an
    optional int32 gather index a_row_index [M] into the a_rows rows of A."""
    dev = a.data.device
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    _check_gemm_args(a, b, M, N, out, group_row_offsets, a_row_index)
    ng = 0 if group_row_offsets is None else group_row_offsets.numel() - 1
    if a_rows is None:
        a_rows = M
    ca, cb = a._c(), b._c()
    _check(lib().mx_gemm(ctypes.byref(ca), ctypes.byref(cb), M, N, K, int(a_rows), _ptr(out),
                         out.stride(0), ng, _ptr(group_row_offsets), _ptr(a_row_index),
                         _stream(stream)))
    return out


def mx_gemm_swiglu(a, b, M, inter, K, out=None, group_row_offsets=None, a_row_index=None, a_rows=None,
                   stream=None):
    """H[M, inter] = SwiGLU of the gate_up GEMM A B^T (B: gate rows then up
    rows), fused into the GEMM's epilogue; NVFP4 operands."""
    dev = a.data.device
    out = torch.empty((M, inter), dtype=torch.bfloat16, device=dev) if out is None else out
    _check_gemm_args(a, b, M, inter, out, group_row_offsets, a_row_index)
    ng = 0 if group_row_offsets is None else group_row_offsets.numel() - 1
    if a_rows is None:
        a_rows = M
    ca, cb = a._c(), b._c()
    _check(lib().mx_gemm_swiglu(ctypes.byref(ca), ctypes.byref(cb), M, inter, K, int(a_rows), _ptr(out),
                                out.stride(0), ng, _ptr(group_row_offsets), _ptr(a_row_index),
                                _stream(stream)))
    return out


def mx_gemm_swiglu_nvfp4(a, b, M, inter, K, group_row_offsets=None, a_row_index=None, a_rows=None,
                         layout=Layout.LINEAR, with_h=False, codes=None, block_scales=None, gscales=None,
                         h=None, stream=None):
    """The gate_up GEMM with SwiGLU and the per-token NVFP4 quantization of H
    in its epilogue.  Returns (codes [M, inter/2] uint8, block scales uint8,
    per-token S float32 [M]), the bytes nvfp4_quantize(H) writes, plus H
    [M, inter] BF16 when with_h (or h) is given."""
    dev = a.data.device
    if codes is None:
        codes = torch.empty((M, inter // 2), dtype=torch.uint8, device=dev)
    if block_scales is None:
        block_scales = torch.empty((M * (inter // 16),), dtype=torch.uint8, device=dev)
    if gscales is None:
        gscales = torch.empty((M,), dtype=torch.float32, device=dev)
    if h is None and with_h:
        h = torch.empty((M, inter), dtype=torch.bfloat16, device=dev)
    _check_gemm_args(a, b, M, inter, h, group_row_offsets, a_row_index)
    _check_2d(codes, torch.uint8, "codes")
    if codes.shape[0] < M or codes.shape[1] < inter // 2:
        raise ValueError(f"codes must hold [{M}, {inter // 2}]")
    for name, t, dt, n in (("block_scales", block_scales, torch.uint8, M * (inter // 16)),
                           ("gscales", gscales, torch.float32, M)):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dt and t.is_contiguous()):
            raise TypeError(f"{name} must be a contiguous {dt} CUDA tensor")
        if t.numel() < n:
            raise ValueError(f"{name} needs {n} elements")
    ng = 0 if group_row_offsets is None else group_row_offsets.numel() - 1
    if a_rows is None:
        a_rows = M
    ca, cb = a._c(), b._c()
    _check(lib().mx_gemm_swiglu_nvfp4(ctypes.byref(ca), ctypes.byref(cb), M, inter, K, int(a_rows), _ptr(codes),
                                      codes.stride(0), _ptr(block_scales), int(layout), _ptr(gscales), _ptr(h),
                                      0 if h is None else h.stride(0), ng, _ptr(group_row_offsets),
                                      _ptr(a_row_index), _stream(stream)))
    return (codes, block_scales, gscales, h) if h is not None else (codes, block_scales, gscales)


def mx_swiglu(gu, inter, out=None, stream=None):
    """h = silu(g) * u for gate_up [rows, 2*inter] BF16 -> [rows, inter] BF16."""
    _check_2d(gu, torch.bfloat16, "gu")
    rows = gu.shape[0]
    out = torch.empty((rows, inter), dtype=torch.bfloat16, device=gu.device) if out is None else out
    _check(lib().mx_swiglu(_ptr(gu), rows, inter, gu.stride(0), _ptr(out), out.stride(0),
                           _stream(stream)))
    return out


def mx_gemm_set_tile(tile):
    """Force the GEMM workgroup tile of every later mx_gemm call in the process
    (0..8, as listed at mx_gemm_set_tile in include/mxq.h), or restore the
    measured choice with -1."""
    _check(lib().mx_gemm_set_tile(int(tile)))
