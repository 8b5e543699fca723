// C ABI of the library: argument validation on the host, then kernel launches
// on the caller's stream.  See include/mxq.h for the contract of every entry.
// No allocation, no synchronization, no state kept between calls except the
// thread-local text of the last error.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "mxq.h"
#include "mxq_kernels.h"

namespace {

thread_local char g_err[512] = "";

mxq_status fail(mxq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mxq_status ok() {
  g_err[0] = 0;
  return MXQ_OK;
}

mxq_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXQ_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int mxq_version(void) { return MXQ_VERSION; }

const char* mxq_last_error(void) { return g_err; }

const char* mxq_status_str(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_EINVAL: return "MXQ_EINVAL: invalid argument";
    case MXQ_ESHAPE: return "MXQ_ESHAPE: size not a multiple of the block";
    case MXQ_EALIGN: return "MXQ_EALIGN: pointer or leading dimension not 16-byte aligned";
    case MXQ_EUNSUPPORTED: return "MXQ_EUNSUPPORTED: unsupported combination";
    case MXQ_EHIP: return "MXQ_EHIP: HIP runtime error";
  }
  return "unknown mxq_status";
}

// ---------------------------------------------------------------- quantize
mxq_status mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                       mxq_block block, mxq_scale_layout layout, uint8_t* codes,
                       int64_t ld_codes, uint8_t* scales, uint8_t* codes_col,
                       int64_t ld_codes_col, uint8_t* scales_col, void* stream) {
  if (rows < 0 || cols < 0) return fail(MXQ_EINVAL, "mx_quantize: negative size");
  if (block != MXQ_BLOCK_ROW && block != MXQ_BLOCK_COL && block != MXQ_BLOCK_TILE &&
      block != MXQ_BLOCK_DUAL)
    return fail(MXQ_EINVAL, "mx_quantize: block must be ROW, COL, TILE or DUAL");
  if (layout != MXQ_LAYOUT_LINEAR && layout != MXQ_LAYOUT_MFMA)
    return fail(MXQ_EINVAL, "mx_quantize: bad scale layout");
  if (rows == 0 || cols == 0) return ok();
  if (!x || !codes || !scales) return fail(MXQ_EINVAL, "mx_quantize: null pointer");
  if (block == MXQ_BLOCK_DUAL && (!codes_col || !scales_col))
    return fail(MXQ_EINVAL, "mx_quantize: DUAL needs codes_col and scales_col");
  // TILE: codes_col (with scales_col) asks for the transposed copy as well
  const bool tile_t = block == MXQ_BLOCK_TILE && codes_col;
  if (tile_t && !scales_col) return fail(MXQ_EINVAL, "mx_quantize: a transposed TILE copy needs scales_col");
  const bool second = block == MXQ_BLOCK_DUAL || tile_t;
  if (cols % 32) return fail(MXQ_ESHAPE, "mx_quantize: cols %% 32 != 0 (cols=%lld)", (long long)cols);
  if (block != MXQ_BLOCK_ROW && rows % 32)
    return fail(MXQ_ESHAPE, "mx_quantize: rows %% 32 != 0 for a COL/TILE/DUAL copy (rows=%lld)", (long long)rows);
  const bool mfma = layout == MXQ_LAYOUT_MFMA;
  if (mfma) {
    if (block == MXQ_BLOCK_TILE)
      return fail(MXQ_EUNSUPPORTED, "mx_quantize: the MFMA scale layout is for 1D blocks only");
    if ((block == MXQ_BLOCK_ROW || block == MXQ_BLOCK_DUAL) && (rows % 32 || cols % 128))
      return fail(MXQ_ESHAPE, "mx_quantize: MFMA layout of a rowwise copy needs rows %% 32 == 0 and cols %% 128 == 0");
    if ((block == MXQ_BLOCK_COL || block == MXQ_BLOCK_DUAL) && rows % 128)
      return fail(MXQ_ESHAPE, "mx_quantize: MFMA layout of a columnwise copy needs rows %% 128 == 0");
  }
  const int64_t need_row = block == MXQ_BLOCK_COL ? rows : cols;
  if (ld_x < cols || ld_codes < need_row || (second && ld_codes_col < rows))
    return fail(MXQ_EINVAL, "mx_quantize: leading dimension smaller than the row");
  if (!aligned16(x) || !aligned16(codes) || (ld_x * 2) % 16 || ld_codes % 16 ||
      (second && (!aligned16(codes_col) || ld_codes_col % 16)))
    return fail(MXQ_EALIGN, "mx_quantize: pointers and leading dimensions must be 16-byte aligned");
  hipError_t e;
  if (block == MXQ_BLOCK_ROW)
    e = mxq::launch_mxfp8_row(x, rows, cols, ld_x, codes, ld_codes, scales, mfma, false, S(stream));
  else
    e = mxq::launch_mxfp8_tile(block == MXQ_BLOCK_COL ? 0 : block == MXQ_BLOCK_TILE ? 1 : 2, x,
                               rows, cols, ld_x, codes, ld_codes, scales,
                               second ? codes_col : nullptr, ld_codes_col,
                               second ? scales_col : nullptr, mfma, false, S(stream));
  return hip_status(e, "mx_quantize");
}

// kind 1: power-of-two (E8M0) scales; 2: binary32 scales (scales point to floats)
static mxq_status fp8bw_impl(const char* fn, int kind, const uint16_t* x, int64_t rows, int64_t cols,
                             int64_t ld_x, mxq_block block, uint8_t* codes, int64_t ld_codes,
                             uint8_t* scales, uint8_t* codes_col, int64_t ld_codes_col,
                             uint8_t* scales_col, void* stream) {
  if (rows < 0 || cols < 0) return fail(MXQ_EINVAL, "%s: negative size", fn);
  if (block != MXQ_BLOCK_ROW && block != MXQ_BLOCK_COL && block != MXQ_BLOCK_TILE &&
      block != MXQ_BLOCK_DUAL)
    return fail(MXQ_EINVAL, "%s: block must be ROW, COL, TILE or DUAL", fn);
  if (rows == 0 || cols == 0) return ok();
  if (!x || !codes || !scales) return fail(MXQ_EINVAL, "%s: null pointer", fn);
  if (block == MXQ_BLOCK_DUAL && (!codes_col || !scales_col))
    return fail(MXQ_EINVAL, "%s: DUAL needs codes_col and scales_col", fn);
  const bool tile_t = block == MXQ_BLOCK_TILE && codes_col;
  if (tile_t && !scales_col) return fail(MXQ_EINVAL, "%s: a transposed TILE copy needs scales_col", fn);
  const bool second = block == MXQ_BLOCK_DUAL || tile_t;
  if (cols % 128) return fail(MXQ_ESHAPE, "%s: cols %% 128 != 0 (cols=%lld)", fn, (long long)cols);
  if (block != MXQ_BLOCK_ROW && rows % 128)
    return fail(MXQ_ESHAPE, "%s: rows %% 128 != 0 for a COL/TILE/DUAL copy (rows=%lld)", fn, (long long)rows);
  const int64_t need_row = block == MXQ_BLOCK_COL ? rows : cols;
  if (ld_x < cols || ld_codes < need_row || (second && ld_codes_col < rows))
    return fail(MXQ_EINVAL, "%s: leading dimension smaller than the row", fn);
  if (!aligned16(x) || !aligned16(codes) || (ld_x * 2) % 16 || ld_codes % 16 ||
      (second && (!aligned16(codes_col) || ld_codes_col % 16)))
    return fail(MXQ_EALIGN, "%s: pointers and leading dimensions must be 16-byte aligned", fn);
  if (kind == 2 && ((reinterpret_cast<uintptr_t>(scales) & 3) ||
                    (second && (reinterpret_cast<uintptr_t>(scales_col) & 3))))
    return fail(MXQ_EALIGN, "%s: binary32 scales must be 4-byte aligned", fn);
  hipError_t e;
  if (block == MXQ_BLOCK_ROW)
    e = mxq::launch_mxfp8_row(x, rows, cols, ld_x, codes, ld_codes, scales, false, kind, S(stream));
  else
    e = mxq::launch_mxfp8_tile(block == MXQ_BLOCK_COL ? 0 : block == MXQ_BLOCK_TILE ? 1 : 2, x,
                               rows, cols, ld_x, codes, ld_codes, scales,
                               second ? codes_col : nullptr, ld_codes_col,
                               second ? scales_col : nullptr, false, kind, S(stream));
  return hip_status(e, fn);
}

mxq_status fp8bw_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          mxq_block block, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                          uint8_t* codes_col, int64_t ld_codes_col, uint8_t* scales_col,
                          void* stream) {
  return fp8bw_impl("fp8bw_quantize", 1, x, rows, cols, ld_x, block, codes, ld_codes, scales,
                    codes_col, ld_codes_col, scales_col, stream);
}

mxq_status fp8bw_quantize_f32(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              mxq_block block, uint8_t* codes, int64_t ld_codes, float* scales,
                              uint8_t* codes_col, int64_t ld_codes_col, float* scales_col,
                              void* stream) {
  return fp8bw_impl("fp8bw_quantize_f32", 2, x, rows, cols, ld_x, block, codes, ld_codes,
                    reinterpret_cast<uint8_t*>(scales), codes_col, ld_codes_col,
                    reinterpret_cast<uint8_t*>(scales_col), stream);
}

// dq != nullptr: also the dequantized BF16 copy (TILE only); codes_t !=
// nullptr: also the transposed copy (TILE only)
static mxq_status nvfp4_quantize_impl(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                      mxq_block block, mxq_gscale gs, mxq_round rnd, uint64_t seed,
                                      uint32_t stream_id, uint32_t tensor_tag, mxq_scale_layout layout,
                                      uint8_t* codes, int64_t ld_codes_bytes, uint8_t* block_scales,
                                      float* gscales, uint16_t* dq, int64_t ld_dq, void* stream,
                                      uint8_t* codes_t = nullptr, int64_t ld_codes_t = 0,
                                      uint8_t* block_scales_t = nullptr) {
  if (rows < 0 || cols < 0) return fail(MXQ_EINVAL, "nvfp4_quantize: negative size");
  if (block != MXQ_BLOCK_ROW && block != MXQ_BLOCK_COL && block != MXQ_BLOCK_TILE)
    return fail(block == MXQ_BLOCK_DUAL ? MXQ_EUNSUPPORTED : MXQ_EINVAL,
                "nvfp4_quantize: block must be ROW, COL or TILE");
  if (gs != MXQ_GS_PER_ROW && gs != MXQ_GS_PER_TENSOR && gs != MXQ_GS_GIVEN)
    return fail(MXQ_EINVAL, "nvfp4_quantize: gs must be PER_ROW, PER_TENSOR or GIVEN");
  if (rnd != MXQ_ROUND_RNE && rnd != MXQ_ROUND_SR && rnd != MXQ_ROUND_RNE_4OVER6)
    return fail(MXQ_EINVAL, "nvfp4_quantize: bad rounding");
  if (rnd == MXQ_ROUND_RNE_4OVER6 && block == MXQ_BLOCK_COL)
    return fail(MXQ_EUNSUPPORTED, "nvfp4_quantize: the Four-Over-Six choice is for ROW and TILE copies");
  if (layout != MXQ_LAYOUT_LINEAR && layout != MXQ_LAYOUT_MFMA)
    return fail(MXQ_EINVAL, "nvfp4_quantize: bad scale layout");
  if (gs == MXQ_GS_PER_ROW && block != MXQ_BLOCK_ROW)
    return fail(MXQ_EUNSUPPORTED, "nvfp4_quantize: a per-row second scale needs ROW blocks "
                                  "(a columnwise or tiled copy takes a per-tensor scale)");
  if (rows == 0 || cols == 0) return ok();
  if (!x || !codes || !block_scales || !gscales) return fail(MXQ_EINVAL, "nvfp4_quantize: null pointer");
  if (cols % 16) return fail(MXQ_ESHAPE, "nvfp4_quantize: cols %% 16 != 0 (cols=%lld)", (long long)cols);
  if (block != MXQ_BLOCK_ROW && rows % 16)
    return fail(MXQ_ESHAPE, "nvfp4_quantize: rows %% 16 != 0 for a COL/TILE copy (rows=%lld)", (long long)rows);
  const bool mfma = layout == MXQ_LAYOUT_MFMA;
  if (mfma) {
    if (block == MXQ_BLOCK_TILE)
      return fail(MXQ_EUNSUPPORTED, "nvfp4_quantize: the MFMA scale layout is for 1D blocks only");
    if (block == MXQ_BLOCK_ROW && (rows % 32 || cols % 64))
      return fail(MXQ_ESHAPE, "nvfp4_quantize: MFMA layout needs rows %% 32 == 0 and cols %% 64 == 0");
    if (block == MXQ_BLOCK_COL && (cols % 32 || rows % 64))
      return fail(MXQ_ESHAPE, "nvfp4_quantize: MFMA layout of a columnwise copy needs cols %% 32 == 0 and rows %% 64 == 0");
  }
  const int64_t need = block == MXQ_BLOCK_COL ? rows / 2 : cols / 2;
  if (ld_x < cols || ld_codes_bytes < need)
    return fail(MXQ_EINVAL, "nvfp4_quantize: leading dimension smaller than the row");
  if (!aligned16(x) || !aligned16(codes) || (ld_x * 2) % 16 || ld_codes_bytes % 8 ||
      ((uintptr_t)gscales & 3u))
    return fail(MXQ_EALIGN, "nvfp4_quantize: x/codes must be 16-byte aligned, ld_x*2 %% 16 == 0, "
                            "ld_codes_bytes %% 8 == 0, gscales 4-byte aligned");
  if (dq) {
    if (block != MXQ_BLOCK_TILE)
      return fail(MXQ_EUNSUPPORTED, "nvfp4_quantize_dq: the fused dequantized copy is for TILE copies");
    if (ld_dq < cols) return fail(MXQ_EINVAL, "nvfp4_quantize_dq: ld_dq < cols");
    if (!aligned16(dq) || (ld_dq * 2) % 16) return fail(MXQ_EALIGN, "nvfp4_quantize_dq: dq 16-byte aligned, ld_dq*2 %% 16 == 0");
  }
  if (codes_t) {
    if (block != MXQ_BLOCK_TILE)
      return fail(MXQ_EUNSUPPORTED, "nvfp4_quantize_tile_t: the transposed copy is for TILE copies");
    if (!block_scales_t) return fail(MXQ_EINVAL, "nvfp4_quantize_tile_t: block_scales_t is NULL");
    if (ld_codes_t < rows / 2) return fail(MXQ_EINVAL, "nvfp4_quantize_tile_t: ld_codes_t_bytes < rows / 2");
    if (((uintptr_t)codes_t & 7u) || ld_codes_t % 8)
      return fail(MXQ_EALIGN, "nvfp4_quantize_tile_t: codes_t 8-byte aligned, ld_codes_t_bytes %% 8 == 0");
  }
  hipStream_t st = S(stream);
  const int rm = rnd == MXQ_ROUND_SR ? 1 : rnd == MXQ_ROUND_RNE_4OVER6 ? 2 : 0;
  hipError_t e = hipSuccess;
  // per-tensor: the amax kernel leaves a tagged amax in gscales[0], which the
  // quantize kernel turns into S (and stores back)
  if (gs == MXQ_GS_PER_TENSOR) {
    e = mxq::launch_nvfp4_tensor_scale(x, rows, cols, ld_x, gscales, st);
    if (e != hipSuccess) return hip_status(e, "nvfp4_quantize (tensor amax)");
  }
  const int gmode = gs == MXQ_GS_PER_ROW ? 0 : gs == MXQ_GS_PER_TENSOR ? 1 : 2;
  if (block == MXQ_BLOCK_ROW)
    e = mxq::launch_nvfp4_row(x, rows, cols, ld_x, codes, ld_codes_bytes, block_scales, gscales,
                              gmode, mfma, rm, seed, stream_id, tensor_tag, st);
  else if (block == MXQ_BLOCK_TILE)
    e = mxq::launch_nvfp4_tile16(x, rows, cols, ld_x, codes, ld_codes_bytes, block_scales, gscales,
                                 gmode, rm, seed, stream_id, tensor_tag, dq, ld_dq, codes_t, ld_codes_t,
                                 block_scales_t, st);
  else
    e = mxq::launch_nvfp4_col(x, rows, cols, ld_x, codes, ld_codes_bytes, block_scales, gscales,
                              gmode, mfma, rm == 1, false, 0u, seed, stream_id, tensor_tag, st);
  return hip_status(e, dq ? "nvfp4_quantize_dq" : codes_t ? "nvfp4_quantize_tile_t" : "nvfp4_quantize");
}

mxq_status nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          mxq_block block, mxq_gscale gs, mxq_round rnd, uint64_t seed,
                          uint32_t stream_id, uint32_t tensor_tag, mxq_scale_layout layout,
                          uint8_t* codes, int64_t ld_codes_bytes, uint8_t* block_scales,
                          float* gscales, void* stream) {
  return nvfp4_quantize_impl(x, rows, cols, ld_x, block, gs, rnd, seed, stream_id, tensor_tag, layout,
                             codes, ld_codes_bytes, block_scales, gscales, nullptr, 0, stream);
}

mxq_status nvfp4_quantize_dq(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                             mxq_gscale gs, mxq_round rnd, uint8_t* codes, int64_t ld_codes_bytes,
                             uint8_t* block_scales, float* gscales, uint16_t* dq, int64_t ld_dq,
                             void* stream) {
  if (!dq && rows > 0 && cols > 0) return fail(MXQ_EINVAL, "nvfp4_quantize_dq: dq is NULL");
  if (rnd == MXQ_ROUND_SR)
    return fail(MXQ_EUNSUPPORTED, "nvfp4_quantize_dq: weights take RNE or RNE_4OVER6");
  return nvfp4_quantize_impl(x, rows, cols, ld_x, MXQ_BLOCK_TILE, gs, rnd, 0, 0, 0, MXQ_LAYOUT_LINEAR,
                             codes, ld_codes_bytes, block_scales, gscales, dq, ld_dq, stream);
}

mxq_status nvfp4_quantize_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                 mxq_round rnd, uint64_t seed, uint32_t tensor_tag, mxq_scale_layout layout,
                                 uint8_t* codes, int64_t ld_codes_bytes, uint8_t* block_scales,
                                 float* gscales, uint8_t* codes_col, int64_t ld_codes_col_bytes,
                                 uint8_t* block_scales_col, float* gscale_col, void* stream) {
  const char* fn = "nvfp4_quantize_rowcol";
  if (rows < 0 || cols < 0) return fail(MXQ_EINVAL, "%s: negative size", fn);
  if (rnd != MXQ_ROUND_RNE && rnd != MXQ_ROUND_SR)
    return fail(rnd == MXQ_ROUND_RNE_4OVER6 ? MXQ_EUNSUPPORTED : MXQ_EINVAL,
                "%s: rounding must be RNE or SR (the columnwise copy takes no Four-Over-Six choice)", fn);
  if (layout != MXQ_LAYOUT_LINEAR && layout != MXQ_LAYOUT_MFMA) return fail(MXQ_EINVAL, "%s: bad scale layout", fn);
  if (rows == 0 || cols == 0) return ok();
  if (!x || !codes || !block_scales || !gscales || !codes_col || !block_scales_col || !gscale_col)
    return fail(MXQ_EINVAL, "%s: null pointer", fn);
  if (cols % 16 || rows % 16)
    return fail(MXQ_ESHAPE, "%s: rows and cols must be multiples of 16 (rows=%lld, cols=%lld)", fn,
                (long long)rows, (long long)cols);
  const bool mfma = layout == MXQ_LAYOUT_MFMA;
  if (mfma && (rows % 64 || cols % 64))
    return fail(MXQ_ESHAPE, "%s: the MFMA scale layout of both copies needs rows and cols multiples of 64", fn);
  if (ld_x < cols || ld_codes_bytes < cols / 2 || ld_codes_col_bytes < rows / 2)
    return fail(MXQ_EINVAL, "%s: leading dimension smaller than the row", fn);
  if (!aligned16(x) || !aligned16(codes) || !aligned16(codes_col) || (ld_x * 2) % 16 || ld_codes_bytes % 8 ||
      ld_codes_col_bytes % 8 || ((uintptr_t)gscales & 3u) || ((uintptr_t)gscale_col & 3u))
    return fail(MXQ_EALIGN, "%s: x/codes/codes_col 16-byte aligned, ld_x*2 %% 16 == 0, ld_codes_bytes and "
                            "ld_codes_col_bytes %% 8 == 0, gscales and gscale_col 4-byte aligned", fn);
  if (gscale_col == gscales || (gscale_col >= gscales && gscale_col < gscales + rows))
    return fail(MXQ_EINVAL, "%s: gscale_col must not alias gscales", fn);
  hipStream_t st = S(stream);
  const int rm = rnd == MXQ_ROUND_SR ? 1 : 0;
  uint32_t* acc = reinterpret_cast<uint32_t*>(gscale_col);
  // the rowwise pass leaves the tagged tensor amax in gscale_col[0], which
  // the columnwise pass turns into S (and stores back), as in PER_TENSOR mode
  hipError_t e = mxq::launch_zero_u32(acc, st);
  if (e == hipSuccess)
    e = mxq::launch_nvfp4_row(x, rows, cols, ld_x, codes, ld_codes_bytes, block_scales, gscales, 0, mfma, rm,
                              seed, 0, tensor_tag, st, acc);
  if (e == hipSuccess)
    e = mxq::launch_nvfp4_col(x, rows, cols, ld_x, codes_col, ld_codes_col_bytes, block_scales_col, gscale_col,
                              1, mfma, rm == 1, false, 0u, seed, 1, tensor_tag, st);
  return hip_status(e, fn);
}

mxq_status nvfp4_quantize_tile_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                 mxq_gscale gs, mxq_round rnd, uint64_t seed, uint32_t stream_id,
                                 uint32_t tensor_tag, uint8_t* codes, int64_t ld_codes_bytes,
                                 uint8_t* block_scales, uint8_t* codes_t, int64_t ld_codes_t_bytes,
                                 uint8_t* block_scales_t, float* gscales, void* stream) {
  if (!codes_t && rows > 0 && cols > 0) return fail(MXQ_EINVAL, "nvfp4_quantize_tile_t: codes_t is NULL");
  return nvfp4_quantize_impl(x, rows, cols, ld_x, MXQ_BLOCK_TILE, gs, rnd, seed, stream_id, tensor_tag,
                             MXQ_LAYOUT_LINEAR, codes, ld_codes_bytes, block_scales, gscales, nullptr, 0,
                             stream, codes_t, ld_codes_t_bytes, block_scales_t);
}

mxq_status nvfp4_quantize_rht(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              uint32_t sign_mask, mxq_gscale gs, mxq_round rnd, uint64_t seed,
                              uint32_t stream_id, uint32_t tensor_tag, mxq_scale_layout layout,
                              uint8_t* codes, int64_t ld_codes_bytes, uint8_t* block_scales,
                              float* gscales, void* stream) {
  if (rows < 0 || cols < 0) return fail(MXQ_EINVAL, "nvfp4_quantize_rht: negative size");
  if (sign_mask > 0xFFFFu) return fail(MXQ_EINVAL, "nvfp4_quantize_rht: sign_mask has bits above 15");
  if (gs != MXQ_GS_PER_TENSOR && gs != MXQ_GS_GIVEN)
    return fail(gs == MXQ_GS_PER_ROW ? MXQ_EUNSUPPORTED : MXQ_EINVAL,
                "nvfp4_quantize_rht: the columnwise copy takes a PER_TENSOR or GIVEN second scale");
  if (rnd == MXQ_ROUND_RNE_4OVER6)
    return fail(MXQ_EUNSUPPORTED, "nvfp4_quantize_rht: the Four-Over-Six choice is for ROW and TILE copies");
  if (rnd != MXQ_ROUND_RNE && rnd != MXQ_ROUND_SR) return fail(MXQ_EINVAL, "nvfp4_quantize_rht: bad rounding");
  if (layout != MXQ_LAYOUT_LINEAR && layout != MXQ_LAYOUT_MFMA)
    return fail(MXQ_EINVAL, "nvfp4_quantize_rht: bad scale layout");
  if (rows == 0 || cols == 0) return ok();
  if (!x || !codes || !block_scales || !gscales) return fail(MXQ_EINVAL, "nvfp4_quantize_rht: null pointer");
  if (rows % 16 || cols % 16)
    return fail(MXQ_ESHAPE, "nvfp4_quantize_rht: rows %% 16 and cols %% 16 must be 0 (rows=%lld, cols=%lld)",
                (long long)rows, (long long)cols);
  const bool mfma = layout == MXQ_LAYOUT_MFMA;
  if (mfma && (cols % 32 || rows % 64))
    return fail(MXQ_ESHAPE, "nvfp4_quantize_rht: MFMA layout needs cols %% 32 == 0 and rows %% 64 == 0");
  if (ld_x < cols || ld_codes_bytes < rows / 2)
    return fail(MXQ_EINVAL, "nvfp4_quantize_rht: leading dimension smaller than the row");
  if (!aligned16(x) || !aligned16(codes) || (ld_x * 2) % 16 || ld_codes_bytes % 8 ||
      ((uintptr_t)gscales & 3u))
    return fail(MXQ_EALIGN, "nvfp4_quantize_rht: x/codes must be 16-byte aligned, ld_x*2 %% 16 == 0, "
                            "ld_codes_bytes %% 8 == 0, gscales 4-byte aligned");
  hipStream_t st = S(stream);
  hipError_t e = hipSuccess;
  if (gs == MXQ_GS_PER_TENSOR) {
    e = mxq::launch_nvfp4_tensor_scale_rht(x, rows, cols, ld_x, sign_mask, gscales, st);
    if (e != hipSuccess) return hip_status(e, "nvfp4_quantize_rht (tensor amax)");
  }
  e = mxq::launch_nvfp4_col(x, rows, cols, ld_x, codes, ld_codes_bytes, block_scales, gscales,
                            gs == MXQ_GS_PER_TENSOR ? 1 : 2, mfma, rnd == MXQ_ROUND_SR, true,
                            sign_mask, seed, stream_id, tensor_tag, st);
  return hip_status(e, "nvfp4_quantize_rht");
}

// ---------------------------------------------------------------- dequantize
mxq_status mx_dequantize(mxq_format fmt, const uint8_t* codes, int64_t ld_codes,
                         const uint8_t* scales, const float* gscales, int64_t rows, int64_t cols,
                         mxq_block block, mxq_gscale gs, mxq_scale_layout layout, uint16_t* out,
                         int64_t ld_out, void* stream) {
  if (rows < 0 || cols < 0) return fail(MXQ_EINVAL, "mx_dequantize: negative size");
  if (fmt != MXQ_FMT_MXFP8 && fmt != MXQ_FMT_NVFP4 && fmt != MXQ_FMT_FP8_B128 &&
      fmt != MXQ_FMT_FP8_B128_F32)
    return fail(MXQ_EINVAL, "mx_dequantize: format must be MXFP8, NVFP4, FP8_B128 or FP8_B128_F32");
  if (block == MXQ_BLOCK_COL || block == MXQ_BLOCK_DUAL)
    return fail(MXQ_EUNSUPPORTED, "mx_dequantize: pass ROW for a stored columnwise copy (it is row-blocked)");
  if (block != MXQ_BLOCK_ROW && block != MXQ_BLOCK_TILE) return fail(MXQ_EINVAL, "mx_dequantize: bad block");
  if (layout != MXQ_LAYOUT_LINEAR && layout != MXQ_LAYOUT_MFMA) return fail(MXQ_EINVAL, "mx_dequantize: bad layout");
  const bool mfma = layout == MXQ_LAYOUT_MFMA;
  if (mfma && block == MXQ_BLOCK_TILE)
    return fail(MXQ_EUNSUPPORTED, "mx_dequantize: the MFMA scale layout is for 1D blocks only");
  if (rows == 0 || cols == 0) return ok();
  if (!codes || !scales || !out) return fail(MXQ_EINVAL, "mx_dequantize: null pointer");
  if (!aligned16(codes) || !aligned16(out) || (ld_out * 2) % 16 || ld_codes % 8)
    return fail(MXQ_EALIGN, "mx_dequantize: codes/out 16-byte aligned, ld_out*2 %% 16 == 0, ld_codes %% 8 == 0");
  if (ld_out < cols) return fail(MXQ_EINVAL, "mx_dequantize: ld_out < cols");
  hipError_t e;
  if (fmt == MXQ_FMT_FP8_B128 || fmt == MXQ_FMT_FP8_B128_F32) {
    if (gs != MXQ_GS_NONE) return fail(MXQ_EUNSUPPORTED, "mx_dequantize: blockwise FP8 has no second-level scale");
    if (mfma) return fail(MXQ_EUNSUPPORTED, "mx_dequantize: blockwise FP8 scales are linear");
    if (cols % 128 || (block == MXQ_BLOCK_TILE && rows % 128))
      return fail(MXQ_ESHAPE, "mx_dequantize: blockwise FP8 needs cols %% 128 == 0 (and rows %% 128 for TILE)");
    if (ld_codes < cols) return fail(MXQ_EINVAL, "mx_dequantize: ld_codes < cols");
    if (fmt == MXQ_FMT_FP8_B128_F32 && (reinterpret_cast<uintptr_t>(scales) & 3))
      return fail(MXQ_EALIGN, "mx_dequantize: binary32 scales must be 4-byte aligned");
    e = mxq::launch_dq_mxfp8(codes, ld_codes, scales, rows, cols, block == MXQ_BLOCK_TILE, false,
                             fmt == MXQ_FMT_FP8_B128_F32 ? 2 : 1, out, ld_out, S(stream));
  } else if (fmt == MXQ_FMT_MXFP8) {
    if (gs != MXQ_GS_NONE) return fail(MXQ_EUNSUPPORTED, "mx_dequantize: MXFP8 has no second-level scale");
    if (cols % 32 || (block == MXQ_BLOCK_TILE && rows % 32))
      return fail(MXQ_ESHAPE, "mx_dequantize: MXFP8 needs cols %% 32 == 0 (and rows %% 32 for TILE)");
    if (mfma && (rows % 32 || cols % 128)) return fail(MXQ_ESHAPE, "mx_dequantize: MFMA layout needs rows %% 32, cols %% 128");
    if (ld_codes < cols) return fail(MXQ_EINVAL, "mx_dequantize: ld_codes < cols");
    e = mxq::launch_dq_mxfp8(codes, ld_codes, scales, rows, cols, block == MXQ_BLOCK_TILE, mfma, false,
                             out, ld_out, S(stream));
  } else {
    if (!gscales) return fail(MXQ_EINVAL, "mx_dequantize: NVFP4 needs gscales");
    if (gs != MXQ_GS_PER_ROW && gs != MXQ_GS_PER_TENSOR && gs != MXQ_GS_GIVEN)
      return fail(MXQ_EINVAL, "mx_dequantize: NVFP4 needs a second-level scale mode");
    if (gs == MXQ_GS_PER_ROW && block != MXQ_BLOCK_ROW)
      return fail(MXQ_EUNSUPPORTED, "mx_dequantize: per-row second scale with tile blocks");
    if (cols % 16 || (block == MXQ_BLOCK_TILE && rows % 16))
      return fail(MXQ_ESHAPE, "mx_dequantize: NVFP4 needs cols %% 16 == 0 (and rows %% 16 for TILE)");
    if (mfma && (rows % 32 || cols % 64)) return fail(MXQ_ESHAPE, "mx_dequantize: MFMA layout needs rows %% 32, cols %% 64");
    if (ld_codes < cols / 2) return fail(MXQ_EINVAL, "mx_dequantize: ld_codes (bytes) < cols/2");
    e = mxq::launch_dq_nvfp4(codes, ld_codes, scales, gscales, rows, cols, block == MXQ_BLOCK_TILE,
                             gs == MXQ_GS_PER_ROW ? 0 : 1, mfma, out, ld_out, S(stream));
  }
  return hip_status(e, "mx_dequantize");
}

// ---------------------------------------------------------------- GEMM
static mxq_status check_operand(const char* name, const mxq_operand* o, bool is_b, int64_t rows,
                                int64_t K, int64_t N_for_bt) {
  if (!o->data) return fail(MXQ_EINVAL, "mx_gemm: %s->data is NULL", name);
  if (o->fmt != MXQ_FMT_MXFP8 && o->fmt != MXQ_FMT_NVFP4 && o->fmt != MXQ_FMT_BF16 &&
      o->fmt != MXQ_FMT_FP8_B128)
    return fail(MXQ_EINVAL, "mx_gemm: %s has a bad format", name);
  if (!aligned16(o->data)) return fail(MXQ_EALIGN, "mx_gemm: %s->data not 16-byte aligned", name);
  if (o->transposed && !is_b) return fail(MXQ_EUNSUPPORTED, "mx_gemm: only B may be stored transposed");
  const int blk = o->fmt == MXQ_FMT_MXFP8 ? 32 : o->fmt == MXQ_FMT_NVFP4 ? 16 : o->fmt == MXQ_FMT_FP8_B128 ? 128 : 1;
  if (o->fmt == MXQ_FMT_FP8_B128 && o->layout != MXQ_LAYOUT_LINEAR)
    return fail(MXQ_EUNSUPPORTED, "mx_gemm: FP8_B128 scales of %s are linear", name);
  if (o->fmt == MXQ_FMT_BF16) {
    if (o->block != MXQ_BLOCK_NONE) return fail(MXQ_EINVAL, "mx_gemm: a BF16 %s takes block NONE", name);
    if ((o->ld * 2) % 16) return fail(MXQ_EALIGN, "mx_gemm: %s->ld*2 %% 16 != 0", name);
  } else {
    if (!o->scales) return fail(MXQ_EINVAL, "mx_gemm: %s->scales is NULL", name);
    if (o->block == MXQ_BLOCK_NONE || o->block == MXQ_BLOCK_DUAL)
      return fail(MXQ_EINVAL, "mx_gemm: %s block must be ROW or TILE", name);
    if (o->block == MXQ_BLOCK_COL)
      return fail(MXQ_EINVAL, "mx_gemm: a stored columnwise copy is row-blocked: pass ROW for %s", name);
    if (o->block == MXQ_BLOCK_TILE && !is_b)
      return fail(MXQ_EUNSUPPORTED, "mx_gemm: tile blocks are supported for B only");
    if (o->ld % 16) return fail(MXQ_EALIGN, "mx_gemm: %s->ld %% 16 != 0", name);
    if (o->layout == MXQ_LAYOUT_MFMA) {
      if (o->block != MXQ_BLOCK_ROW) return fail(MXQ_EUNSUPPORTED, "mx_gemm: MFMA layout with tile blocks");
      if (rows % 32 || (K / blk) % 4) return fail(MXQ_ESHAPE, "mx_gemm: MFMA layout of %s needs rows %% 32 and K/block %% 4", name);
    } else if (o->layout != MXQ_LAYOUT_LINEAR) {
      return fail(MXQ_EINVAL, "mx_gemm: bad scale layout for %s", name);
    }
  }
  if (o->fmt == MXQ_FMT_NVFP4) {
    if (!o->gscales) return fail(MXQ_EINVAL, "mx_gemm: %s->gscales is NULL", name);
    if (o->gs == MXQ_GS_PER_ROW) {
      if (is_b) return fail(MXQ_EUNSUPPORTED, "mx_gemm: B takes a per-tensor second scale");
    } else if (o->gs != MXQ_GS_PER_TENSOR && o->gs != MXQ_GS_GIVEN) {
      return fail(MXQ_EINVAL, "mx_gemm: NVFP4 %s needs a second-level scale mode", name);
    }
  }
  if (o->transposed) {
    if (o->fmt != MXQ_FMT_BF16 && o->block != MXQ_BLOCK_TILE)
      return fail(MXQ_EUNSUPPORTED, "mx_gemm: a transposed quantized B must be tile-blocked");
    const int t = o->fmt == MXQ_FMT_MXFP8 ? 32 : o->fmt == MXQ_FMT_NVFP4 ? 16 : o->fmt == MXQ_FMT_FP8_B128 ? 128 : 8;
    if (N_for_bt % t || K % t) return fail(MXQ_ESHAPE, "mx_gemm: transposed B needs N and K multiples of %d", t);
    if (o->ld < N_for_bt) return fail(MXQ_EINVAL, "mx_gemm: B->ld < N");
  } else {
    if (o->ld < K) return fail(MXQ_EINVAL, "mx_gemm: %s->ld < K", name);
    if (o->block == MXQ_BLOCK_TILE && (rows % blk || K % blk))
      return fail(MXQ_ESHAPE, "mx_gemm: tile-blocked %s needs rows and K multiples of %d", name, blk);
  }
  return MXQ_OK;
}

// Blockwise FP8 with binary32 block scales: dense, row-major operands, ROW
// ([rows, K/128]) or TILE ([rows/128, K/128]) scales, its own kernel.
static mxq_status check_fp8s(const char* name, const mxq_operand* o, int64_t rows, int64_t K) {
  if (!o->data || !o->scales) return fail(MXQ_EINVAL, "mx_gemm: %s->data or ->scales is NULL", name);
  if (o->transposed)
    return fail(MXQ_EUNSUPPORTED, "mx_gemm: FP8_B128_F32 operands are read as stored (use the transposed TILE copy)");
  if (o->block != MXQ_BLOCK_ROW && o->block != MXQ_BLOCK_TILE)
    return fail(MXQ_EINVAL, "mx_gemm: %s block must be ROW or TILE", name);
  if (o->layout != MXQ_LAYOUT_LINEAR) return fail(MXQ_EUNSUPPORTED, "mx_gemm: FP8_B128_F32 scales of %s are linear", name);
  if (o->gs != MXQ_GS_NONE) return fail(MXQ_EUNSUPPORTED, "mx_gemm: FP8_B128_F32 has no second-level scale");
  if (!aligned16(o->data) || o->ld % 16) return fail(MXQ_EALIGN, "mx_gemm: %s data 16-byte aligned, ld %% 16 == 0", name);
  if (reinterpret_cast<uintptr_t>(o->scales) & 3) return fail(MXQ_EALIGN, "mx_gemm: %s binary32 scales 4-byte aligned", name);
  if (o->ld < K) return fail(MXQ_EINVAL, "mx_gemm: %s->ld < K", name);
  if (o->block == MXQ_BLOCK_TILE && rows % 128)
    return fail(MXQ_ESHAPE, "mx_gemm: tile-blocked %s needs rows %% 128 == 0", name);
  return MXQ_OK;
}

static mxq_status gemm_fp8s_impl(const mxq_operand* a, const mxq_operand* b, int64_t M, int64_t N,
                                 int64_t K, uint16_t* c, int64_t ldc, int32_t num_groups,
                                 const int32_t* a_row_index, void* stream) {
  if (num_groups > 0 || a_row_index)
    return fail(MXQ_EUNSUPPORTED, "mx_gemm: FP8_B128_F32 is dense (no groups, no gather)");
  mxq_status s = check_fp8s("A", a, M, K);
  if (s != MXQ_OK) return s;
  s = check_fp8s("B", b, N, K);
  if (s != MXQ_OK) return s;
  mxq::Fp8sArgs g = {};
  g.a = static_cast<const uint8_t*>(a->data);
  g.a_scales = reinterpret_cast<const float*>(a->scales);
  g.lda = a->ld;
  g.a_tile = a->block == MXQ_BLOCK_TILE;
  g.b = static_cast<const uint8_t*>(b->data);
  g.b_scales = reinterpret_cast<const float*>(b->scales);
  g.ldb = b->ld;
  g.b_tile = b->block == MXQ_BLOCK_TILE;
  g.c = c;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  return hip_status(mxq::launch_gemm_fp8s(g, S(stream)), "mx_gemm");
}

// inter > 0: the gate_up GEMM with SwiGLU fused (N = 2 inter, c = H [M, inter]).
// The per-token NVFP4 copy of H that mx_gemm_swiglu_nvfp4 writes.
struct QhArgs {
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  bool mfma;
  float* gscales;
};

static mxq_status gemm_impl(const mxq_operand* a, const mxq_operand* b, int64_t M, int64_t N, int64_t K,
                            int64_t a_rows, uint16_t* c, int64_t ldc, int32_t num_groups,
                            const int32_t* group_row_offsets, const int32_t* a_row_index,
                            int64_t inter, void* stream, const QhArgs* q = nullptr) {
  if (!a || !b) return fail(MXQ_EINVAL, "mx_gemm: null operand");
  if (M < 0 || N < 0 || K < 0 || num_groups < 0 || a_rows < 0) return fail(MXQ_EINVAL, "mx_gemm: negative size");
  if (a->fmt != b->fmt) return fail(MXQ_EUNSUPPORTED, "mx_gemm: A and B formats differ");
  if (M == 0 || N == 0) return ok();
  if (K == 0) return fail(MXQ_EUNSUPPORTED, "mx_gemm: K == 0 (nothing would be written)");
  if (!c && !q) return fail(MXQ_EINVAL, "mx_gemm: c is NULL");
  if (num_groups > 0 && !group_row_offsets) return fail(MXQ_EINVAL, "mx_gemm: grouped call without offsets");
  if (!a_row_index && a_rows != M) return fail(MXQ_EINVAL, "mx_gemm: a_rows must equal M without a gather index");
  if (a_rows < 1) return fail(MXQ_EINVAL, "mx_gemm: a_rows < 1");
  const int blk = a->fmt == MXQ_FMT_MXFP8 ? 32 : a->fmt == MXQ_FMT_NVFP4 ? 16
                  : (a->fmt == MXQ_FMT_FP8_B128 || a->fmt == MXQ_FMT_FP8_B128_F32) ? 128 : 8;
  if (K % blk) return fail(MXQ_ESHAPE, "mx_gemm: K %% %d != 0 (K=%lld)", blk, (long long)K);
  if (c && ldc < (inter ? inter : N)) return fail(MXQ_EINVAL, "mx_gemm: ldc smaller than the output row");
  if (inter) {
    if (a->fmt != MXQ_FMT_NVFP4)
      return fail(MXQ_EUNSUPPORTED, "mx_gemm_swiglu: the fused SwiGLU epilogue is built for NVFP4 operands");
    if (b->transposed) return fail(MXQ_EUNSUPPORTED, "mx_gemm_swiglu: B must be row-major (the gate_up weight)");
    if (inter % 64) return fail(MXQ_ESHAPE, "mx_gemm_swiglu: inter %% 64 != 0 (inter=%lld)", (long long)inter);
    if (K % 64) return fail(MXQ_ESHAPE, "mx_gemm_swiglu: K %% 64 != 0 (K=%lld)", (long long)K);
    if (q && inter != 256 && inter != 512 && inter != 768)
      return fail(MXQ_EUNSUPPORTED, "mx_gemm_swiglu_nvfp4: inter must be 256, 512 or 768 (inter=%lld)",
                  (long long)inter);
  }
  if (a->fmt == MXQ_FMT_FP8_B128_F32)
    return gemm_fp8s_impl(a, b, M, N, K, c, ldc, num_groups, a_row_index, stream);
  mxq_status s = check_operand("A", a, false, a_rows, K, 0);
  if (s != MXQ_OK) return s;
  s = check_operand("B", b, true, N, K, N);
  if (s != MXQ_OK) return s;
  if (a->fmt != MXQ_FMT_BF16 && a->block != MXQ_BLOCK_ROW) return fail(MXQ_EUNSUPPORTED, "mx_gemm: A must be row-blocked");
  // the kernels address each operand with 32-bit offsets
  {
    auto row_bytes = [](const mxq_operand* o) {
      return o->fmt == MXQ_FMT_NVFP4 ? o->ld / 2 : o->fmt == MXQ_FMT_BF16 ? o->ld * 2 : o->ld;
    };
    const int64_t lim = (int64_t)1 << 31;
    if (a_rows * row_bytes(a) >= lim || (b->transposed ? K : N) * row_bytes(b) >= lim)
      return fail(MXQ_EUNSUPPORTED, "mx_gemm: an operand (one group of B) must be smaller than 2 GiB");
  }

  mxq::GemmArgs g = {};
  g.a = static_cast<const uint8_t*>(a->data);
  g.a_scales = a->scales;
  g.a_gs = a->gscales;
  g.lda = a->ld;
  g.a_mfma_layout = a->layout == MXQ_LAYOUT_MFMA;
  g.a_gs_per_row = a->gs == MXQ_GS_PER_ROW;
  g.b = static_cast<const uint8_t*>(b->data);
  g.b_scales = b->scales;
  g.b_gs = b->gscales;
  g.ldb = b->ld;
  g.b_mfma_layout = b->layout == MXQ_LAYOUT_MFMA;
  g.b_tile = b->block == MXQ_BLOCK_TILE;
  g.b_group_elems = (b->transposed ? K : N) * b->ld;
  const int bb = b->fmt == MXQ_FMT_MXFP8 ? 32 : b->fmt == MXQ_FMT_FP8_B128 ? 128 : 16;
  g.b_group_scales = b->fmt == MXQ_FMT_BF16 ? 0 : (g.b_tile ? (N / bb) * (K / bb) : N * (K / bb));
  g.a_b128 = a->fmt == MXQ_FMT_FP8_B128;
  g.b_b128 = b->fmt == MXQ_FMT_FP8_B128;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a_rows = a_rows;
  g.c = c;
  g.ldc = ldc;
  g.num_groups = num_groups;
  g.offsets = group_row_offsets;
  g.row_index = a_row_index;
  g.swiglu_inter = inter;
  const int path = (a->fmt == MXQ_FMT_MXFP8 || a->fmt == MXQ_FMT_FP8_B128) ? mxq::P_FP8
                   : a->fmt == MXQ_FMT_NVFP4 ? mxq::P_F16 : mxq::P_BF16;
  if (q)
    return hip_status(mxq::launch_gemm_swiglu_q(g, q->codes, q->ld_codes, q->scales, q->gscales, q->mfma, S(stream)),
                      "mx_gemm_swiglu_nvfp4");
  return hip_status(mxq::launch_gemm(path, b->transposed != 0, g, S(stream)), inter ? "mx_gemm_swiglu" : "mx_gemm");
}

mxq_status mx_gemm(const mxq_operand* a, const mxq_operand* b, int64_t M, int64_t N, int64_t K,
                   int64_t a_rows, uint16_t* c, int64_t ldc, int32_t num_groups,
                   const int32_t* group_row_offsets, const int32_t* a_row_index, void* stream) {
  return gemm_impl(a, b, M, N, K, a_rows, c, ldc, num_groups, group_row_offsets, a_row_index, 0, stream);
}

mxq_status mx_gemm_swiglu(const mxq_operand* a, const mxq_operand* b, int64_t M, int64_t inter,
                          int64_t K, int64_t a_rows, uint16_t* h, int64_t ldh, int32_t num_groups,
                          const int32_t* group_row_offsets, const int32_t* a_row_index, void* stream) {
  if (inter < 0) return fail(MXQ_EINVAL, "mx_gemm_swiglu: negative size");
  if (inter == 0 || M == 0) return ok();
  return gemm_impl(a, b, M, 2 * inter, K, a_rows, h, ldh, num_groups, group_row_offsets, a_row_index,
                   inter, stream);
}

mxq_status mx_gemm_swiglu_nvfp4(const mxq_operand* a, const mxq_operand* b, int64_t M, int64_t inter,
                                int64_t K, int64_t a_rows, uint8_t* codes, int64_t ld_codes,
                                uint8_t* block_scales, int32_t layout, float* gscales, uint16_t* h,
                                int64_t ldh, int32_t num_groups, const int32_t* group_row_offsets,
                                const int32_t* a_row_index, void* stream) {
  if (inter < 0 || M < 0 || ld_codes < 0) return fail(MXQ_EINVAL, "mx_gemm_swiglu_nvfp4: negative size");
  if (inter == 0 || M == 0) return ok();
  if (!codes || !block_scales || !gscales) return fail(MXQ_EINVAL, "mx_gemm_swiglu_nvfp4: null output");
  if (ld_codes < inter / 2) return fail(MXQ_EINVAL, "mx_gemm_swiglu_nvfp4: ld_codes smaller than a row's codes");
  if (!aligned16(codes) || ld_codes % 16) return fail(MXQ_EALIGN, "mx_gemm_swiglu_nvfp4: codes rows must be 16-byte aligned");
  if (layout != MXQ_LAYOUT_LINEAR && layout != MXQ_LAYOUT_MFMA)
    return fail(MXQ_EINVAL, "mx_gemm_swiglu_nvfp4: bad scale layout");
  if (layout == MXQ_LAYOUT_MFMA && M % 32)
    return fail(MXQ_ESHAPE, "mx_gemm_swiglu_nvfp4: MFMA scale layout needs M %% 32 == 0");
  if (h && (!aligned16(h) || (ldh * 2) % 16))
    return fail(MXQ_EALIGN, "mx_gemm_swiglu_nvfp4: h rows must be 16-byte aligned");
  const QhArgs q = {codes, ld_codes, block_scales, layout == MXQ_LAYOUT_MFMA, gscales};
  return gemm_impl(a, b, M, 2 * inter, K, a_rows, h, ldh, num_groups, group_row_offsets, a_row_index, inter,
                   stream, &q);
}

// ---------------------------------------------------------------- SwiGLU
mxq_status mx_swiglu(const uint16_t* gu, int64_t rows, int64_t inter, int64_t ld_gu, uint16_t* h,
                     int64_t ld_h, void* stream) {
  if (rows < 0 || inter < 0) return fail(MXQ_EINVAL, "mx_swiglu: negative size");
  if (rows == 0 || inter == 0) return ok();
  if (!gu || !h) return fail(MXQ_EINVAL, "mx_swiglu: null pointer");
  if (inter % 8) return fail(MXQ_ESHAPE, "mx_swiglu: inter %% 8 != 0");
  if (ld_gu < 2 * inter || ld_h < inter) return fail(MXQ_EINVAL, "mx_swiglu: leading dimension too small");
  if (!aligned16(gu) || !aligned16(h) || (ld_gu * 2) % 16 || (ld_h * 2) % 16)
    return fail(MXQ_EALIGN, "mx_swiglu: 16-byte alignment required");
  return hip_status(mxq::launch_swiglu(gu, rows, inter, ld_gu, h, ld_h, S(stream)), "mx_swiglu");
}

mxq_status mx_gemm_set_tile(int32_t tile) {
  if (tile < -1 || tile > 8) return fail(MXQ_EINVAL, "mx_gemm_set_tile: tile %d outside [-1, 8]", (int)tile);
  mxq::gemm_set_tile((int)tile);
  return ok();
}

}  // extern "C"
