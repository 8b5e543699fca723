// Dequantizers and the SwiGLU elementwise kernel.
//
// The dequantized backward runs its BF16 GEMMs on DQ(Q(w)), the BF16 values
// the forward pass actually used ("NVFP4 RL training" (The 4-bitter Lesson),
// section on the dequantized backward; "Miles Blackwell RL ...", section "O
// Suporte Miles Blackwell Agora Abrange Todo o Loop de RL").
//   MXFP8: bf16_RNE(value(c) * 2^e)            (ldexp is exact in binary32)
//   NVFP4: bf16_RNE(fl(fl(value(c) * s_b) * S)) (value(c) * s_b is exact)
// Both are pure bandwidth kernels: codes and scales in, 16-byte BF16 stores out.

#include "mxq_device.h"
#include "mxq_kernels.h"

namespace mxq {

// MXFP8: one lane per 8 codes.  tile = 1 for 32x32 scales; b128 = 1 for
// blockwise FP8 (128-wide blocks, 128x128 tiles, linear scales), 2 for
// blockwise FP8 with binary32 scales.
// IDX32: the chunk index fits 32 bits, so the row comes from a 32-bit division.
template <bool IDX32>
__global__ __launch_bounds__(256) void dq_mxfp8_kernel(
    const uint8_t* __restrict__ codes, int64_t ld_codes, const uint8_t* __restrict__ scales,
    int64_t rows, int64_t cols, int tile, int mfma_layout, int b128, uint16_t* __restrict__ out,
    int64_t ld_out) {
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * 256) {
    int64_t r, c;
    if (IDX32) {
      const uint32_t u = (uint32_t)id, d = (uint32_t)cpr, q32 = u / d;
      r = q32;
      c = u - q32 * d;
    } else {
      r = id / cpr;
      c = id - r * cpr;
    }
    uint2 q = *reinterpret_cast<const uint2*>(codes + r * ld_codes + c * 8);
    const int64_t si = b128 ? (tile ? (r >> 7) * (cols >> 7) + (c >> 4) : r * (cols >> 7) + (c >> 4))
                            : tile ? (r >> 5) * (cols >> 5) + (c >> 2)
                                   : scale_offset(r, c >> 2, cols >> 5, mfma_layout);
    uint32_t w[2] = {q.x, q.y};
    uint32_t o[4];
    if (b128 == 2) {
      // binary32 block scale: the product value(c) * s rounded once to binary32
      const float sc = reinterpret_cast<const float*>(scales)[si];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t word = w[i >> 1] >> (16 * (i & 1));
        o[i] = f32x2_to_bf16x2(e4m3_to_f32(word & 0xFF) * sc, e4m3_to_f32((word >> 8) & 0xFF) * sc);
      }
    } else {
      int e = (int)scales[si] - 127;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t word = w[i >> 1] >> (16 * (i & 1));
        float a = __builtin_ldexpf(e4m3_to_f32(word & 0xFF), e);
        float b = __builtin_ldexpf(e4m3_to_f32((word >> 8) & 0xFF), e);
        o[i] = f32x2_to_bf16x2(a, b);
      }
    }
    *reinterpret_cast<uint4*>(out + r * ld_out + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// NVFP4: one lane per half block (8 values, 4 code bytes), so each 16-byte
// store instruction of a wave covers one contiguous kilobyte of output.
// gmode: 0 = S per row, 1 = S per tensor.  tile = 1 for 16x16 scales.
// Codes become binary32 through the hardware FP4 conversion with unit scale
// (exact code values); IDX32: the half-block index fits 32 bits, so the row
// comes from a 32-bit division.
template <bool IDX32>
__global__ __launch_bounds__(256) void dq_nvfp4_kernel(
    const uint8_t* __restrict__ codes, int64_t ld_codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscales, int64_t rows, int64_t cols, int tile, int gmode,
    int mfma_layout, uint16_t* __restrict__ out, int64_t ld_out) {
  const int64_t hpr = cols >> 3, bpr = cols >> 4;
  const int64_t total = rows * hpr;
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * 256) {
    int64_t r, h;
    if (IDX32) {
      const uint32_t u = (uint32_t)id, d = (uint32_t)hpr, q32 = u / d;
      r = q32;
      h = u - q32 * d;
    } else {
      r = id / hpr;
      h = id - r * hpr;
    }
    const int64_t b = h >> 1;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * ld_codes + h * 4);
    const uint32_t sc = tile ? scales[(r >> 4) * bpr + b] : scales[scale_offset(r, b, bpr, mfma_layout)];
    const float sb = e4m3_to_f32(sc);
    const float S = gmode == 0 ? gscales[r] : gscales[0];
    mxq_f32x2 v[4];            // byte i of w: elements 2i (low nibble) and 2i + 1
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float da = (v[i].x * sb) * S, db = (v[i].y * sb) * S;   // exact product, then one rounding
      o[i] = f32x2_to_bf16x2(da, db);
    }
    *reinterpret_cast<uint4*>(out + r * ld_out + h * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// SwiGLU: h = silu(g) * u, silu(g) = g / (1 + exp(-g)), binary32, BF16 out.
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ gu, int64_t rows,
                                                     int64_t inter, int64_t ld_gu,
                                                     uint16_t* __restrict__ h, int64_t ld_h) {
  const int64_t cpr = inter >> 3;
  const int64_t total = rows * cpr;
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total;
       id += (int64_t)gridDim.x * 256) {
    int64_t r = id / cpr, c = id - r * cpr;
    uint4 g = *reinterpret_cast<const uint4*>(gu + r * ld_gu + c * 8);
    uint4 u = *reinterpret_cast<const uint4*>(gu + r * ld_gu + inter + c * 8);
    uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w}, o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = swiglu_bf16x2(gw[i], uw[i]);
    *reinterpret_cast<uint4*>(h + r * ld_h + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

static unsigned grid_for(int64_t total) {
  int64_t b = (total + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

hipError_t launch_dq_mxfp8(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                           int64_t rows, int64_t cols, bool tile, bool mfma, int b128,
                           uint16_t* out, int64_t ld_out, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  auto kern = total < (int64_t(1) << 32) ? dq_mxfp8_kernel<true> : dq_mxfp8_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid_for(total)), dim3(256), 0, st, codes, ld_codes, scales, rows,
                     cols, (int)tile, (int)mfma, (int)b128, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_dq_nvfp4(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                           const float* gscales, int64_t rows, int64_t cols, bool tile,
                           int gmode, bool mfma, uint16_t* out, int64_t ld_out, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  auto kern = total < (int64_t(1) << 32) ? dq_nvfp4_kernel<true> : dq_nvfp4_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(grid_for(total)), dim3(256), 0, st, codes, ld_codes, scales,
                     gscales, rows, cols, (int)tile, gmode, (int)mfma, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t* gu, int64_t rows, int64_t inter, int64_t ld_gu,
                         uint16_t* h, int64_t ld_h, hipStream_t st) {
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(rows * (inter / 8))), dim3(256), 0, st, gu, rows,
                     inter, ld_gu, h, ld_h);
  return hipGetLastError();
}

}  // namespace mxq
