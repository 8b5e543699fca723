// MXFP8 quantizers for gfx950.
//
// MXFP8 = 32 E4M3 values under one E8M0 power-of-two scale ("Miles Blackwell
// RL Troca a Uniformidade BF16 por MXFP8 e NVFP4 Nativos", section "O Suporte
// Miles Blackwell Agora Abrange Todo o Loop de RL").  Blocks follow the GEMM
// reduction dimension, so the rowwise and the columnwise copy are both made
// from the BF16 original (same page, section "Um Quantizador Compartilhado É o
// Verdadeiro Mecanismo").
//
// Block exponent: the smallest e in [-127, 127] with amax <= 448 * 2^e.
// With amax = 1.m * 2^p taken from the BF16 magnitude bits (exponent field E,
// 7-bit mantissa M), amax <= 1.75 * 2^p iff M <= 96, so
//     e + 127 = max(0, E - 8 + (M > 96))
// which also covers amax = 0 and BF16 subnormals (both give code 0).
// Codes: E4M3 round-to-nearest-even of x * 2^-e (exact scaling, never > 448).
//
// These are bandwidth kernels: 16-byte loads per lane, block max over four
// lanes with lane shuffles, 8-byte code stores, and the scale byte written
// straight into the layout the GEMM reads (no separate rearrangement pass).

#include "mxq_device.h"
#include "mxq_kernels.h"

namespace mxq {

__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax16) {
  int E = (int)(amax16 >> 7);
  int M = (int)(amax16 & 0x7F);
  int code = E - 8 + (M > 96 ? 1 : 0);
  return (uint32_t)(code < 0 ? 0 : code);
}

// Encode 8 BF16 values (in 4 words) with block exponent code s (e = s - 127):
// returns 8 E4M3 bytes in two words.
__device__ __forceinline__ uint2 mx_encode8(uint4 v, uint32_t s) {
  int sh = 127 - (int)s;   // multiply by 2^-e
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = __builtin_ldexpf(bf16_lo(w[i]), sh);
    float b = __builtin_ldexpf(bf16_hi(w[i]), sh);
    o[i] = f32x2_to_e4m3(a, b);
  }
  return make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
}

__device__ __forceinline__ uint32_t absmax8(uint4 v) {
  return umax(umax(bf16x2_absmax_bits(v.x), bf16x2_absmax_bits(v.y)),
              umax(bf16x2_absmax_bits(v.z), bf16x2_absmax_bits(v.w)));
}

// ---------------------------------------------------------------- ROW 1x32
// One lane per 8 elements, 4 lanes per block; each lane handles UNROLL chunks
// spaced a grid apart so several 16-byte loads are in flight.
template <int UNROLL>
__global__ __launch_bounds__(256) void mxfp8_row_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales, int mfma_layout) {
  const int64_t cpr = cols >> 3;                 // chunks per row
  const int64_t total = rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; base < total + 0; base += stride * UNROLL) {
    uint4 v[UNROLL];
    int64_t id[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      id[u] = base + (int64_t)u * stride;
      int64_t r = id[u] / cpr, c = id[u] - r * cpr;
      v[u] = id[u] < total ? *reinterpret_cast<const uint4*>(x + r * ld_x + c * 8)
                           : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      uint32_t m = absmax8(v[u]);
      m = umax(m, lane_xor_u32(m, 1));
      m = umax(m, lane_xor_u32(m, 2));
      uint32_t s = e8m0_from_amax_bits(m);
      if (id[u] < total) {
        int64_t r = id[u] / cpr, c = id[u] - r * cpr;
        uint2 out = mx_encode8(v[u], s);
        *reinterpret_cast<uint2*>(codes + r * ld_codes + c * 8) = out;
        if ((c & 3) == 0) scales[scale_offset(r, c >> 2, cols >> 5, mfma_layout)] = (uint8_t)s;
      }
    }
  }
}

// ------------------------------------------------ COL / TILE / DUAL (LDS tile)
// A workgroup stages a 32-row x 256-column BF16 tile in LDS.
//  * rowwise part (ROW copy of DUAL): one thread per (row, 32-column block);
//  * columnwise part (COL, DUAL): one thread per column, 32 rows, stored into
//    the transposed copy as 32 contiguous bytes;
//  * TILE: one thread per (row, block); the 32x32 amax is a 32-lane reduction;
//    optionally also the transposed copy (the same codes, tile grid transposed).
constexpr int TROWS = 32, TCOLS = 256, TPAD = 8;   // pad breaks LDS bank aliasing

template <int MODE>   // 0 = COL, 1 = TILE, 2 = DUAL
__global__ __launch_bounds__(256) void mxfp8_tile_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ codes_col, int64_t ld_codes_col, uint8_t* __restrict__ scales_col,
    int mfma_layout) {
  __shared__ uint16_t tile[TROWS][TCOLS + TPAD];
  const int64_t r0 = (int64_t)blockIdx.y * TROWS;
  const int64_t c0 = (int64_t)blockIdx.x * TCOLS;
  const int t = threadIdx.x;
  // load: 32 rows x 256 cols = 1024 chunks of 8, 4 per thread
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int chunk = t + 256 * k;
    int rr = chunk >> 5, cc = (chunk & 31) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c0 + cc < cols) v = *reinterpret_cast<const uint4*>(x + (r0 + rr) * ld_x + c0 + cc);
    *reinterpret_cast<uint4*>(&tile[rr][cc]) = v;
  }
  __syncthreads();

  if (MODE == 1 || MODE == 2) {
    // (row, block) per thread: threads 0..31 = rows 0..31 of block 0, etc.
    const int rr = t & 31, blk = t >> 5;
    const int cc = blk * 32;
    const bool valid = c0 + cc < cols;
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint4*>(&tile[rr][cc + 8 * q]);
    uint32_t m = umax(umax(absmax8(v[0]), absmax8(v[1])), umax(absmax8(v[2]), absmax8(v[3])));
    if (MODE == 1) {
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) m = umax(m, lane_xor_u32(m, o));
    }
    uint32_t s = e8m0_from_amax_bits(m);
    if (valid) {
      uint2 o0 = mx_encode8(v[0], s), o1 = mx_encode8(v[1], s);
      uint2 o2 = mx_encode8(v[2], s), o3 = mx_encode8(v[3], s);
      uint8_t* dst = codes + (r0 + rr) * ld_codes + c0 + cc;
      *reinterpret_cast<uint4*>(dst) = make_uint4(o0.x, o0.y, o1.x, o1.y);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o2.x, o2.y, o3.x, o3.y);
      if (MODE == 1) {
        if (rr == 0) scales[(r0 >> 5) * (cols >> 5) + ((c0 + cc) >> 5)] = (uint8_t)s;
      } else {
        scales[scale_offset(r0 + rr, (c0 + cc) >> 5, cols >> 5, mfma_layout)] = (uint8_t)s;
      }
    }
    // TILE with a transposed copy: a 32x32 tile's scale is shared by its rows
    // and columns, so the transposed copy is the same codes transposed.  The
    // thread of (row rr, block blk) also encodes column 32 blk + rr of the
    // staged tile with the block's scale s (it holds s after the reduction)
    // and writes it as 32 contiguous bytes of codes_col [cols, rows].
    if (MODE == 1 && codes_col) {
      const int ct = cc + rr;                        // tile column of this thread
      if (c0 + ct < cols) {
        uint32_t col[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          col[q] = (uint32_t)tile[2 * q][ct] | ((uint32_t)tile[2 * q + 1][ct] << 16);
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint2 e = mx_encode8(make_uint4(col[4 * q], col[4 * q + 1], col[4 * q + 2], col[4 * q + 3]), s);
          o[2 * q] = e.x;
          o[2 * q + 1] = e.y;
        }
        uint8_t* dst = codes_col + (c0 + ct) * ld_codes_col + r0;
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
        if (rr == 0) scales_col[((c0 + cc) >> 5) * (rows >> 5) + (r0 >> 5)] = (uint8_t)s;
      }
    }
  }
  if (MODE == 0 || MODE == 2) {
    uint8_t* dcodes = MODE == 0 ? codes : codes_col;
    uint8_t* dscales = MODE == 0 ? scales : scales_col;
    const int64_t ldc = MODE == 0 ? ld_codes : ld_codes_col;
    const int cc = t;                      // one column per thread
    if (c0 + cc < cols) {
      uint32_t col[16];                    // 32 values, two per word (row pairs)
      uint32_t m = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        uint32_t a = tile[2 * q][cc], b = tile[2 * q + 1][cc];
        col[q] = a | (b << 16);
        m = umax(m, bf16x2_absmax_bits(col[q]));
      }
      uint32_t s = e8m0_from_amax_bits(m);
      uint32_t o[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 e = mx_encode8(make_uint4(col[4 * q], col[4 * q + 1], col[4 * q + 2], col[4 * q + 3]), s);
        o[2 * q] = e.x;
        o[2 * q + 1] = e.y;
      }
      uint8_t* dst = dcodes + (c0 + cc) * ldc + r0;
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
      dscales[scale_offset(c0 + cc, r0 >> 5, rows >> 5, mfma_layout)] = (uint8_t)s;
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_mxfp8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* codes, int64_t ld_codes, uint8_t* scales, bool mfma,
                            hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  constexpr int UNROLL = 4;
  int64_t blocks = (total + 256 * UNROLL - 1) / (256 * UNROLL);
  if (blocks < 1) blocks = 1;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  hipLaunchKernelGGL((mxfp8_row_kernel<UNROLL>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                     rows, cols, ld_x, codes, ld_codes, scales, (int)mfma);
  return hipGetLastError();
}

hipError_t launch_mxfp8_tile(int mode, const uint16_t* x, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                             uint8_t* codes_col, int64_t ld_codes_col, uint8_t* scales_col,
                             bool mfma, hipStream_t st) {
  dim3 grid((unsigned)((cols + TCOLS - 1) / TCOLS), (unsigned)(rows / TROWS));
  if (grid.y > 65535u) return hipErrorInvalidValue;      // more row strips than a grid holds
  if (mode == 0)
    hipLaunchKernelGGL((mxfp8_tile_kernel<0>), grid, dim3(256), 0, st, x, rows, cols, ld_x,
                       codes, ld_codes, scales, codes_col, ld_codes_col, scales_col, (int)mfma);
  else if (mode == 1)
    hipLaunchKernelGGL((mxfp8_tile_kernel<1>), grid, dim3(256), 0, st, x, rows, cols, ld_x,
                       codes, ld_codes, scales, codes_col, ld_codes_col, scales_col, (int)mfma);
  else
    hipLaunchKernelGGL((mxfp8_tile_kernel<2>), grid, dim3(256), 0, st, x, rows, cols, ld_x,
                       codes, ld_codes, scales, codes_col, ld_codes_col, scales_col, (int)mfma);
  return hipGetLastError();
}

}  // namespace mxq
