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

// Blockwise FP8 with binary32 scales (F32S): s = amax / 448 (one correctly
// rounded division), codes E4M3 RNE of the binary32 quotient x / s clamped to
// +-448 (the quotient of the block maximum may exceed 448 by an ulp); a zero
// block stores s = 0 and zero codes.  A scale travels as its binary32 bits in
// the same uint32_t that carries an E8M0 code otherwise.
__device__ __forceinline__ uint32_t f32s_from_amax_bits(uint32_t amax16) {
  return __float_as_uint(__uint_as_float(amax16 << 16) / 448.0f);
}

// The quotient without a division per element: with r = RN(1/s) (one
// correctly rounded division per block), q0 = RN(x r), the exact residual
// x - q0 s by one FMA and the corrected q0 + residual * r by another.  The
// result can differ from RN(x / s) in its last bits, but for every BF16 x in
// a block and every scale s >= 2^-80 of a BF16 block maximum it gives the
// same E4M3 code (an exhaustive check over all 1.0e9 such pairs is among the
// host tests); smaller scales divide directly.
// (The sign is x's: for x = -0 the corrected sum would come out +0.)
__device__ __forceinline__ float f32s_quotient(float x, float sc, float r) {
  const float q0 = x * r;
  return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, sc, x), r, q0), x);
}

__device__ __forceinline__ uint2 f32s_encode8(uint4 v, uint32_t sbits) {
  const float sc = __uint_as_float(sbits);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float q[8];
  if (sbits == 0u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = 0.0f;
  } else if (sc < 0x1p-80f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = bf16_lo(w[i]) / sc;
      q[2 * i + 1] = bf16_hi(w[i]) / sc;
    }
  } else {
    const float r = 1.0f / sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = f32s_quotient(bf16_lo(w[i]), sc, r);
      q[2 * i + 1] = f32s_quotient(bf16_hi(w[i]), sc, r);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32x2_to_e4m3(fminf(fmaxf(q[2 * i], -448.0f), 448.0f), fminf(fmaxf(q[2 * i + 1], -448.0f), 448.0f));
  return make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
}

template <bool F32S>
__device__ __forceinline__ uint32_t blk_scale(uint32_t amax16) {
  if constexpr (F32S) return f32s_from_amax_bits(amax16);
  return e8m0_from_amax_bits(amax16);
}

template <bool F32S>
__device__ __forceinline__ uint2 blk_encode8(uint4 v, uint32_t s) {
  if constexpr (F32S) return f32s_encode8(v, s);
  return mx_encode8(v, s);
}

// store scale s at element index i of a byte (E8M0) or binary32 scale array
template <bool F32S>
__device__ __forceinline__ void blk_store(uint8_t* scales, int64_t i, uint32_t s) {
  if constexpr (F32S) reinterpret_cast<float*>(scales)[i] = __uint_as_float(s);
  else scales[i] = (uint8_t)s;
}

// ---------------------------------------------------------------- ROW 1x32
// One lane per 8 elements, LPB lanes per block (4: MXFP8's 32 values; 16: a
// 128-value blockwise-FP8 block); each lane handles UNROLL chunks spaced a
// grid apart so several 16-byte loads are in flight.  A block's lanes are
// aligned and consecutive (cols is a multiple of the block), so they run the
// loop's iterations together and can exchange their maxima.
template <int UNROLL, int LPB, bool F32S = false>
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
#pragma unroll
      for (int o = 1; o < LPB; o <<= 1) m = umax(m, lane_xor_u32(m, o));
      uint32_t s = blk_scale<F32S>(m);
      if (id[u] < total) {
        int64_t r = id[u] / cpr, c = id[u] - r * cpr;
        uint2 out = blk_encode8<F32S>(v[u], s);
        *reinterpret_cast<uint2*>(codes + r * ld_codes + c * 8) = out;
        if (c % LPB == 0) blk_store<F32S>(scales, scale_offset(r, c / LPB, cols / (8 * LPB), mfma_layout), s);
      }
    }
  }
}

// ------------------------------------------------ COL / TILE / DUAL (LDS tile)
// A workgroup stages a 128-row x 128-column BF16 tile in LDS (16-byte loads,
// each wave instruction four whole 256-byte row segments), then:
//  * rowwise part (ROW copy of DUAL, TILE): thread = (row, 32-column block),
//    block index fastest, so the four lanes of a row write its 128 code bytes
//    side by side;
//  * columnwise part (COL, DUAL, TILE's transposed copy): thread = (column,
//    32-row group), group fastest, so the four threads of a column write its
//    128 bytes of the transposed copy side by side;
//  * TILE: a wave's rows are one 32-row group, so the 32x32 amax is a
//    reduction over the wave's lanes of one block; the transposed copy reads
//    the tile scales through LDS.
// LDS holds 16-byte chunks (8 columns) of each 256-byte row; chunk ch of row
// r sits at slot ch ^ (r & 3) ^ (4 * ((r >> 5) & 3)).  The first term spreads
// the four rows read together by the rowwise part over all 16 slots, the
// second spreads the four 32-row groups read together by the columnwise part
// over the banks.
constexpr int TR = 128, TC = 128;

__device__ __forceinline__ int mx_slot(int r, int ch) {
  return r * 16 + (ch ^ (r & 3) ^ (((r >> 5) & 3) << 2));
}

// B128 (blockwise FP8, power-of-two scales): the blocks are 128 wide, so a
// row's block is the tile's whole row (its four 32-column maxima combined by
// two lane exchanges), a column's block the tile's whole column (its four
// 32-row groups likewise), and TILE's block the whole 128x128 tile (a wave
// reduction, then the four waves through LDS).  Scales are linear:
// [rows, cols/128], [cols, rows/128], [rows/128, cols/128].  The shapes are
// whole tiles (checked on the host).
template <int MODE, bool B128, bool F32S = false>   // MODE 0 = COL, 1 = TILE, 2 = DUAL
__global__ __launch_bounds__(256) void mxfp8_tile_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ codes_col, int64_t ld_codes_col, uint8_t* __restrict__ scales_col,
    int mfma_layout) {
  __shared__ uint4 tile[TR * TC / 8];
  __shared__ uint32_t tscale[4][4];            // TILE: scale of 32x32 tile (group, block)
  __shared__ uint32_t wmax[4];                 // TILE with B128: each wave's maximum
  const int64_t r0 = (int64_t)blockIdx.y * TR;
  const int64_t c0 = (int64_t)blockIdx.x * TC;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = t + 256 * k, r = i >> 4, ch = i & 15;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < rows && c0 + ch * 8 < cols)
      v = *reinterpret_cast<const uint4*>(x + (r0 + r) * ld_x + c0 + ch * 8);
    tile[mx_slot(r, ch)] = v;
  }
  __syncthreads();

  if (MODE == 1 || MODE == 2) {
    // wave w owns rows 32w .. 32w + 31 (one 32-row group): lane l takes row
    // 32w + 16k + l / 4, block l % 4
    const int w = t >> 6, l = t & 63, j = l & 3;
    uint4 v[2][4];
    uint32_t m[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 32 * w + 16 * k + (l >> 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[k][q] = tile[mx_slot(r, 4 * j + q)];
      m[k] = umax(umax(absmax8(v[k][0]), absmax8(v[k][1])), umax(absmax8(v[k][2]), absmax8(v[k][3])));
    }
    uint32_t s[2];
    if (MODE == 1) {
      uint32_t mt = umax(m[0], m[1]);
#pragma unroll
      for (int o = 4; o < 64; o <<= 1) mt = umax(mt, lane_xor_u32(mt, o));
      if (B128) {
        mt = umax(mt, lane_xor_u32(mt, 1));
        mt = umax(mt, lane_xor_u32(mt, 2));
        if (l == 0) wmax[w] = mt;
        __syncthreads();
        mt = umax(umax(wmax[0], wmax[1]), umax(wmax[2], wmax[3]));
      }
      s[0] = s[1] = blk_scale<F32S>(mt);
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (B128) {
          m[k] = umax(m[k], lane_xor_u32(m[k], 1));
          m[k] = umax(m[k], lane_xor_u32(m[k], 2));
        }
        s[k] = blk_scale<F32S>(m[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 32 * w + 16 * k + (l >> 2);
      if (r0 + r < rows && c0 + 32 * j < cols) {
        const uint2 o0 = blk_encode8<F32S>(v[k][0], s[k]), o1 = blk_encode8<F32S>(v[k][1], s[k]);
        const uint2 o2 = blk_encode8<F32S>(v[k][2], s[k]), o3 = blk_encode8<F32S>(v[k][3], s[k]);
        uint8_t* dst = codes + (r0 + r) * ld_codes + c0 + 32 * j;
        *reinterpret_cast<uint4*>(dst) = make_uint4(o0.x, o0.y, o1.x, o1.y);
        *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o2.x, o2.y, o3.x, o3.y);
        if (MODE == 1) {
          if (B128) {
            if (t == 0) {
              blk_store<F32S>(scales, (r0 >> 7) * (cols >> 7) + (c0 >> 7), s[k]);
              tscale[0][0] = s[k];
            }
          } else if ((r & 31) == 0) {
            scales[((r0 + r) >> 5) * (cols >> 5) + ((c0 >> 5) + j)] = (uint8_t)s[k];
            tscale[w][j] = s[k];
          }
        } else if (B128) {
          if (j == 0) blk_store<F32S>(scales, (r0 + r) * (cols >> 7) + (c0 >> 7), s[k]);
        } else {
          scales[scale_offset(r0 + r, (c0 >> 5) + j, cols >> 5, mfma_layout)] = (uint8_t)s[k];
        }
      }
    }
  }
  if (MODE == 0 || MODE == 2 || (MODE == 1 && codes_col)) {
    if (MODE == 1) __syncthreads();              // tscale
    uint8_t* dcodes = MODE == 0 ? codes : codes_col;
    uint8_t* dscales = MODE == 0 ? scales : scales_col;
    const int64_t ldc = MODE == 0 ? ld_codes : ld_codes_col;
    const uint16_t* tv = reinterpret_cast<const uint16_t*>(tile);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = t + 256 * k, g = i & 3, c = i >> 2;
      uint32_t col[16];                          // 32 values, two per word (row pairs)
      uint32_t m = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t a = tv[mx_slot(32 * g + 2 * q, c >> 3) * 8 + (c & 7)];
        const uint32_t b = tv[mx_slot(32 * g + 2 * q + 1, c >> 3) * 8 + (c & 7)];
        col[q] = a | (b << 16);
        m = umax(m, bf16x2_absmax_bits(col[q]));
      }
      if (B128) {                                // the column's four 32-row groups
        m = umax(m, lane_xor_u32(m, 1));
        m = umax(m, lane_xor_u32(m, 2));
      }
      if (r0 + 32 * g >= rows || c0 + c >= cols) continue;
      const uint32_t s = MODE == 1 ? (B128 ? tscale[0][0] : tscale[g][c >> 5]) : blk_scale<F32S>(m);
      uint32_t o[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint2 e = blk_encode8<F32S>(make_uint4(col[4 * q], col[4 * q + 1], col[4 * q + 2], col[4 * q + 3]), s);
        o[2 * q] = e.x;
        o[2 * q + 1] = e.y;
      }
      uint8_t* dst = dcodes + (c0 + c) * ldc + r0 + 32 * g;
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
      if (MODE == 1) {
        if (B128) {
          if (t == 0 && k == 0) blk_store<F32S>(scales_col, (c0 >> 7) * (rows >> 7) + (r0 >> 7), s);
        } else if ((c & 31) == 0) {
          scales_col[((c0 + c) >> 5) * (rows >> 5) + ((r0 >> 5) + g)] = (uint8_t)s;
        }
      } else if (B128) {
        if (g == 0) blk_store<F32S>(dscales, (c0 + c) * (rows >> 7) + (r0 >> 7), s);
      } else {
        dscales[scale_offset(c0 + c, (r0 >> 5) + g, rows >> 5, mfma_layout)] = (uint8_t)s;
      }
    }
  }
}

// TILE without the transposed copy: a 32-row x 256-column tile per workgroup
// (twice the workgroups of the 128x128 kernel, which pays off when nothing is
// written column-wise).  Thread = (row, block) with the row fastest, so the
// 32 lanes of a block hold the tile's 32 rows and the 32x32 amax is a lane
// reduction.
constexpr int T32R = 32, T32C = 256, T32PAD = 8;   // pad breaks LDS bank aliasing

__global__ __launch_bounds__(256) void mxfp8_tile32_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales) {
  __shared__ uint16_t tile[T32R][T32C + T32PAD];
  const int64_t r0 = (int64_t)blockIdx.y * T32R;
  const int64_t c0 = (int64_t)blockIdx.x * T32C;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int chunk = t + 256 * k, rr = chunk >> 5, cc = (chunk & 31) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c0 + cc < cols) v = *reinterpret_cast<const uint4*>(x + (r0 + rr) * ld_x + c0 + cc);
    *reinterpret_cast<uint4*>(&tile[rr][cc]) = v;
  }
  __syncthreads();
  const int rr = t & 31, cc = (t >> 5) * 32;
  uint4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint4*>(&tile[rr][cc + 8 * q]);
  uint32_t m = umax(umax(absmax8(v[0]), absmax8(v[1])), umax(absmax8(v[2]), absmax8(v[3])));
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) m = umax(m, lane_xor_u32(m, o));
  const uint32_t s = e8m0_from_amax_bits(m);
  if (c0 + cc < cols) {
    const uint2 o0 = mx_encode8(v[0], s), o1 = mx_encode8(v[1], s);
    const uint2 o2 = mx_encode8(v[2], s), o3 = mx_encode8(v[3], s);
    uint8_t* dst = codes + (r0 + rr) * ld_codes + c0 + cc;
    *reinterpret_cast<uint4*>(dst) = make_uint4(o0.x, o0.y, o1.x, o1.y);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o2.x, o2.y, o3.x, o3.y);
    if (rr == 0) scales[(r0 >> 5) * (cols >> 5) + ((c0 + cc) >> 5)] = (uint8_t)s;
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_mxfp8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* codes, int64_t ld_codes, uint8_t* scales, bool mfma, int b128,
                            hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  constexpr int UNROLL = 4;
  int64_t blocks = (total + 256 * UNROLL - 1) / (256 * UNROLL);
  if (blocks < 1) blocks = 1;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  if (b128 == 2)
    hipLaunchKernelGGL((mxfp8_row_kernel<UNROLL, 16, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                       x, rows, cols, ld_x, codes, ld_codes, scales, 0);
  else if (b128)
    hipLaunchKernelGGL((mxfp8_row_kernel<UNROLL, 16>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                       rows, cols, ld_x, codes, ld_codes, scales, 0);
  else
    hipLaunchKernelGGL((mxfp8_row_kernel<UNROLL, 4>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                       rows, cols, ld_x, codes, ld_codes, scales, (int)mfma);
  return hipGetLastError();
}

hipError_t launch_mxfp8_tile(int mode, const uint16_t* x, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                             uint8_t* codes_col, int64_t ld_codes_col, uint8_t* scales_col,
                             bool mfma, int b128, hipStream_t st) {
  if (mode == 1 && !codes_col && !b128) {
    dim3 g32((unsigned)((cols + T32C - 1) / T32C), (unsigned)(rows / T32R));
    if (g32.y > 65535u) return hipErrorInvalidValue;     // more row strips than a grid holds
    hipLaunchKernelGGL(mxfp8_tile32_kernel, g32, dim3(256), 0, st, x, rows, cols, ld_x, codes,
                       ld_codes, scales);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((cols + TC - 1) / TC), (unsigned)((rows + TR - 1) / TR));
  if (grid.y > 65535u) return hipErrorInvalidValue;      // more row strips than a grid holds
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, x, rows, cols, ld_x, codes, ld_codes, scales,
                       codes_col, ld_codes_col, scales_col, (int)mfma);
  };
  if (b128 == 2) {
    if (mode == 0) go(mxfp8_tile_kernel<0, true, true>);
    else if (mode == 1) go(mxfp8_tile_kernel<1, true, true>);
    else go(mxfp8_tile_kernel<2, true, true>);
  } else if (b128) {
    if (mode == 0) go(mxfp8_tile_kernel<0, true>);
    else if (mode == 1) go(mxfp8_tile_kernel<1, true>);
    else go(mxfp8_tile_kernel<2, true>);
  } else {
    if (mode == 0) go(mxfp8_tile_kernel<0, false>);
    else if (mode == 1) go(mxfp8_tile_kernel<1, false>);
    else go(mxfp8_tile_kernel<2, false>);
  }
  return hipGetLastError();
}

}  // namespace mxq
