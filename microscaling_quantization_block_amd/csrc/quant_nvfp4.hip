// NVFP4 quantizers for gfx950.
//
// NVFP4 = 16 E2M1 values with an E4M3 block scale under a second FP32 scale
// ("Miles Blackwell RL Troca a Uniformidade BF16 por MXFP8 e NVFP4 Nativos",
// section "O Suporte Miles Blackwell Agora Abrange Todo o Loop de RL").  Miles
// computes the second scale per token online and fuses it into the activation
// quantizer, which yields packed FP4, block scales and token scales in one op
// (same page, section "Um Quantizador Compartilhado É o Verdadeiro
// Mecanismo"); the NVIDIA pretraining recipe uses a per-tensor scale, 16x16
// weight tiles, and stochastic rounding for gradients ("Train models faster
// with JAX and MaxText using NVFP4 on NVIDIA Blackwell", section "NVFP4
// pretraining recipe").
//
// Binary32 chain (each step one IEEE operation, RNE, subnormals kept, no FMA):
//   S   = A / 2688                 (A = max|x| of the row or tensor)
//   s_b = E4M3_RNE(a_b / (6 * S))  (0 when S == 0)
//   r   = 1 / (s_b * S)            (once per block)
//   q   = E2M1(x * r)              (RNE, or SR with a Philox4x32-10 draw)
// When S < 2^-64, s_b * S can fall below the binary32 normal range (its
// reciprocal would lose bits or overflow, and a zero times infinity is NaN),
// so r and q are taken in a frame scaled by 2^64: r = 1 / (s_b * (S * 2^64)),
// q = E2M1((x * 2^64) * r).  Every scaling by 2^64 is exact, so wherever
// s_b * S is normal this gives the unscaled result.  S is uniform across a
// wave (one wave per token, or one S per tensor), so the kernels branch on it
// once and the common path pays nothing.
// Divisions are the correctly rounded IEEE ones (the build keeps HIP's
// correctly rounded fp32 division and sqrt).
//
// Kernels:
//   * nvfp4_row_kernel: one wave per row, the row held in registers, the
//     token amax a wave reduction; 16-byte loads, two lanes per 16-block.
//   * nvfp4_tile16_kernel: each lane owns 8 columns x 16 rows; two lanes form
//     a 16x16 tile.
//   * nvfp4_col_kernel: each lane owns 8 columns x 16 rows, each column one
//     16x1 block, written into the transposed copy (optionally after the
//     random Hadamard transform of the 16 rows).
//   * nvfp4_col_pair_kernel: the same copy without the transform, each
//     16-row block split over two lanes (with stochastic rounding, registers
//     for four waves per SIMD instead of two).
//   * per-tensor scale: a one-thread kernel zeroes gscale[0], then an
//     unsigned atomic max on the magnitude bits (exact and order-independent)
//     leaves A there tagged with bit 31.  The quantize kernel that follows
//     decodes it (S = A / 2688) and every block writes the same S back, so
//     gscale[0] ends as S whatever order the blocks run in, and a block that
//     reads after another's write-back sees S itself (untagged).

#include "mxq_device.h"
#include "mxq_kernels.h"
#include "nvfp4_device.h"

#include <type_traits>

namespace mxq {

// ------------------------------------------------------------ Four-Over-Six
// "NVFP4 RL training" / "The 4-bitter Lesson", section on Four-Over-Six for
// RL weights and activations: a block may scale its max onto 4 instead of 6,
// which moves values near the max out of the grid's widest gap.  Each block
// is encoded under both block scales (a_b / (6 S) and a_b / (4 S), E4M3,
// saturating), and keeps 4 iff the binary32 sum of squared dequantization
// errors is strictly smaller.  The sum is a pairwise tree in element order
// (neighbours first); for a 16x16 tile, each row's 16 squares by that tree,
// then the 16 row sums by it in row order.  A dequantized value is
// fl(fl(value(code) s_b) S), as the dequantizer computes it.

// Squares of the 8 errors of one chunk (BF16 values v, codes q), summed by
// the first three levels of the tree.
__device__ __forceinline__ float nv_sse8(uint4 v, uint32_t q, float sb, float S) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  mxq_f32x2 c[4];
  c[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  c[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  c[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  c[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ea = bf16_lo(w[i]) - (c[i].x * sb) * S;
    const float eb = bf16_hi(w[i]) - (c[i].y * sb) * S;
    p[i] = ea * ea + eb * eb;                 // three roundings, no fused multiply-add
  }
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// One candidate's codes for a chunk of 8 values and the chunk's error sum.
struct Cand8 { uint32_t q; float e; };
template <bool TINY>
__device__ __forceinline__ Cand8 nv_cand8(uint4 v, const BlockScale& bs, float S) {
  const u32x4 none = {0, 0, 0, 0};
  Cand8 c;
  c.q = nv_encode8<false, TINY>(v, bs.r, none);
  c.e = nv_sse8(v, c.q, e4m3_to_f32(bs.code), S);
  return c;
}

// A whole 16-value block held by one lane: the chosen scale code and codes.
struct Enc16 { uint32_t code, q0, q1; };
template <bool TINY>
__device__ __forceinline__ Enc16 nv_encode16_46(uint4 v0, uint4 v1, float a_b, float S) {
  const BlockScale b6 = nv_block_scale(a_b, S, 6.0f), b4 = nv_block_scale(a_b, S, 4.0f);
  const Cand8 x60 = nv_cand8<TINY>(v0, b6, S), x61 = nv_cand8<TINY>(v1, b6, S);
  const Cand8 x40 = nv_cand8<TINY>(v0, b4, S), x41 = nv_cand8<TINY>(v1, b4, S);
  const float e6 = x60.e + x61.e, e4 = x40.e + x41.e;
  if (e4 < e6) return Enc16{b4.code, x40.q, x41.q};
  return Enc16{b6.code, x60.q, x61.q};
}

// Second-level scale of a tensor-scaled call.  gmode 1: gscale[0] holds the
// tagged amax (bit 31 set) or, once some block wrote it back, S itself.
// gmode 2: S given by the caller.
__device__ __forceinline__ float tensor_scale(const float* g, int gmode) {
  const uint32_t v = __float_as_uint(g[0]);
  if (gmode == 1 && (v >> 31)) return __uint_as_float(v & 0x7FFFFFFFu) / 2688.0f;
  return __uint_as_float(v);
}

// Tensor amax accumulated by a rowwise per-token pass (for the columnwise
// per-tensor copy made next from the same tensor): the tagged binary32
// magnitude bits of a row (or a wave's rows) go into *amax_out by an unsigned
// atomic max, skipped when the value there is already at least as large (a
// stale read only costs an extra atomic; the maximum is order-independent).
__device__ __forceinline__ void amax_accumulate(uint32_t* amax_out, uint32_t bits) {
  const uint32_t tagged = bits | 0x80000000u;
  if (__hip_atomic_load(amax_out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < tagged)
    atomicMax(amax_out, tagged);
}

// ------------------------------------------------------------ ROW (1x16)
// gmode: 0 = per row (S computed here and stored), 1 = per tensor (tagged
// amax, see tensor_scale), 2 = given.  One wave per row; lane owns the
// 16-value blocks b = lane + 64k (k < BPT): two 16-byte loads, the block amax
// and scale chain in the lane, 8 code bytes out.  Each wave walks rows row0,
// row0 + W, ... (W = waves in the grid) with the next row's loads in flight
// while the current one is encoded; a prefetch past the end is clamped to
// the last row (a valid address, never used).  FULL: every lane's blocks
// exist (cols == 1024 BPT).
// RM: 0 = RNE, 1 = stochastic rounding, 2 = RNE with the Four-Over-Six choice.
// amax_out (per-token mode only, else nullptr): also accumulate the tensor
// amax there (see amax_accumulate), one atomic per wave.
template <int BPT, int RM, bool FULL>
__global__ __launch_bounds__(256) void nvfp4_row_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ bscales,
    float* __restrict__ gscales, int gmode, int mfma_layout,
    uint64_t seed, uint32_t stream_id, uint32_t tensor_tag, uint32_t* __restrict__ amax_out) {
  constexpr bool SR = RM == 1;
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * 4;
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;                       // whole wave leaves together
  const int64_t bpr = cols >> 4;
  float St = 0.0f;
  if (gmode != 0) {
    St = tensor_scale(gscales, gmode);
    if (gmode == 1 && threadIdx.x == 0) gscales[0] = St;
  }
  auto load = [&](int64_t r, uint4 (*v)[2]) {
    const uint16_t* xr = x + (r < rows ? r : rows - 1) * ld_x;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int64_t b = lane + 64 * k;
      const int64_t bb = FULL ? b : (b < bpr ? b : bpr - 1);
      v[k][0] = *reinterpret_cast<const uint4*>(xr + bb * 16);
      v[k][1] = *reinterpret_cast<const uint4*>(xr + bb * 16 + 8);
    }
  };
  uint32_t wave_amax = 0;
  auto process = [&](int64_t r, uint4 (*v)[2]) {
    uint32_t ab[BPT];
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      ab[k] = umax(amax8_bits(v[k][0]), amax8_bits(v[k][1]));
      if (!FULL && lane + 64 * k >= bpr) ab[k] = 0;
    }
    float S = St;
    if (gmode == 0) {
      uint32_t mb = ab[0];
#pragma unroll
      for (int k = 1; k < BPT; ++k) mb = umax(mb, ab[k]);
      mb = wave_max_u32(mb);
      wave_amax = umax(wave_amax, mb);
      S = __uint_as_float(mb) / 2688.0f;
      if (lane == 0) gscales[r] = S;
    }
    with_frame(S, [&](auto tiny) {
      constexpr bool TINY = decltype(tiny)::value;
#pragma unroll
      for (int k = 0; k < BPT; ++k) {
        const int64_t b = lane + 64 * k;
        if (FULL || b < bpr) {
          uint32_t q0, q1, code;
          if (RM == 2) {
            const Enc16 e = nv_encode16_46<TINY>(v[k][0], v[k][1], __uint_as_float(ab[k]), S);
            q0 = e.q0;
            q1 = e.q1;
            code = e.code;
          } else {
            const BlockScale bs = nv_block_scale(__uint_as_float(ab[k]), S);
            u32x4 d0 = {0, 0, 0, 0}, d1 = {0, 0, 0, 0};
            if (SR) {
              const uint64_t n = (uint64_t)(r * cols + b * 16) >> 3;
              d0 = philox_draws8(n, seed, stream_id, tensor_tag);
              d1 = philox_draws8(n + 1, seed, stream_id, tensor_tag);
            }
            q0 = nv_encode8<SR, TINY>(v[k][0], bs.r, d0);
            q1 = nv_encode8<SR, TINY>(v[k][1], bs.r, d1);
            code = bs.code;
          }
          *reinterpret_cast<uint2*>(codes + r * ld_codes + b * 8) = make_uint2(q0, q1);
          bscales[scale_offset(r, b, bpr, mfma_layout)] = (uint8_t)code;
        }
      }
    });
  };
  uint4 va[BPT][2], vb[BPT][2];
  load(row, va);
  while (true) {                                 // trip count uniform across the wave
    load(row + W, vb);
    process(row, va);
    row += W;
    if (row >= rows) break;
    load(row + W, va);
    process(row, vb);
    row += W;
    if (row >= rows) break;
  }
  if (amax_out && lane == 0) amax_accumulate(amax_out, wave_amax);
}

// Long rows (more than 8192 values, up to 32768): one workgroup of 256
// threads per row, the whole row held in registers, so the row is read from
// HBM once.  Thread t owns chunks c = t + 256 i (8 values each, i < CPT); a
// 16-value block is the chunk pair (c, c ^ 1), held by threads t and t ^ 1 of
// one wave.  The token amax is a wave reduction, then one across the four
// waves through LDS.  Same arithmetic as the one-wave kernels.
template <int CPT, int RM>
__global__ __launch_bounds__(256) void nvfp4_row_wg_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ bscales,
    float* __restrict__ gscales, int gmode, int mfma_layout,
    uint64_t seed, uint32_t stream_id, uint32_t tensor_tag, uint32_t* __restrict__ amax_out) {
  constexpr bool SR = RM == 1;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int cpr = (int)(cols >> 3);
  const uint16_t* xr = x + row * ld_x;
  uint4 v[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    v[i] = c < cpr ? *reinterpret_cast<const uint4*>(xr + (int64_t)c * 8) : make_uint4(0, 0, 0, 0);
  }
  uint32_t ab[CPT];
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    ab[i] = amax8_bits(v[i]);
    mb = umax(mb, ab[i]);
  }
  float S;
  if (gmode == 0) {
    __shared__ uint32_t wmax[4];
    mb = wave_max_u32(mb);
    if ((tid & 63) == 0) wmax[tid >> 6] = mb;
    __syncthreads();
    mb = umax(umax(wmax[0], wmax[1]), umax(wmax[2], wmax[3]));
    S = __uint_as_float(mb) / 2688.0f;
    if (tid == 0) {
      gscales[row] = S;
      if (amax_out) amax_accumulate(amax_out, mb);
    }
  } else {
    S = tensor_scale(gscales, gmode);
    if (gmode == 1 && tid == 0) gscales[0] = S;
  }
  const int64_t bpr = cols >> 4;
  with_frame(S, [&](auto tiny) {
    constexpr bool TINY = decltype(tiny)::value;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      // a block's two chunks are both in range or both out (cols % 16 == 0)
      const float a = __uint_as_float(umax(ab[i], lane_xor_u32(ab[i], 1)));
      uint32_t q, code;
      if (RM == 2) {
        const BlockScale b6 = nv_block_scale(a, S, 6.0f), b4 = nv_block_scale(a, S, 4.0f);
        const Cand8 x6 = nv_cand8<TINY>(v[i], b6, S), x4 = nv_cand8<TINY>(v[i], b4, S);
        const float e6 = x6.e + __uint_as_float(lane_xor_u32(__float_as_uint(x6.e), 1));
        const float e4 = x4.e + __uint_as_float(lane_xor_u32(__float_as_uint(x4.e), 1));
        const bool take4 = e4 < e6;
        q = take4 ? x4.q : x6.q;
        code = take4 ? b4.code : b6.code;
      } else {
        const BlockScale bs = nv_block_scale(a, S);
        u32x4 dr = {0, 0, 0, 0};
        if (SR && c < cpr) dr = philox_draws8((uint64_t)(row * cols + (int64_t)c * 8) >> 3, seed, stream_id, tensor_tag);
        q = nv_encode8<SR, TINY>(v[i], bs.r, dr);
        code = bs.code;
      }
      if (c < cpr) {
        *reinterpret_cast<uint32_t*>(codes + row * ld_codes + (int64_t)c * 4) = q;
        if ((c & 1) == 0) bscales[scale_offset(row, c >> 1, bpr, mfma_layout)] = (uint8_t)code;
      }
    }
  });
}

// Rows longer than 32768 values: two passes over the row (the second read
// mostly misses the cache).  One wave per row.
template <int RM>
__global__ __launch_bounds__(256) void nvfp4_row_long_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ bscales,
    float* __restrict__ gscales, int gmode, int mfma_layout,
    uint64_t seed, uint32_t stream_id, uint32_t tensor_tag, uint32_t* __restrict__ amax_out) {
  constexpr bool SR = RM == 1;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t cpr = cols >> 3;
  const uint16_t* xr = x + row * ld_x;
  float S;
  if (gmode == 0) {
    uint32_t mb = 0;
    for (int64_t c = lane; c < cpr; c += 64)
      mb = umax(mb, amax8_bits(*reinterpret_cast<const uint4*>(xr + c * 8)));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mb = umax(mb, lane_xor_u32(mb, o));
    S = __uint_as_float(mb) / 2688.0f;
    if (lane == 0) {
      gscales[row] = S;
      if (amax_out) amax_accumulate(amax_out, mb);
    }
  } else {
    S = tensor_scale(gscales, gmode);
    if (gmode == 1 && threadIdx.x == 0) gscales[0] = S;
  }
  const int64_t bpr = cols >> 4;
  for (int64_t c0 = 0; c0 < cpr; c0 += 64) {     // uniform trip count across the wave
    int64_t c = c0 + lane;
    uint4 v = c < cpr ? *reinterpret_cast<const uint4*>(xr + c * 8) : make_uint4(0, 0, 0, 0);
    uint32_t ab = amax8_bits(v);
    float a = __uint_as_float(umax(ab, lane_xor_u32(ab, 1)));
    uint32_t q, code;
    with_frame(S, [&](auto tiny) {
      constexpr bool TINY = decltype(tiny)::value;
      if (RM == 2) {
        // the block's two halves sit in lanes c and c ^ 1: the tree's last
        // level adds their half sums (the same in both lanes)
        const BlockScale b6 = nv_block_scale(a, S, 6.0f), b4 = nv_block_scale(a, S, 4.0f);
        const Cand8 x6 = nv_cand8<TINY>(v, b6, S), x4 = nv_cand8<TINY>(v, b4, S);
        const float e6 = x6.e + __uint_as_float(lane_xor_u32(__float_as_uint(x6.e), 1));
        const float e4 = x4.e + __uint_as_float(lane_xor_u32(__float_as_uint(x4.e), 1));
        const bool take4 = e4 < e6;
        q = take4 ? x4.q : x6.q;
        code = take4 ? b4.code : b6.code;
      } else {
        const BlockScale bs = nv_block_scale(a, S);
        u32x4 dr = {0, 0, 0, 0};
        if (SR && c < cpr) dr = philox_draws8((uint64_t)(row * cols + c * 8) >> 3, seed, stream_id, tensor_tag);
        q = nv_encode8<SR, TINY>(v, bs.r, dr);
        code = bs.code;
      }
    });
    if (c < cpr) {
      *reinterpret_cast<uint32_t*>(codes + row * ld_codes + c * 4) = q;
      if ((c & 1) == 0) bscales[scale_offset(row, c >> 1, bpr, mfma_layout)] = (uint8_t)code;
    }
  }
}

// ------------------------------------------------------------ TILE (16x16)
// A wave covers 16 chunk columns (128 columns) x 16 rows: lane = 16 rg + jj
// owns columns [8j, 8j+8) of rows 4rg..4rg+3 of the strip, and the 8 lanes
// {16 rg + 2t, 16 rg + 2t + 1 : rg = 0..3} form tile t (amax by three lane
// exchanges).  Consecutive lanes read consecutive 16-byte chunks of a row.
// dq (optional): also the dequantized copy bf16_RNE(fl(fl(value(code) s_b) S))
// [rows, cols] (ld_dq elements), the operand of the dequantized backward,
// from the codes just encoded (the dequantizer's arithmetic and order).
__device__ __forceinline__ uint4 nv_dq8(uint32_t q, float sb, float S) {
  mxq_f32x2 c[4];
  c[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  c[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  c[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  c[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x2_to_bf16x2((c[i].x * sb) * S, (c[i].y * sb) * S);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// TT: also the transposed copy, the 16x16 quantization of x^T ([cols, rows]
// codes, [cols/16, rows/16] scales): a 16x16 tile's scale serves its rows and
// its columns, so that copy is these codes transposed.  Each wave stages its
// 16 rows x 128 columns of codes in LDS and writes 128 transposed rows of 8
// bytes (16 codes); the tile scales go to the transposed scale grid.  A DGRAD
// reads it row-major instead of transposing the weight on the way into LDS.
template <int RM, bool TT>
__global__ __launch_bounds__(256) void nvfp4_tile16_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ bscales,
    float* __restrict__ gscales, int gmode, uint64_t seed, uint32_t stream_id,
    uint32_t tensor_tag, uint16_t* __restrict__ dq, int64_t ld_dq,
    uint8_t* __restrict__ codes_t, int64_t ld_codes_t, uint8_t* __restrict__ bscales_t) {
  constexpr bool SR = RM == 1;
  const int lane = threadIdx.x & 63;
  const int64_t cpr = cols >> 3;
  const int64_t j = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16 + (lane & 15);
  const int rg = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.y * 16 + rg * 4;
  const bool valid = j < cpr;
  const int64_t jc = valid ? j : cpr - 1;        // a valid address; data unused
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + i) * ld_x + jc * 8);
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) mb = umax(mb, amax8_bits(v[i]));
  mb = umax(mb, lane_xor_u32(mb, 1));
  mb = umax(mb, lane_xor_u32(mb, 16));
  mb = umax(mb, lane_xor_u32(mb, 32));
  const float S = tensor_scale(gscales, gmode);
  if (gmode == 1 && threadIdx.x == 0) gscales[0] = S;
  uint32_t q[4], code;
  if (RM == 2) {
    // Four-Over-Six per tile.  Tree order: a lane's 8 columns of a row (three
    // levels), the row's other half in lane ^ 1, the lane's 4 rows (two
    // levels), then the row groups in lane ^ 16 and lane ^ 32.  Every lane of
    // the tile ends with the same sums (each addition is commutative); lanes
    // of a tile past the last column carry unused values through the
    // exchanges and store nothing.
    const BlockScale b6 = nv_block_scale(__uint_as_float(mb), S, 6.0f);
    const BlockScale b4 = nv_block_scale(__uint_as_float(mb), S, 4.0f);
    uint32_t q6[4], q4[4];
    float r6[4], r4[4];
    with_frame(S, [&](auto tiny) {
      constexpr bool TINY = decltype(tiny)::value;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const Cand8 c6 = nv_cand8<TINY>(v[i], b6, S), c4 = nv_cand8<TINY>(v[i], b4, S);
        q6[i] = c6.q;
        q4[i] = c4.q;
        r6[i] = c6.e;
        r4[i] = c4.e;
      }
    });
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r6[i] = r6[i] + __uint_as_float(lane_xor_u32(__float_as_uint(r6[i]), 1));
      r4[i] = r4[i] + __uint_as_float(lane_xor_u32(__float_as_uint(r4[i]), 1));
    }
    float e6 = (r6[0] + r6[1]) + (r6[2] + r6[3]);
    float e4 = (r4[0] + r4[1]) + (r4[2] + r4[3]);
    e6 = e6 + __uint_as_float(lane_xor_u32(__float_as_uint(e6), 16));
    e4 = e4 + __uint_as_float(lane_xor_u32(__float_as_uint(e4), 16));
    e6 = e6 + __uint_as_float(lane_xor_u32(__float_as_uint(e6), 32));
    e4 = e4 + __uint_as_float(lane_xor_u32(__float_as_uint(e4), 32));
    const bool take4 = e4 < e6;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = take4 ? q4[i] : q6[i];
    code = take4 ? b4.code : b6.code;
  } else {
    const BlockScale bs = nv_block_scale(__uint_as_float(mb), S);
    with_frame(S, [&](auto tiny) {
      constexpr bool TINY = decltype(tiny)::value;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 dr = {0, 0, 0, 0};
        if (SR) dr = philox_draws8((uint64_t)((r0 + i) * cols + jc * 8) >> 3, seed, stream_id, tensor_tag);
        q[i] = nv_encode8<SR, TINY>(v[i], bs.r, dr);
      }
    });
    code = bs.code;
  }
  if (valid) {
    const float sbc = e4m3_to_f32(code);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint32_t*>(codes + (r0 + i) * ld_codes + j * 4) = q[i];
      if (dq) *reinterpret_cast<uint4*>(dq + (r0 + i) * ld_dq + j * 8) = nv_dq8(q[i], sbc, S);
    }
    if ((j & 1) == 0 && rg == 0) {
      bscales[(int64_t)blockIdx.y * (cols >> 4) + (j >> 1)] = (uint8_t)code;
      if (TT) bscales_t[(j >> 1) * (rows >> 4) + blockIdx.y] = (uint8_t)code;
    }
  }
  if constexpr (TT) {
    // stage: tw[wave][row r of the strip][chunk jj of the wave] = the 8 codes
    // of row r, columns 8jj .. 8jj + 7 (no lane has returned: every lane of the
    // workgroup reaches the barrier)
    __shared__ uint32_t tw[4][16][16];
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i) tw[w][rg * 4 + i][lane & 15] = q[i];
    __syncthreads();
    // lane -> columns 2l, 2l + 1 of the wave's 128: chunk l / 4, codes k, k + 1
    const int jl = lane >> 2, k = 2 * (lane & 3);
    const int64_t jg = ((int64_t)blockIdx.x * 4 + w) * 16 + jl;
    if (jg < cpr) {
      uint32_t o[4] = {0, 0, 0, 0};              // column k: o[0..1], column k + 1: o[2..3]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t word = tw[w][r][jl];
        o[r >> 3] |= ((word >> (4 * k)) & 0xFu) << (4 * (r & 7));
        o[2 + (r >> 3)] |= ((word >> (4 * k + 4)) & 0xFu) << (4 * (r & 7));
      }
      const int64_t c0 = jg * 8 + k;
      *reinterpret_cast<uint2*>(codes_t + c0 * ld_codes_t + (int64_t)blockIdx.y * 8) = make_uint2(o[0], o[1]);
      *reinterpret_cast<uint2*>(codes_t + (c0 + 1) * ld_codes_t + (int64_t)blockIdx.y * 8) = make_uint2(o[2], o[3]);
    }
  }
}

// ------------------------------------------------------------ COL (16x1)
// Each column of a 16-row strip is one block of the transposed copy ([cols,
// rows], 8 bytes per block).
//
// RHT: the 16 values of the column are first replaced by (1/4) H16 D v, the
// random Hadamard transform that the NVFP4 pretraining recipe applies to the
// WGRAD inputs ("Train models faster with JAX and MaxText using NVFP4 on
// NVIDIA Blackwell", section "NVFP4 pretraining recipe"): H16 the Sylvester
// Hadamard matrix, D = diag(-1 where bit i of sign_mask is set).  Binary32:
// sign flip (exact), butterfly strides 1, 2, 4, 8 (one rounded add or subtract
// each), times 1/4 (exact).  The block amax and the codes come from these
// binary32 values; the stochastic draws keep the element's [rows, cols] index.

// The transform of one column's 16 values (binary32 bit patterns, row order).
__device__ __forceinline__ void rht_column(const uint32_t (&bits)[16], uint32_t sign_mask,
                                           float (&u)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = __uint_as_float(bits[i] ^ (((sign_mask >> i) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = u[i], c = u[i + h];
      u[i] = a + c;
      u[i + h] = a - c;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] *= 0.25f;
}

template <bool SR, bool RHT>
__global__ __launch_bounds__(256) void nvfp4_col_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ bscales,
    float* __restrict__ gscales, int gmode, int mfma_layout, uint32_t sign_mask, uint64_t seed,
    uint32_t stream_id, uint32_t tensor_tag, int64_t n_ct) {
  const float S = tensor_scale(gscales, gmode);
  if (gmode == 1 && threadIdx.x == 0) gscales[0] = S;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t rt = blockIdx.x / n_ct, ct = blockIdx.x - rt * n_ct;
  const int64_t strips = rows >> 4;
  // a workgroup: 16 strips x 128 columns; wave w: strips 8 (w & 1) .. + 8,
  // columns 64 (w >> 1) .. + 64; lane l: strip l % 8, 8 columns from 8 (l / 8),
  // so each row's 128 bytes of a wave come from one 16-byte load of 8 lanes
  const int64_t strip = rt * 16 + (wv & 1) * 8 + (lane & 7);
  const int64_t c0 = ct * 128 + (wv >> 1) * 64 + (lane >> 3) * 8;
  if (strip >= strips || c0 >= cols) return;
  const int64_t r0 = strip * 16;
  uint4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + i) * ld_x + c0);
  u32x4 dr[16];
  if (SR) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dr[i] = philox_draws8((uint64_t)((r0 + i) * cols + c0) >> 3, seed, stream_id, tensor_tag);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // column k of row i: half (k & 1) of word (k >> 1); so is its draw
    uint32_t col[16];
    uint32_t rr16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w = (k >> 1) == 0 ? v[i].x : (k >> 1) == 1 ? v[i].y : (k >> 1) == 2 ? v[i].z : v[i].w;
      col[i] = (k & 1) ? (w & 0xFFFF0000u) : (w << 16);            // binary32 bits
      if (SR) {
        const uint32_t d = (k >> 1) == 0 ? dr[i].x : (k >> 1) == 1 ? dr[i].y : (k >> 1) == 2 ? dr[i].z : dr[i].w;
        rr16[i] = (k & 1) ? (d >> 16) : (d & 0xFFFFu);
      }
    }
    // the draws of rows 2i and 2i + 1 as one word (low and high half)
    uint32_t dw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) dw[i] = rr16[2 * i] | (rr16[2 * i + 1] << 16);
    float u[16];
    if (RHT) {
      rht_column(col, sign_mask, u);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = __uint_as_float(col[i]);
    }
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) mb = umax(mb, __float_as_uint(u[i]) & 0x7FFFFFFFu);
    const BlockScale bs = nv_block_scale(__uint_as_float(mb), S);
    // a zero block has r = 0, and a finite u times 0 is u's signed zero
    float yv[16];
    if (S < TINY_S) {
#pragma unroll
      for (int i = 0; i < 16; ++i) yv[i] = nv_frame<true>(u[i]) * bs.r;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) yv[i] = u[i] * bs.r;
    }
    uint32_t out[2] = {0, 0};
    if (SR) {
      out[0] = f32x8_to_e2m1_sr(yv, dw);
      out[1] = f32x8_to_e2m1_sr(yv + 8, dw + 4);
    } else {
      out[0] = e2m1_rne_pair<0>(out[0], yv[0], yv[1]);
      out[0] = e2m1_rne_pair<1>(out[0], yv[2], yv[3]);
      out[0] = e2m1_rne_pair<2>(out[0], yv[4], yv[5]);
      out[0] = e2m1_rne_pair<3>(out[0], yv[6], yv[7]);
      out[1] = e2m1_rne_pair<0>(out[1], yv[8], yv[9]);
      out[1] = e2m1_rne_pair<1>(out[1], yv[10], yv[11]);
      out[1] = e2m1_rne_pair<2>(out[1], yv[12], yv[13]);
      out[1] = e2m1_rne_pair<3>(out[1], yv[14], yv[15]);
    }
    const int64_t c = c0 + k;
    *reinterpret_cast<uint2*>(codes + c * ld_codes + (r0 >> 1)) = make_uint2(out[0], out[1]);
    bscales[scale_offset(c, strip, strips, mfma_layout)] = (uint8_t)bs.code;
  }
}

// Columnwise without the transform: the 16-row block of a column is split
// over two lanes (rows 0-7 and 8-15), which take the block maximum from each
// other.  With stochastic rounding a lane's 8 rows of data and their 8
// Philox calls then fit in about half the registers of the kernel above,
// which holds all 16 (two waves per SIMD there, four here).  The two lanes of a pair compute
// the same block scale; each writes its 4 code bytes, the first the scale.
// A workgroup covers 8 strips (128 rows) x 128 columns.
template <bool SR>
__global__ __launch_bounds__(256) void nvfp4_col_pair_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ bscales,
    float* __restrict__ gscales, int gmode, int mfma_layout, uint64_t seed,
    uint32_t stream_id, uint32_t tensor_tag, int64_t n_ct) {
  const float S = tensor_scale(gscales, gmode);
  if (gmode == 1 && threadIdx.x == 0) gscales[0] = S;
  const int lane = threadIdx.x & 63;
  const int hf = lane & 1;
  const int64_t rt = blockIdx.x / n_ct, ct = blockIdx.x - rt * n_ct;
  const int64_t strips = rows >> 4;
  const int64_t strip = rt * 8 + ((lane >> 1) & 7);
  const int64_t c0 = ct * 128 + (threadIdx.x >> 6) * 32 + (lane >> 4) * 8;
  // the two lanes of a pair leave together (same strip, same columns)
  if (strip >= strips || c0 >= cols) return;
  const int64_t r0 = strip * 16 + hf * 8;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + i) * ld_x + c0);
  u32x4 dr[8];
  if (SR) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dr[i] = philox_draws8((uint64_t)((r0 + i) * cols + c0) >> 3, seed, stream_id, tensor_tag);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // column k of row i: half (k & 1) of word (k >> 1); so is its draw
    float u[8];
    uint32_t rr16[8];
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = (k >> 1) == 0 ? v[i].x : (k >> 1) == 1 ? v[i].y : (k >> 1) == 2 ? v[i].z : v[i].w;
      const uint32_t b = (k & 1) ? (w & 0xFFFF0000u) : (w << 16);     // binary32 bits
      u[i] = __uint_as_float(b);
      mb = umax(mb, b & 0x7FFFFFFFu);
      if (SR) {
        const uint32_t d = (k >> 1) == 0 ? dr[i].x : (k >> 1) == 1 ? dr[i].y : (k >> 1) == 2 ? dr[i].z : dr[i].w;
        rr16[i] = (k & 1) ? (d >> 16) : (d & 0xFFFFu);
      }
    }
    mb = umax(mb, lane_xor_u32(mb, 1));
    const BlockScale bs = nv_block_scale(__uint_as_float(mb), S);
    // a zero block has r = 0, and a finite u times 0 is u's signed zero
    float yv[8];
    if (S < TINY_S) {
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[i] = nv_frame<true>(u[i]) * bs.r;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[i] = u[i] * bs.r;
    }
    uint32_t q = 0;
    if (SR) {
      uint32_t dw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dw[i] = rr16[2 * i] | (rr16[2 * i + 1] << 16);
      q = f32x8_to_e2m1_sr(yv, dw);
    } else {
      q = e2m1_rne_pair<0>(q, yv[0], yv[1]);
      q = e2m1_rne_pair<1>(q, yv[2], yv[3]);
      q = e2m1_rne_pair<2>(q, yv[4], yv[5]);
      q = e2m1_rne_pair<3>(q, yv[6], yv[7]);
    }
    const int64_t c = c0 + k;
    *reinterpret_cast<uint32_t*>(codes + c * ld_codes + (r0 >> 1)) = q;
    if (hf == 0) bscales[scale_offset(c, strip, strips, mfma_layout)] = (uint8_t)bs.code;
  }
}

// ------------------------------------------------------------ tensor amax
__global__ void nv_zero_u32(uint32_t* p) { *p = 0u; }

// IDX32: the chunk index fits 32 bits, so rows come from 32-bit divisions.
template <bool IDX32>
__global__ __launch_bounds__(256) void nv_amax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ld_x,
                                                      uint32_t* __restrict__ out_bits) {
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t m = 0;
  // four independent 16-byte loads in flight per lane
  for (int64_t base = (int64_t)blockIdx.x * 256 + threadIdx.x; base < total; base += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t id = base + u * stride;
      int64_t r, c;
      if (IDX32) {
        const uint32_t i32 = (uint32_t)id, d = (uint32_t)cpr, q32 = i32 / d;
        r = q32;
        c = i32 - q32 * d;
      } else {
        r = id / cpr;
        c = id - r * cpr;
      }
      v[u] = id < total ? *reinterpret_cast<const uint4*>(x + r * ld_x + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      m = umax(m, umax(umax(bf16x2_absmax_bits(v[u].x), bf16x2_absmax_bits(v[u].y)),
                       umax(bf16x2_absmax_bits(v[u].z), bf16x2_absmax_bits(v[u].w))));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = umax(m, lane_xor_u32(m, o));
  __shared__ uint32_t wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = umax(umax(wm[0], wm[1]), umax(wm[2], wm[3]));
    atomicMax(out_bits, (b << 16) | 0x80000000u);   // tagged binary32 bits of the magnitude
  }
}


// Max |y| over the transformed tensor y (see rht_column), as tagged binary32
// magnitude bits.  Lane layout of the COL kernel (4 columns x 16 rows); a
// workgroup walks the strips blockIdx.y, blockIdx.y + gridDim.y, ...
__global__ __launch_bounds__(256) void nv_amax_rht_kernel(const uint16_t* __restrict__ x,
                                                          int64_t rows, int64_t cols, int64_t ld_x,
                                                          uint32_t sign_mask,
                                                          uint32_t* __restrict__ out_bits) {
  const int64_t q4 = cols >> 2;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t strips = rows >> 4;
  uint32_t m = 0;
  if (j < q4) {
    for (int64_t s = blockIdx.y; s < strips; s += gridDim.y) {
      uint2 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = *reinterpret_cast<const uint2*>(x + (s * 16 + i) * ld_x + j * 4);
#pragma unroll
      for (int cidx = 0; cidx < 4; ++cidx) {
        uint32_t bits[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t w = (cidx >> 1) ? v[i].y : v[i].x;
          bits[i] = (cidx & 1) ? (w & 0xFFFF0000u) : (w << 16);
        }
        float u[16];
        rht_column(bits, sign_mask, u);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = umax(m, __float_as_uint(u[i]) & 0x7FFFFFFFu);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = umax(m, lane_xor_u32(m, o));
  __shared__ uint32_t wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = umax(umax(wm[0], wm[1]), umax(wm[2], wm[3]));
    atomicMax(out_bits, b | 0x80000000u);
  }
}

// ------------------------------------------------------------ launchers
hipError_t launch_zero_u32(uint32_t* p, hipStream_t st) {
  hipLaunchKernelGGL(nv_zero_u32, dim3(1), dim3(1), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_nvfp4_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                     float* gscale, hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(gscale);
  hipLaunchKernelGGL(nv_zero_u32, dim3(1), dim3(1), 0, st, bits);
  int64_t total = rows * (cols / 8);
  int64_t blocks = (total + 1023) / 1024;          // 4 chunks per lane
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  auto kern = total < (int64_t(1) << 32) ? nv_amax_kernel<true> : nv_amax_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, cols, ld_x, bits);
  return hipGetLastError();
}


template <int RM>
static hipError_t row_dispatch(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                               uint8_t* codes, int64_t ld_codes, uint8_t* bscales, float* gscales,
                               int gmode, bool mfma, uint64_t seed, uint32_t sid, uint32_t tag,
                               uint32_t* amax_out, hipStream_t st) {
  // at most 2048 workgroups of 4 waves (32 waves per CU, 8 per SIMD: the
  // stochastic-rounding encode is VALU work that needs them to hide its
  // dependent chains, and short rows need them to keep loads in flight); a
  // wave walks rows / 8192 rows with the next row's loads in flight
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  dim3 grid((unsigned)blocks), block(256);
  const int64_t bpr = cols / 16;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, st, x, rows, cols, ld_x, codes, ld_codes, bscales,
                       gscales, gmode, (int)mfma, seed, sid, tag, amax_out);
  };
  if (bpr == 64) go(nvfp4_row_kernel<1, RM, true>);
  else if (bpr < 64) go(nvfp4_row_kernel<1, RM, false>);
  else if (bpr == 128) go(nvfp4_row_kernel<2, RM, true>);
  else if (bpr < 128) go(nvfp4_row_kernel<2, RM, false>);
  else if (bpr == 256) go(nvfp4_row_kernel<4, RM, true>);
  else if (bpr < 256) go(nvfp4_row_kernel<4, RM, false>);
  else if (bpr == 512) go(nvfp4_row_kernel<8, RM, true>);
  else if (bpr < 512) go(nvfp4_row_kernel<8, RM, false>);
  else if (cols <= 16384 && rows <= 0x7FFFFFFF)
    // a workgroup per row, the row in registers (8 chunks per thread)
    hipLaunchKernelGGL((nvfp4_row_wg_kernel<8, RM>), dim3((unsigned)rows), block, 0, st, x, rows, cols, ld_x,
                       codes, ld_codes, bscales, gscales, gmode, (int)mfma, seed, sid, tag, amax_out);
  else if (cols <= 32768 && rows <= 0x7FFFFFFF)
    hipLaunchKernelGGL((nvfp4_row_wg_kernel<16, RM>), dim3((unsigned)rows), block, 0, st, x, rows, cols, ld_x,
                       codes, ld_codes, bscales, gscales, gmode, (int)mfma, seed, sid, tag, amax_out);
  else
    // one wave per row (no row loop in this kernel)
    hipLaunchKernelGGL(nvfp4_row_long_kernel<RM>, dim3((unsigned)((rows + 3) / 4)), block, 0, st, x,
                       rows, cols, ld_x, codes, ld_codes, bscales, gscales, gmode, (int)mfma, seed,
                       sid, tag, amax_out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* codes, int64_t ld_codes, uint8_t* bscales, float* gscales,
                            int gmode, bool mfma, int rm, uint64_t seed, uint32_t sid,
                            uint32_t tag, hipStream_t st, uint32_t* amax_out) {
  if (rm == 1)
    return row_dispatch<1>(x, rows, cols, ld_x, codes, ld_codes, bscales, gscales, gmode, mfma,
                           seed, sid, tag, amax_out, st);
  if (rm == 2)
    return row_dispatch<2>(x, rows, cols, ld_x, codes, ld_codes, bscales, gscales, gmode, mfma,
                           seed, sid, tag, amax_out, st);
  return row_dispatch<0>(x, rows, cols, ld_x, codes, ld_codes, bscales, gscales, gmode, mfma, seed,
                         sid, tag, amax_out, st);
}

hipError_t launch_nvfp4_tile16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                               uint8_t* codes, int64_t ld_codes, uint8_t* bscales,
                               float* gscales, int gmode, int rm, uint64_t seed, uint32_t sid,
                               uint32_t tag, uint16_t* dq, int64_t ld_dq, uint8_t* codes_t,
                               int64_t ld_codes_t, uint8_t* bscales_t, hipStream_t st) {
  // four waves per workgroup, each 128 columns of a 16-row strip
  dim3 grid((unsigned)((cols / 8 + 63) / 64), (unsigned)(rows / 16));
  if (grid.y > 65535u) return hipErrorInvalidValue;      // more row strips than a grid holds
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, x, rows, cols, ld_x, codes, ld_codes, bscales,
                       gscales, gmode, seed, sid, tag, dq, ld_dq, codes_t, ld_codes_t, bscales_t);
  };
  if (codes_t) {
    if (rm == 1) go(nvfp4_tile16_kernel<1, true>);
    else if (rm == 2) go(nvfp4_tile16_kernel<2, true>);
    else go(nvfp4_tile16_kernel<0, true>);
  } else {
    if (rm == 1) go(nvfp4_tile16_kernel<1, false>);
    else if (rm == 2) go(nvfp4_tile16_kernel<2, false>);
    else go(nvfp4_tile16_kernel<0, false>);
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* codes, int64_t ld_codes, uint8_t* bscales,
                            float* gscales, int gmode, bool mfma, bool sr, bool rht,
                            uint32_t sign_mask, uint64_t seed, uint32_t sid, uint32_t tag,
                            hipStream_t st) {
  // workgroup tile 256 rows x 128 columns
  const int64_t n_rt = (rows / 16 + 15) / 16, n_ct = (cols + 127) / 128;
  const int64_t nwg = n_rt * n_ct;
  if (nwg > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(256), 0, st, x, rows, cols, ld_x, codes,
                       ld_codes, bscales, gscales, gmode, (int)mfma, sign_mask, seed, sid, tag, n_ct);
  };
  if (rht) {
    if (sr) go(nvfp4_col_kernel<true, true>);
    else go(nvfp4_col_kernel<false, true>);
  } else if (sr) {
    // workgroup tile 128 rows x 128 columns (the pair split measured slower
    // for round-to-nearest-even: 135.8 against 127.8 us at 32768x4096)
    const int64_t n_rt2 = (rows / 16 + 7) / 8;
    if (n_rt2 * n_ct > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(nvfp4_col_pair_kernel<true>, dim3((unsigned)(n_rt2 * n_ct)), dim3(256), 0, st, x, rows,
                       cols, ld_x, codes, ld_codes, bscales, gscales, gmode, (int)mfma, seed, sid, tag, n_ct);
  } else {
    go(nvfp4_col_kernel<false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_nvfp4_tensor_scale_rht(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ld_x, uint32_t sign_mask, float* gscale,
                                         hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(gscale);
  hipLaunchKernelGGL(nv_zero_u32, dim3(1), dim3(1), 0, st, bits);
  // about 2048 workgroups, each walking a share of the 16-row strips
  const int64_t gx = (cols / 4 + 255) / 256;
  int64_t gy = 2048 / gx;
  if (gy < 1) gy = 1;
  if (gy > rows / 16) gy = rows / 16;
  if (gy > 65535) gy = 65535;
  hipLaunchKernelGGL(nv_amax_rht_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st, x,
                     rows, cols, ld_x, sign_mask, bits);
  return hipGetLastError();
}

}  // namespace mxq
