// Device helpers shared by the quantizer, dequantizer and GEMM kernels
// (gfx950 / CDNA4, wave64).  Everything here is bit-level format handling;
// no routine depends on fast-math, and the library is compiled with
// -ffp-contract=off so that a*b+c is never fused where the format contract
// names two roundings.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round a binary32 value to BF16, nearest-even (finite or infinite inputs;
// a finite value that rounds past the largest BF16 becomes infinity).
// Two binary32 values to packed BF16 (a in the low half), round to nearest
// even, by the hardware conversion: on MI355X it matches the integer rounding
// (u + 0x7FFF + lsb) >> 16 on every tie and neighbour pattern of every BF16
// value (subnormals, overflow to infinity included) and on 2^30 strided
// patterns; NaN stays NaN.
typedef __bf16 mxq_bf16x2 __attribute__((ext_vector_type(2)));
typedef float mxq_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const mxq_f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, mxq_bf16x2));
}

// |x| of both BF16 halves, then the larger as a 16-bit magnitude pattern.
// For finite values the order of magnitude patterns is the order of |x|.
__device__ __forceinline__ uint32_t bf16x2_absmax_bits(uint32_t w) {
  uint32_t a = w & 0x7FFFu;
  uint32_t b = (w >> 16) & 0x7FFFu;
  return a > b ? a : b;
}

// ------------------------------------------------------------------ E4M3
// Exact value of an E4M3 byte (OCP FN variant, no infinities) via the
// hardware conversion (exact: every E4M3 value is a binary32 value).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Round-to-nearest-even of two binary32 values to E4M3, packed into the low
// 16 bits (first value in the low byte).  Inputs must be below 464 in
// magnitude (they are: every caller bounds them by 448 * (1 + 2^-22)).
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// ------------------------------------------------------------------ E2M1
// E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7.

// Round-to-nearest-even onto the E2M1 grid, saturating at 6.  Returns the
// 4-bit code (sign in bit 3 taken from the sign bit of y).
//   |y| in [1, 5]: round the binary32 mantissa to one bit (RNE on the bit
//                  pattern); the result (exponent, bit) maps to the code.
//   |y| < 1:       the code is rint(2|y|) (0 -> 0, 1 -> 0.5, 2 -> 1.0).
//   |y| > 5:       6 (code 7).
__device__ __forceinline__ uint32_t f32_to_e2m1_rne(float y) {
  uint32_t b = __float_as_uint(y);
  uint32_t s = (b >> 28) & 8u;
  uint32_t a = b & 0x7FFFFFFFu;
  uint32_t rnd = a + 0x1FFFFFu + ((a >> 22) & 1u);
  uint32_t big = (rnd >> 22) - 252u;                       // 2..6 for |y| in [1, 5]
  uint32_t small = (uint32_t)__builtin_rintf(2.0f * __uint_as_float(a));
  uint32_t mag = a >= 0x3F800000u ? big : small;
  mag = a > 0x40A00000u ? 7u : mag;
  return s | mag;
}

// Stochastic rounding of eight binary32 values onto the E2M1 grid: with
// lo <= |y| < hi the grid neighbours, round up iff r < (|y| - lo) / (hi - lo)
// * 2^16 for the value's 16-bit draw r; |y| >= 6 gives 6; the sign is kept.
// Returns 8 nibbles, value 2j in the low nibble of byte j.
//
// The work is done by the hardware conversion v_cvt_scalef32_sr_pk_fp4_f32,
// whose behaviour on MI355X was measured (every BF16 value below 8, a million
// random binary32 values, subnormals, huge values, infinities, each with the
// draws 0, 65535, the three around its rounding boundary and a random one):
//   * the pair's first value is rounded up iff F + (seed >> (32 - w)) >= 2^w,
//     where F = floor(frac * 2^w) and w = 23 below 1, 22 from 1 up;
//   * the second value uses seed << 1 in place of seed, so one instruction
//     cannot give the two values independent draws;
//   * below 1 the fraction keeps only 22 bits: F loses the lowest bit of a
//     value in [0.5, 1), and more below 0.5;
//   * magnitudes from 6 up (infinity included) give 6;
//   * the scale operand divides the input by its power of two before rounding.
// Hence:
//   * |y| is first rounded up to a multiple of 2^-17. For an integer r,
//     r < frac * 2^16 is unchanged by that, because 2^-17 divides the
//     neighbours and (hi - lo) / 2^-17 >= 2^16, so frac * 2^16 only moves up
//     to the next integer or a finer grid point. After it, every fraction is
//     a multiple of 2^-18, which F holds exactly at either width.
//   * The rounding is a ceil of |y| * 2^17; the conversion's scale 2^17
//     undoes that power of two exactly.
//   * A first-value seed with ~r in bits 31..16 and ones in bits 15..9 makes
//     seed >> (32 - w) equal 2^w - 1 - r * 2^(w-16), so the test reads
//     F > r * 2^(w-16), that is r < frac * 2^16. A second-value seed has ~r
//     in bits 30..15 and ones in bits 14..8.
// Each pair (a, b) is converted as (b, a), twice: once with b's draw in the
// first-value seed (the low nibble of that result is b's code), once with a's
// draw in the second-value seed (its high nibble is a's code).  Then b's
// draw, the high half of the draw word d = r_a | r_b << 16, gives the seed
// ~d | 0xFFFF, and a's gives ~(d << 15).  The two result words are merged
// nibble by nibble.  The instructions sit in one asm block, because the
// compiler does not pass the destination's previous bytes to them (the
// hardware keeps them). The block orders them so that a result written to
// bytes 2 or 3 is not read by the very next instruction.
__device__ __forceinline__ float e2m1_sr_prescale(float y) {
  return __builtin_copysignf(__builtin_ceilf(__builtin_fabsf(y) * 0x1p17f), y);
}

// y[0..7]; d[i] holds the draws of y[2i] (low half) and y[2i + 1] (high half).
__device__ __forceinline__ uint32_t f32x8_to_e2m1_sr(const float* y, const uint32_t* d) {
  mxq_f32x2 p[4];
  uint32_t s_hi[4], s_lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = mxq_f32x2{e2m1_sr_prescale(y[2 * i + 1]), e2m1_sr_prescale(y[2 * i])};
    s_hi[i] = ~d[i] | 0xFFFFu;
    s_lo[i] = ~(d[i] << 15);
  }
  uint32_t a, b;
  asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %2, %6, %14 op_sel:[0,0,1,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %2, %10, %14 op_sel:[0,0,1,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %3, %7, %14 op_sel:[0,0,0,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %3, %11, %14 op_sel:[0,0,0,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %4, %8, %14 op_sel:[0,0,1,0]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %4, %12, %14 op_sel:[0,0,1,0]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %5, %9, %14\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %5, %13, %14"
      : "=&v"(a), "=&v"(b)
      : "v"(p[3]), "v"(p[2]), "v"(p[1]), "v"(p[0]),
        "v"(s_hi[3]), "v"(s_hi[2]), "v"(s_hi[1]), "v"(s_hi[0]),
        "v"(s_lo[3]), "v"(s_lo[2]), "v"(s_lo[1]), "v"(s_lo[0]), "s"(0x1p17f));
  // odd values: low nibbles of a; even values: high nibbles of b
  return ((a << 4) & 0xF0F0F0F0u) | ((b >> 4) & 0x0F0F0F0Fu);
}

// ------------------------------------------------------------------ Philox
// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64
// multiplies with the published multipliers and Weyl key increments.
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    // one 32x32->64 product gives both halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    // three-input XOR in one instruction (truth table 0x96)
    c = u32x4{(uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
              (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0};
  }
  return c;
}

// The 8 16-bit draws of elements [8n, 8n+8) of the logical input.
__device__ __forceinline__ u32x4 philox_draws8(uint64_t n, uint64_t seed, uint32_t stream_id,
                                               uint32_t tensor_tag) {
  return philox4x32_10(u32x4{(uint32_t)n, (uint32_t)(n >> 32), stream_id, tensor_tag},
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

// ------------------------------------------------------------------ lanes
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, 64);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max over the 64 lanes of a wave (every lane active), wave-uniform result:
// DPP quad permutes [1,0,3,2] and [2,3,0,1], then half-row and row mirrors
// give each 16-lane row its max; four lane reads combine the rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return umax(umax(a, b), umax(c, d));
}

// SwiGLU of two BF16 pairs (gate g, up u; element 0 in the low half):
// bf16_RNE(g / (1 + exp(-g)) * u) in binary32, with the hardware exp2 and
// reciprocal (a few binary32 ulps; the result is rounded to BF16).  The
// standalone kernel and the GEMM epilogue that fuses it share this code, so
// their bits agree.  exp(-g) = inf for very negative g gives -0.
__device__ __forceinline__ uint32_t swiglu_bf16x2(uint32_t g, uint32_t u) {
  const float g0 = bf16_lo(g), g1 = bf16_hi(g);
  const float u0 = bf16_lo(u), u1 = bf16_hi(u);
  const float h0 = __fdividef(g0, 1.0f + __expf(-g0)) * u0;
  const float h1 = __fdividef(g1, 1.0f + __expf(-g1)) * u1;
  return f32x2_to_bf16x2(h0, h1);
}

// MFMA scale layout (1D blocks): chunks of 32 rows x 4 blocks, 128 bytes.
__device__ __forceinline__ int64_t scale_offset(int64_t r, int64_t b, int64_t blocks_per_row,
                                                bool mfma) {
  if (!mfma) return r * blocks_per_row + b;
  return ((r >> 5) * (blocks_per_row >> 2) + (b >> 2)) * 128 + (r & 31) * 4 + (b & 3);
}

}  // namespace mxq
