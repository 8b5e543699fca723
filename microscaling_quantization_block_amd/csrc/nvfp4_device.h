// NVFP4 element chain shared by the quantizers and by the GEMM epilogue that
// requantizes its output (the same code, so the same bits): the block scale
// and reciprocal from a block's amax and the second scale S, the frame for
// tiny S, and the 8-value encoders (RNE, stochastic rounding).
#pragma once

#include "mxq_device.h"

#include <type_traits>

namespace mxq {

// Block scale and per-block reciprocal from the block amax (binary32 bits of
// a BF16 magnitude widened) and S.  r is the reciprocal in the frame of S:
// scaled by 2^-64 when S < 2^-64 (TINY_S), where the encoders scale x by 2^64.
struct BlockScale { uint32_t code; float r; };

constexpr float TINY_S = 0x1p-64f;
constexpr float FRAME = 0x1p64f;

// m = 6 maps the block max onto the largest E2M1 value (plain NVFP4); m = 4
// is Four-Over-Six's second candidate.
__device__ __forceinline__ BlockScale nv_block_scale(float a_b, float S, float m = 6.0f) {
  BlockScale bs;
  if (!(S > 0.0f)) { bs.code = 0; bs.r = 0.0f; return bs; }
  float m_s = m * S;
  float t = a_b / m_s;
  // saturating encode: with a caller-given S, t may exceed the E4M3 range
  // (every value >= 448 rounds to 448; the hardware conversion would not
  // saturate on its own)
  t = t < 448.0f ? t : 448.0f;
  bs.code = f32x2_to_e4m3(t, 0.0f) & 0xFFu;
  float sb = e4m3_to_f32(bs.code);
  const float Sf = S < TINY_S ? S * FRAME : S;   // exact
  float den = sb * Sf;
  bs.r = bs.code ? 1.0f / den : 0.0f;
  return bs;
}

// x in the frame of S (TINY: S < 2^-64, x times 2^64, exact).
template <bool TINY>
__device__ __forceinline__ float nv_frame(float x) { return TINY ? x * FRAME : x; }

// Encode the 8 BF16 values of one chunk with reciprocal r; returns 8 nibbles
// (element 2j in the low nibble of byte j).  zero_block forces signed zeros.
// RNE encode of a pair of binary32 values onto E2M1 by the hardware
// conversion with unit scale (its scale only divides by a power of two, so 1.0
// leaves y unchanged).  It rounds to nearest even, saturates at 6 and keeps
// the sign of zero, identically to the integer encoder f32_to_e2m1_rne; the
// two were compared on every BF16 value below 8 and a million random binary32
// values, and the exhaustive quantizer tests check it against the oracle.
// The result's byte `sel` holds the pair (first value in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_rne_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// A block whose scale code is 0 has r = 0, and x * 0 is the signed zero of
// the (finite) input, so zero blocks need no separate path.
template <bool SR, bool TINY = false>
__device__ __forceinline__ uint32_t nv_encode8(uint4 v, float r, u32x4 draws) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t d[4] = {draws.x, draws.y, draws.z, draws.w};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = nv_frame<TINY>(bf16_lo(w[i])) * r;
    y[2 * i + 1] = nv_frame<TINY>(bf16_hi(w[i])) * r;
  }
  if (SR) {
    return f32x8_to_e2m1_sr(y, d);
  }
  uint32_t out = 0;
  out = e2m1_rne_pair<0>(out, y[0], y[1]);
  out = e2m1_rne_pair<1>(out, y[2], y[3]);
  out = e2m1_rne_pair<2>(out, y[4], y[5]);
  out = e2m1_rne_pair<3>(out, y[6], y[7]);
  return out;
}

// Calls f(std::true_type) when S is below 2^-64 (the scaled frame), else
// f(std::false_type).  S is wave-uniform at every call site.
template <class F>
__device__ __forceinline__ void with_frame(float S, F&& f) {
  if (S < TINY_S) f(std::true_type{});
  else f(std::false_type{});
}

// Max |x| of 8 BF16 values as the binary32 bit pattern of the magnitude
// (integer max on magnitude bits: exact, and immune to denormal flushing).
__device__ __forceinline__ uint32_t amax8_bits(uint4 v) {
  uint32_t m = umax(umax(bf16x2_absmax_bits(v.x), bf16x2_absmax_bits(v.y)),
                    umax(bf16x2_absmax_bits(v.z), bf16x2_absmax_bits(v.w)));
  return m << 16;
}

}  // namespace mxq
