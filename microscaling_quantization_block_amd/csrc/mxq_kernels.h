// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mxq {

// Raises kernel fn's dynamic-LDS limit to `bytes` on the current device, once
// per device (bit d of `done` records device d; devices from 32 on set it on
// every call).  Safe to call from several host threads.
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<uint32_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = dev < 32 ? (1u << dev) : 0u;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// b128: 1 = DeepSeek-style blockwise FP8 (128-value blocks, power-of-two
// scales, linear scale layouts), 2 = the same with binary32 scales (scales
// then points to floats); mfma ignored for both.
hipError_t launch_mxfp8_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* codes, int64_t ld_codes, uint8_t* scales, bool mfma, int b128,
                            hipStream_t st);
// mode: 0 COL, 1 TILE (codes_col optional transposed copy), 2 DUAL
hipError_t launch_mxfp8_tile(int mode, const uint16_t* x, int64_t rows, int64_t cols,
                             int64_t ld_x, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                             uint8_t* codes_col, int64_t ld_codes_col, uint8_t* scales_col,
                             bool mfma, int b128, hipStream_t st);

// per-tensor amax: zeroes gscale[0], then leaves the tensor amax there tagged
// with bit 31 (the quantize kernel decodes it and writes S back)
hipError_t launch_nvfp4_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                     float* gscale, hipStream_t st);
// gmode: 0 = per row (computed), 1 = per tensor (tagged amax in gscales[0]),
// 2 = given (S in gscales[0]).  rm: 0 = RNE, 1 = stochastic rounding, 2 = RNE
// with the Four-Over-Six block-scale choice.
// amax_out (per-row mode only): also accumulate the tensor amax there as
// tagged binary32 bits (the protocol of launch_nvfp4_tensor_scale; zero it first)
hipError_t launch_nvfp4_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* codes, int64_t ld_codes, uint8_t* bscales, float* gscales,
                            int gmode, bool mfma, int rm, uint64_t seed, uint32_t sid,
                            uint32_t tag, hipStream_t st, uint32_t* amax_out = nullptr);
hipError_t launch_zero_u32(uint32_t* p, hipStream_t st);
// dq (optional, else nullptr): the dequantized BF16 copy written in the same pass;
// codes_t (optional, with bscales_t): the transposed copy [cols, rows/2] bytes,
// scales [cols/16, rows/16]
hipError_t launch_nvfp4_tile16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                               uint8_t* codes, int64_t ld_codes, uint8_t* bscales,
                               float* gscales, int gmode, int rm, uint64_t seed, uint32_t sid,
                               uint32_t tag, uint16_t* dq, int64_t ld_dq, uint8_t* codes_t,
                               int64_t ld_codes_t, uint8_t* bscales_t, hipStream_t st);
// rht: the random Hadamard transform of each 16-row block before quantizing
// (sign_mask bit i negates row i of the block)
hipError_t launch_nvfp4_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                            uint8_t* codes, int64_t ld_codes, uint8_t* bscales,
                            float* gscales, int gmode, bool mfma, bool sr, bool rht,
                            uint32_t sign_mask, uint64_t seed, uint32_t sid, uint32_t tag,
                            hipStream_t st);
// per-tensor amax of the transformed tensor (same protocol as above)
hipError_t launch_nvfp4_tensor_scale_rht(const uint16_t* x, int64_t rows, int64_t cols,
                                         int64_t ld_x, uint32_t sign_mask, float* gscale,
                                         hipStream_t st);

hipError_t launch_dq_mxfp8(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                           int64_t rows, int64_t cols, bool tile, bool mfma, int b128,
                           uint16_t* out, int64_t ld_out, hipStream_t st);
hipError_t launch_dq_nvfp4(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                           const float* gscales, int64_t rows, int64_t cols, bool tile,
                           int gmode, bool mfma, uint16_t* out, int64_t ld_out, hipStream_t st);
hipError_t launch_swiglu(const uint16_t* gu, int64_t rows, int64_t inter, int64_t ld_gu,
                         uint16_t* h, int64_t ld_h, hipStream_t st);

// Blockwise FP8 GEMM with binary32 block scales: C = A B^T, A [M, K] and
// B [N, K] E4M3 codes (row-major, lda / ldb bytes), scales [rows, K/128]
// (ROW) or [rows/128, K/128] (TILE), C BF16 [M, N] (ldc elements).
struct Fp8sArgs {
  const uint8_t* a;
  const float* a_scales;
  int64_t lda;
  int a_tile;
  const uint8_t* b;
  const float* b_scales;
  int64_t ldb;
  int b_tile;
  uint16_t* c;
  int64_t ldc;
  int64_t M, N, K;
};
hipError_t launch_gemm_fp8s(const Fp8sArgs& a, hipStream_t st);

enum Path { P_FP8 = 0, P_F16 = 1, P_BF16 = 2 };

struct GemmArgs {
  const uint8_t* a;            // A data (codes / values)
  const uint8_t* a_scales;
  const float* a_gs;
  int64_t lda;                 // elements
  int a_mfma_layout;
  int a_gs_per_row;
  const uint8_t* b;
  const uint8_t* b_scales;
  const float* b_gs;
  int64_t ldb;                 // elements
  int b_mfma_layout;
  int b_tile;                  // 2D blocks (32x32 / 16x16 / 128x128)
  int a_b128, b_b128;          // FP8 path: 128-wide power-of-two scale blocks (linear)
  int64_t swiglu_inter;        // > 0: NVFP4 gate_up with SwiGLU fused, c = H [M, inter], N = 2 inter
  int64_t b_group_elems;       // elements between groups' matrices (N * ldb)
  int64_t b_group_scales;      // scale bytes between groups
  int64_t M, N, K;
  int64_t a_rows;              // rows stored in A (the gather index points into them)
  uint16_t* c;
  int64_t ldc;
  int num_groups;
  const int32_t* offsets;
  const int32_t* row_index;
};

hipError_t launch_gemm(int path, bool b_transposed, const GemmArgs& a, hipStream_t st);
// NVFP4 gate_up GEMM with SwiGLU and the per-token NVFP4 quantization of H in
// its epilogue (a.swiglu_inter in {256, 512, 768}; a.c = H or null).
hipError_t launch_gemm_swiglu_q(const GemmArgs& a, uint8_t* codes, int64_t ld_codes, uint8_t* scales, float* gs,
                                bool mfma, hipStream_t st);
void gemm_set_tile(int tile);   // -1 = measured choice, 0..6 = forced configuration

}  // namespace mxq
