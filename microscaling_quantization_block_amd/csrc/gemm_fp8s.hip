// Blockwise FP8 GEMM with binary32 block scales (the DeepSeek-V3 recipe that
// "NVIDIA NeMo RL agora roda treino ... FP8 ponta a ponta" (section "FP8 nas
// camadas lineares") describes: E4M3 with one scale per 1x128 block of
// activations and gradients and per 128x128 block of weights; "End-to-End
// MXFP8 Reinforcement Learning on Blackwell", Table 1, names its FP32-scale
// arm).
//
// C[m, n] = sum over 128-wide K blocks kb of s_a(m, kb) * s_b(n, kb) * P_kb(m, n),
// P_kb = sum_{k in kb} value(a[m, k]) * value(b[n, k]).  The scaled MFMA takes
// only power-of-two (E8M0) scales, so each stage (one K block) runs its two
// v_mfma_scale_f32_32x32x64_f8f6f4 steps with unit scales into fresh binary32
// accumulators, and the partial sums are then folded in as
// acc = fma(s_a * s_b, P_kb, acc).
//
// Workgroup: 256 threads, a 128x128 output tile, 4 waves as 2x2, each wave a
// 64x64 block of 32x32 MFMA tiles.  A stage (128 K bytes of 128 A rows and
// 128 B rows, and the stage's 128 + 128 scales) goes global -> registers ->
// LDS, two LDS buffers, one barrier per stage; the next stage's global loads
// are in flight during the MFMAs.  LDS rows are 128 bytes of 16-byte chunks;
// chunk ch of row r sits at slot ch ^ ((r >> 1) & 7), so the 16 rows a
// fragment read touches per cycle cover all 64 banks, and the 8 chunks of a
// row written per cycle cover 32.  Scale vectors sit beside each buffer.
// Epilogue: each wave stages its 64x64 BF16 block in LDS and reads it back so
// that 8 lanes store one contiguous 128-byte run of a C row.

#include "mxq_device.h"
#include "mxq_kernels.h"

namespace mxq {

namespace {

constexpr int FS_BM = 128, FS_BN = 128, FS_BK = 128;
constexpr int FS_ROWB = 128;                                  // LDS bytes per operand row
constexpr int FS_OPB = FS_BM * FS_ROWB;                       // one operand tile, bytes
constexpr int FS_BUF = 2 * FS_OPB + (FS_BM + FS_BN) * 4;      // A, B, scales
constexpr int FS_EROW = 64 * 2 + 8;                           // epilogue row bytes (padded)
static_assert(4 * 64 * FS_EROW <= 2 * FS_BUF, "epilogue staging fits the stage buffers");

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int fs_slot(int r, int ch) { return r * 8 + (ch ^ ((r >> 1) & 7)); }

}  // namespace

// BU: B has 128x128 tile scales, so its scale is one value per stage for the
// whole workgroup (tiles start at multiples of 128)
template <bool BU>
__global__ __launch_bounds__(256, 2) void gemm_fp8s_kernel(Fp8sArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;

  // XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD takes a
  // contiguous range of the tile order below
  const int tiles_n = (int)((p.N + FS_BN - 1) / FS_BN);
  const int G = (int)gridDim.x;
  const int b = blockIdx.x;
  const int q8 = G >> 3, r8 = G & 7, x = b & 7;
  if ((b >> 3) >= q8 + (x < r8 ? 1 : 0)) return;             // (the grid holds exactly the tiles)
  const int logical = x * q8 + (x < r8 ? x : r8) + (b >> 3);
  // grouped order: runs of 8 tile rows walked column by column, so the
  // tiles in flight on an XCD form a block that shares A and B panels in its
  // L2 (row by row, they would share one A panel and stream all of B)
  const int tiles_m = G / tiles_n;
  const int grp = logical / (8 * tiles_n), in = logical - grp * 8 * tiles_n;
  const int gm = min(8, tiles_m - grp * 8);
  const int64_t m0 = (int64_t)(grp * 8 + in % gm) * FS_BM;
  const int64_t n0 = (int64_t)(in / gm) * FS_BN;
  const int nk = (int)(p.K / FS_BK);
  const int64_t kb_stride = p.K / FS_BK;                      // scales per row

  // ---- loader: 4 chunks of A and 4 of B per thread, one scale per thread
  uint4 ra[4], rb[4];
  float rs = 0.0f;
  auto load = [&](int kt) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + 256 * k, row = i >> 3, ch = i & 7;
      const int64_t m = m0 + row, n = n0 + row;
      ra[k] = m < p.M ? *reinterpret_cast<const uint4*>(p.a + m * p.lda + (int64_t)kt * FS_BK + ch * 16)
                      : make_uint4(0, 0, 0, 0);
      rb[k] = n < p.N ? *reinterpret_cast<const uint4*>(p.b + n * p.ldb + (int64_t)kt * FS_BK + ch * 16)
                      : make_uint4(0, 0, 0, 0);
    }
    if (tid < FS_BM) {
      const int64_t m = m0 + tid;
      rs = m < p.M ? p.a_scales[(p.a_tile ? (m >> 7) : m) * kb_stride + kt] : 0.0f;
    } else {
      const int64_t n = n0 + (tid - FS_BM);
      rs = n < p.N ? p.b_scales[(p.b_tile ? (n >> 7) : n) * kb_stride + kt] : 0.0f;
    }
  };
  auto store = [&](int buf) {
    uint8_t* base = lds + buf * FS_BUF;
    uint4* LA = reinterpret_cast<uint4*>(base);
    uint4* LB = reinterpret_cast<uint4*>(base + FS_OPB);
    float* LS = reinterpret_cast<float*>(base + 2 * FS_OPB);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = tid + 256 * k, row = i >> 3, ch = i & 7;
      LA[fs_slot(row, ch)] = ra[k];
      LB[fs_slot(row, ch)] = rb[k];
    }
    LS[tid] = rs;                                             // A scales 0..127, B scales 128..255
  };

  v16f_t acc[2][2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[tm][tn][j] = 0.0f;

  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    const uint8_t* base = lds + buf * FS_BUF;
    const uint4* LA = reinterpret_cast<const uint4*>(base);
    const uint4* LB = reinterpret_cast<const uint4*>(base + FS_OPB);
    const float* LS = reinterpret_cast<const float*>(base + 2 * FS_OPB);
    // fragments of both 64-wide K steps: lane (row r32, half h) holds K bytes
    // [16h, 16h + 16) and [32 + 16h, 32 + 16h + 16) of each step in both
    // operands (chunks 4ks + h and 4ks + 2 + h)
    v8i_t af[2][2], bf[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra_ = wm * 64 + t * 32 + r32, rb_ = wn * 64 + t * 32 + r32;
        const uint4 a0 = LA[fs_slot(ra_, 4 * ks + h)], a1 = LA[fs_slot(ra_, 4 * ks + 2 + h)];
        const uint4 b0 = LB[fs_slot(rb_, 4 * ks + h)], b1 = LB[fs_slot(rb_, 4 * ks + 2 + h)];
        af[ks][t] = v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        bf[ks][t] = v8i_t{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
    // per output tile: the block's partial sums (two MFMA steps from zero,
    // unit E8M0 scales; B first, so lane l holds output row m = l % 32 and
    // columns 8g + 4(l / 32) + i in element 4g + i), then the fold with
    // s_a(m) * s_b(n)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const float sa = LS[wm * 64 + tm * 32 + r32];
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        v16f_t part;
#pragma unroll
        for (int j = 0; j < 16; ++j) part[j] = 0.0f;
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[0][tn], af[0][tm], part, 0, 0, 0, 127, 0, 127);
        part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[1][tn], af[1][tm], part, 0, 0, 0, 127, 0, 127);
        if constexpr (BU) {
          const float f = sa * LS[FS_BM];
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[tm][tn][j] = __builtin_fmaf(f, part[j], acc[tm][tn][j]);
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 sb = *reinterpret_cast<const float4*>(LS + FS_BM + wn * 64 + tn * 32 + 8 * g + 4 * h);
            const float sbv[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[tm][tn][4 * g + i] = __builtin_fmaf(sa * sbv[i], part[4 * g + i], acc[tm][tn][4 * g + i]);
          }
        }
      }
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue (the last barrier above ends every LDS read of the loop)
  uint8_t* const E = lds + wave * (64 * FS_EROW);
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v16f_t& v = acc[tm][tn];
        *reinterpret_cast<uint2*>(E + (tm * 32 + r32) * FS_EROW + (tn * 32 + 8 * g + 4 * h) * 2) =
            make_uint2(f32x2_to_bf16x2(v[4 * g], v[4 * g + 1]), f32x2_to_bf16x2(v[4 * g + 2], v[4 * g + 3]));
      }
  // (a wave's LDS operations complete in order: its reads below see its writes)
  const bool vec16 = ((p.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int rr = it * 8 + (lane >> 3), cc = lane & 7;       // 8 lanes per 128-byte row run
    const uint4 val = *reinterpret_cast<const uint4*>(E + rr * FS_EROW + cc * 16);
    const int64_t m = m0 + wm * 64 + rr;
    const int64_t n = n0 + wn * 64 + cc * 8;
    if (m < p.M && n < p.N) {
      uint16_t* dst = p.c + m * p.ldc + n;
      if (vec16 && n + 7 < p.N) {
        *reinterpret_cast<uint4*>(dst) = val;
      } else {
        const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (n + i < p.N) dst[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
      }
    }
  }
}

hipError_t launch_gemm_fp8s(const Fp8sArgs& a, hipStream_t st) {
  const int64_t tiles = ((a.M + FS_BM - 1) / FS_BM) * ((a.N + FS_BN - 1) / FS_BN);
  if (tiles < 1 || tiles >= (1ll << 31)) return hipErrorInvalidValue;
  const size_t lds = 2 * (size_t)FS_BUF;
  auto go = [&](auto kern, std::atomic<uint32_t>& lds_set) -> hipError_t {
    if (hipError_t e = ensure_lds_limit((const void*)kern, (int)lds, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(256), lds, st, a);
    return hipGetLastError();
  };
  static std::atomic<uint32_t> set_u{0}, set_r{0};
  return a.b_tile ? go(gemm_fp8s_kernel<true>, set_u) : go(gemm_fp8s_kernel<false>, set_r);
}

}  // namespace mxq
