// Block-scaled GEMMs for gfx950: C[M, N] = sum_k A[m, k] * B[n, k], FP32
// accumulation, BF16 output.
//
// The three GEMMs of a linear layer (FPROP, DGRAD, WGRAD) take quantized
// operands and emit BF16 ("Train models faster with JAX and MaxText using
// NVFP4 on NVIDIA Blackwell", section "NVFP4 pretraining recipe"; MXFP8 on
// every GEMM: "Miles Blackwell RL ...", section "O Suporte Miles Blackwell
// Agora Abrange Todo o Loop de RL").  The dequantized backward uses BF16 GEMMs
// on DQ(Q(w)) ("NVFP4 RL training", dequantized-backward section).
//
// Three compute paths share one LDS-staged, double-buffered tile loop:
//  * MXFP8: E4M3 bytes staged as they are; v_mfma_scale_f32_32x32x64_f8f6f4
//    applies the E8M0 block scales itself (lane r + 32j supplies the scale of
//    row r, 32-wide K block j), so scaling costs nothing in the inner loop.  A
//    scaled MMA takes exponent-only scales, which is exactly what MXFP8 has
//    ("End-to-End MXFP8 RL on Blackwell", Table 10 F6).
//  * NVFP4: the E4M3 block scale has a mantissa, which no scaled MFMA of this
//    chip accepts, and an E2M1 x E4M3 product needs 6 significant bits, more
//    than any 8-bit format holds.  Each value c * s_b is exact in FP16, so the
//    loader dequantizes codes to FP16 on the way into LDS and the inner loop
//    runs v_mfma_f32_32x32x16_f16; FP4 x FP8 products being exact in FP16 is
//    the same observation the Four-Over-Six work relies on ("NVFP4 RL
//    training", Four-Over-Six section).  The FP32 second scales multiply the
//    accumulator in the epilogue.
//  * BF16: v_mfma_f32_32x32x16_bf16 (the dequantized-backward DGRAD).
//
// Workgroup: 256 lanes as 2 x 2 waves; BM x BN output tile, each wave a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles.  Every LDS row holds 128 bytes
// of K (128 FP8 or 64 FP16/BF16 values) plus 16 bytes of padding, which makes
// the 16-byte fragment reads of 8 consecutive rows hit 32 distinct banks.
// B may be stored transposed ([K, N], the FPROP weight copy read by DGRAD);
// the loader then transposes 4x8 / 8x8 sub-blocks in registers on the way
// into LDS.  Grouped (MoE) launches map each workgroup to (group, m-tile)
// with a scan of the device-side group offsets.

#include "mxq_device.h"
#include "mxq_kernels.h"

namespace mxq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int LDS_ROW = 144;     // bytes per LDS row: 128 data + 16 pad

// ------------------------------------------------------------ FP4 -> FP16
// Two E2M1 codes per byte; returns, for 8 codes in one word, four words of
// packed FP16 pairs (element 2j low, 2j+1 high) equal to value(code) * s_b.
__device__ __forceinline__ void fp4x8_to_f16(uint32_t w, uint32_t sb_pair, uint32_t out[4]) {
  // high bytes of the FP16 encodings of 0, 0.5, 1, 1.5 | 2, 3, 4, 6
  const uint32_t T0 = 0x3E3C3800u, T1 = 0x46444240u;
  uint32_t lo = w & 0x0F0F0F0Fu;              // codes of elements 0, 2, 4, 6
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;       // codes of elements 1, 3, 5, 7
  uint32_t he = __builtin_amdgcn_perm(T1, T0, lo & 0x07070707u) | ((lo & 0x08080808u) << 4);
  uint32_t ho = __builtin_amdgcn_perm(T1, T0, hi & 0x07070707u) | ((hi & 0x08080808u) << 4);
  // pair j: [0, he.byte j, 0, ho.byte j]; selector 0x0C gives a zero byte
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t s = 0x0Cu | ((uint32_t)j << 8) | (0x0Cu << 16) | ((uint32_t)(4 + j) << 24);
    uint32_t p = __builtin_amdgcn_perm(ho, he, s);
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 a = __builtin_bit_cast(h2, p);
    h2 b = __builtin_bit_cast(h2, sb_pair);
    out[j] = __builtin_bit_cast(uint32_t, a * b);
  }
}

__device__ __forceinline__ uint32_t e4m3_to_f16_pair(uint32_t code) {
  _Float16 h = (_Float16)e4m3_to_f32(code);     // exact
  uint32_t b = __builtin_bit_cast(uint16_t, h);
  return b | (b << 16);
}

// ------------------------------------------------------------ tile origin
struct TileOrigin {
  int64_t m0, m_end;      // rows [m0, m_end) of C (and of the grouped A row space)
  int group;
  bool active;
};

template <int BM>
__device__ __forceinline__ TileOrigin tile_origin(const GemmArgs& p, int mt) {
  TileOrigin o;
  if (p.num_groups == 0) {
    o.m0 = (int64_t)mt * BM;
    o.m_end = p.M;
    o.group = 0;
    o.active = o.m0 < p.M;
    return o;
  }
  // walk the groups: group g owns ceil(rows_g / BM) m-tiles
  int acc = 0;
  o.active = false;
  o.group = 0;
  o.m0 = 0;
  o.m_end = 0;
  for (int g = 0; g < p.num_groups; ++g) {
    int lo = p.offsets[g], hi = p.offsets[g + 1];
    int t = (hi - lo + BM - 1) / BM;
    if (mt < acc + t) {
      o.group = g;
      o.m0 = lo + (int64_t)(mt - acc) * BM;
      o.m_end = hi;
      o.active = true;
      break;
    }
    acc += t;
  }
  return o;
}

// ------------------------------------------------------------ the kernel
template <int PATH, int BM, int BN, bool BT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int ROWS = BM + BN;

  const int nt = blockIdx.x;
  const int mt = blockIdx.y;
  const TileOrigin to = tile_origin<BM>(p, mt);
  if (!to.active) return;
  const int64_t n0 = (int64_t)nt * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;

  // byte offset of this group's B matrix: FP8 1 B, NVFP4 1/2 B, BF16 2 B per element
  const int64_t gel = (int64_t)to.group * p.b_group_elems;
  const uint8_t* bbase = p.b + (PATH == P_FP8 ? gel : PATH == P_F16 ? (gel >> 1) : gel * 2);
  const uint8_t* bscl = p.b_scales ? p.b_scales + (int64_t)to.group * p.b_group_scales : nullptr;

  // ------------------------------------------------ global -> register staging
  // A: rows m0 .. m0+BM; per stage 128 LDS bytes per row.
  //   FP8 / BF16: 8 chunks of 16 B per row -> BM*8/256 chunks per lane.
  //   F16 (NVFP4): 4 blocks of 16 codes (8 B) per row -> BM*4/256 per lane.
  constexpr int A_CH = PATH == P_F16 ? BM * 4 / 256 : BM * 8 / 256;
  constexpr int B_CH = PATH == P_F16 ? BN * 4 / 256 : BN * 8 / 256;
  constexpr int KSTEP = PATH == P_FP8 ? 128 : 64;          // K elements per stage
  const int64_t nk = (p.K + KSTEP - 1) / KSTEP;

  // per-lane A row pointers (gather + group bounds resolved once)
  const uint8_t* arow[A_CH];
  int a_r[A_CH], a_c[A_CH];
  bool a_ok[A_CH];
  int64_t a_logical[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    int id = tid + 256 * i;
    int r = PATH == P_F16 ? id >> 2 : id >> 3;
    int c = PATH == P_F16 ? id & 3 : id & 7;
    a_r[i] = r;
    a_c[i] = c;
    int64_t m = to.m0 + r;
    a_ok[i] = m < to.m_end;
    int64_t src = m;
    if (a_ok[i] && p.row_index) src = p.row_index[m];
    if (!a_ok[i]) src = 0;
    a_logical[i] = src;
    int64_t esz = PATH == P_BF16 ? 2 : 1;
    arow[i] = PATH == P_F16 ? p.a + src * (p.lda >> 1) : p.a + src * p.lda * esz;
  }

  uint4 ra[A_CH];
  uint2 ra4[A_CH];
  uint32_t rsa[A_CH];
  uint4 rb[BT ? 1 : B_CH];
  uint2 rb4[BT ? 1 : B_CH];
  uint32_t rsb[BT ? 1 : B_CH];
  // transposed-B staging: a lane owns 4 (BF16/F16) or 8 (FP8) K rows x 8 N
  constexpr int BT_KR = PATH == P_FP8 ? 8 : 4;
  uint32_t rbt[BT ? (PATH == P_FP8 ? 16 : (PATH == P_BF16 ? 16 : 4)) : 1];
  uint32_t rbt_s[BT ? 1 : 1];

  auto load_stage = [&](int64_t kt) {
    const int64_t k0 = kt * KSTEP;
    // ---- A
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (PATH == P_F16) {
        int64_t kb = (k0 >> 4) + a_c[i];                 // 16-block index
        bool ok = a_ok[i] && kb * 16 < p.K;
        ra4[i] = ok ? *reinterpret_cast<const uint2*>(arow[i] + kb * 8) : make_uint2(0, 0);
        int64_t nb = p.K >> 4;
        rsa[i] = ok ? p.a_scales[scale_offset(a_logical[i], kb, nb, p.a_mfma_layout)] : 0u;
      } else {
        int64_t ke = k0 + a_c[i] * (PATH == P_FP8 ? 16 : 8);   // first element of the chunk
        bool ok = a_ok[i] && ke < p.K;
        int64_t boff = PATH == P_FP8 ? ke : ke * 2;
        ra[i] = ok ? *reinterpret_cast<const uint4*>(arow[i] + boff) : make_uint4(0, 0, 0, 0);
      }
    }
    // ---- B
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        int id = tid + 256 * i;
        int r = PATH == P_F16 ? id >> 2 : id >> 3;
        int c = PATH == P_F16 ? id & 3 : id & 7;
        int64_t n = n0 + r;
        bool rok = n < p.N;
        if (PATH == P_F16) {
          int64_t kb = (k0 >> 4) + c;
          bool ok = rok && kb * 16 < p.K;
          rb4[i] = ok ? *reinterpret_cast<const uint2*>(bbase + n * (p.ldb >> 1) + kb * 8) : make_uint2(0, 0);
          int64_t nb = p.K >> 4;
          uint32_t s = 0;
          if (ok) s = p.b_tile ? bscl[(n >> 4) * nb + kb] : bscl[scale_offset(n, kb, nb, p.b_mfma_layout)];
          rsb[i] = s;
        } else {
          int64_t ke = k0 + c * (PATH == P_FP8 ? 16 : 8);
          bool ok = rok && ke < p.K;
          int64_t boff = PATH == P_FP8 ? n * p.ldb + ke : (n * p.ldb + ke) * 2;
          rb[i] = ok ? *reinterpret_cast<const uint4*>(bbase + boff) : make_uint4(0, 0, 0, 0);
        }
      }
    } else {
      // lane -> (k group, n group of 8); K and N are multiples of the tile
      const int kg = tid / (BN / 8), ng = tid % (BN / 8);
      const int64_t kr = k0 + (int64_t)kg * BT_KR;
      const int64_t n = n0 + (int64_t)ng * 8;
      const bool ok = kr < p.K && n < p.N;
      if (PATH == P_FP8) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint2 v = ok ? *reinterpret_cast<const uint2*>(bbase + (kr + q) * p.ldb + n) : make_uint2(0, 0);
          rbt[2 * q] = v.x;
          rbt[2 * q + 1] = v.y;
        }
      } else if (PATH == P_BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint4 v = ok ? *reinterpret_cast<const uint4*>(bbase + ((kr + q) * p.ldb + n) * 2) : make_uint4(0, 0, 0, 0);
          rbt[4 * q] = v.x; rbt[4 * q + 1] = v.y; rbt[4 * q + 2] = v.z; rbt[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          rbt[q] = ok ? *reinterpret_cast<const uint32_t*>(bbase + ((kr + q) * p.ldb + n) / 2) : 0u;
        // one 16x16 tile covers these 4 rows x 8 columns
        rbt_s[0] = ok ? bscl[(kr >> 4) * (p.N >> 4) + (n >> 4)] : 0u;
      }
    }
  };

  auto store_stage = [&](uint8_t* L) {
    uint8_t* LA = L;
    uint8_t* LB = L + BM * LDS_ROW;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (PATH == P_F16) {
        uint32_t sp = e4m3_to_f16_pair(rsa[i]);
        uint32_t o[8];
        fp4x8_to_f16(ra4[i].x, sp, o);
        fp4x8_to_f16(ra4[i].y, sp, o + 4);
        uint8_t* d = LA + a_r[i] * LDS_ROW + a_c[i] * 32;
        *reinterpret_cast<uint4*>(d) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(d + 16) = make_uint4(o[4], o[5], o[6], o[7]);
      } else {
        *reinterpret_cast<uint4*>(LA + a_r[i] * LDS_ROW + a_c[i] * 16) = ra[i];
      }
    }
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        int id = tid + 256 * i;
        int r = PATH == P_F16 ? id >> 2 : id >> 3;
        int c = PATH == P_F16 ? id & 3 : id & 7;
        if (PATH == P_F16) {
          uint32_t sp = e4m3_to_f16_pair(rsb[i]);
          uint32_t o[8];
          fp4x8_to_f16(rb4[i].x, sp, o);
          fp4x8_to_f16(rb4[i].y, sp, o + 4);
          uint8_t* d = LB + r * LDS_ROW + c * 32;
          *reinterpret_cast<uint4*>(d) = make_uint4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<uint4*>(d + 16) = make_uint4(o[4], o[5], o[6], o[7]);
        } else {
          *reinterpret_cast<uint4*>(LB + r * LDS_ROW + c * 16) = rb[i];
        }
      }
    } else {
      const int kg = tid / (BN / 8), ng = tid % (BN / 8);
      if (PATH == P_FP8) {
        // 8 K rows x 8 N bytes -> for each n, 8 consecutive K bytes
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lo |= ((rbt[2 * q + (j >> 2)] >> (8 * (j & 3))) & 0xFFu) << (8 * q);
            hi |= ((rbt[2 * (q + 4) + (j >> 2)] >> (8 * (j & 3))) & 0xFFu) << (8 * q);
          }
          *reinterpret_cast<uint2*>(LB + (ng * 8 + j) * LDS_ROW + kg * 8) = make_uint2(lo, hi);
        }
      } else if (PATH == P_BF16) {
        // 4 K rows x 8 N values -> for each n, 4 consecutive K values (8 B)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = (rbt[4 * q + (j >> 1)] >> (16 * (j & 1))) & 0xFFFFu;
          *reinterpret_cast<uint2*>(LB + (ng * 8 + j) * LDS_ROW + kg * 8) =
              make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
        }
      } else {
        uint32_t sp = e4m3_to_f16_pair(rbt_s[0]);
        uint32_t h[4][4];     // [k row][pair]: FP16 of n = 2p, 2p+1
#pragma unroll
        for (int q = 0; q < 4; ++q) fp4x8_to_f16(rbt[q], sp, h[q]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = (h[q][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          *reinterpret_cast<uint2*>(LB + (ng * 8 + j) * LDS_ROW + kg * 8) =
              make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
        }
      }
    }
  };

  // ------------------------------------------------ MXFP8 scale registers
  // For the scaled MFMA a lane supplies the E8M0 byte of (its row, its K block).
  auto a_scale_fp8 = [&](int tm, int64_t kblk) -> uint32_t {
    int64_t m = to.m0 + wm * WM + tm * 32 + (lane & 31);
    if (m >= to.m_end || kblk * 32 >= p.K) return 127u;
    int64_t src = p.row_index ? p.row_index[m] : m;
    return p.a_scales[scale_offset(src, kblk, p.K >> 5, p.a_mfma_layout)];
  };
  auto b_scale_fp8 = [&](int tn, int64_t kblk) -> uint32_t {
    int64_t n = n0 + wn * WN + tn * 32 + (lane & 31);
    if (n >= p.N || kblk * 32 >= p.K) return 127u;
    if (BT) return bscl[kblk * (p.N >> 5) + (n >> 5)];        // stored [K/32, N/32]
    if (p.b_tile) return bscl[(n >> 5) * (p.K >> 5) + kblk];
    return bscl[scale_offset(n, kblk, p.K >> 5, p.b_mfma_layout)];
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  load_stage(0);
  store_stage(lds);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const uint8_t* Lcur = lds + cur * (ROWS * LDS_ROW);
    const uint8_t* LA = Lcur + (wm * WM) * LDS_ROW;
    const uint8_t* LB = Lcur + (BM + wn * WN) * LDS_ROW;
    if (PATH == P_FP8) {
      uint32_t sa[TM][2], sb[TN][2];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) sa[tm][ks] = a_scale_fp8(tm, kt * 4 + ks * 2 + (lane >> 5));
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) sb[tn][ks] = b_scale_fp8(tn, kt * 4 + ks * 2 + (lane >> 5));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i af[TM], bf[TN];
        // lane (row r, half h) holds K bytes [16h, 16h+16) of block 0 and
        // [32+16h, 32+16h+16) of block 1 of this 64-wide slice; the scale of
        // (row r, block j) is taken from lane r + 32j.
        const int koff = ks * 64 + (lane >> 5) * 16;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const uint8_t* s = LA + (tm * 32 + (lane & 31)) * LDS_ROW + koff;
          uint4 x0 = *reinterpret_cast<const uint4*>(s);
          uint4 x1 = *reinterpret_cast<const uint4*>(s + 32);
          af[tm] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const uint8_t* s = LB + (tn * 32 + (lane & 31)) * LDS_ROW + koff;
          uint4 x0 = *reinterpret_cast<const uint4*>(s);
          uint4 x1 = *reinterpret_cast<const uint4*>(s + 32);
          bf[tn] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[tm], bf[tn], acc[tm][tn], 0, 0, 0, (int)sa[tm][ks], 0, (int)sb[tn][ks]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int koff = ks * 32 + (lane >> 5) * 16;   // bytes
        uint4 af[TM], bf[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          af[tm] = *reinterpret_cast<const uint4*>(LA + (tm * 32 + (lane & 31)) * LDS_ROW + koff);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          bf[tn] = *reinterpret_cast<const uint4*>(LB + (tn * 32 + (lane & 31)) * LDS_ROW + koff);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            if (PATH == P_F16)
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(v8h, af[tm]), __builtin_bit_cast(v8h, bf[tn]), acc[tm][tn], 0, 0, 0);
            else
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(v8bf, af[tm]), __builtin_bit_cast(v8bf, bf[tn]), acc[tm][tn], 0, 0, 0);
          }
      }
    }
    if (kt + 1 < nk) store_stage(lds + (cur ^ 1) * (ROWS * LDS_ROW));
    __syncthreads();
  }

  // ------------------------------------------------ epilogue
  float sbg = 1.0f;
  if (PATH == P_F16) sbg = p.b_gs[to.group];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int64_t n = n0 + wn * WN + tn * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = to.m0 + wm * WM + tm * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (m < to.m_end && n < p.N) {
          float v = acc[tm][tn][e];
          if (PATH == P_F16) {
            float sa = 1.0f;
            if (p.a_gs_per_row) {
              int64_t src = p.row_index ? p.row_index[m] : m;
              sa = p.a_gs[src];
            } else {
              sa = p.a_gs[0];
            }
            v = (v * sa) * sbg;
          }
          p.c[m * p.ldc + n] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
  }
}

// ------------------------------------------------------------ launcher
template <int PATH, int BM, int BN, bool BT>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  int64_t tiles_n = (a.N + BN - 1) / BN;
  int64_t tiles_m = a.num_groups == 0 ? (a.M + BM - 1) / BM : a.M / BM + a.num_groups;
  if (tiles_m < 1) tiles_m = 1;
  size_t lds = 2 * (size_t)(BM + BN) * LDS_ROW;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<PATH, BM, BN, BT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_kernel<PATH, BM, BN, BT>), dim3((unsigned)tiles_n, (unsigned)tiles_m),
                     dim3(256), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm(int path, bool bt, const GemmArgs& a, hipStream_t st) {
  if (path == P_FP8) return bt ? launch_t<P_FP8, 128, 128, true>(a, st) : launch_t<P_FP8, 128, 128, false>(a, st);
  if (path == P_F16) return bt ? launch_t<P_F16, 128, 128, true>(a, st) : launch_t<P_F16, 128, 128, false>(a, st);
  return bt ? launch_t<P_BF16, 128, 128, true>(a, st) : launch_t<P_BF16, 128, 128, false>(a, st);
}

}  // namespace mxq
