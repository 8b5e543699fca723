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
//    loader converts codes to FP16 (hardware conversion with unit scale, then
//    one packed FP16 multiply by s_b, both exact) on the way into LDS and the
//    inner loop runs v_mfma_f32_32x32x16_f16.  FP4 x FP8 products being exact
//    in FP16 is the same observation the Four-Over-Six work relies on ("NVFP4
//    RL training", Four-Over-Six section).  The FP32 second scales multiply
//    the accumulator in the epilogue.
//  * BF16: v_mfma_f32_32x32x16_bf16 (the dequantized-backward DGRAD).
//
// Workgroup: 256 lanes as 2 x 2 waves; a BM x BN output tile, each wave a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles.  An LDS row holds 128 bytes of K
// (128 FP8 or 64 FP16/BF16 values) as eight 16-byte chunks plus 16 bytes of
// padding; chunk c of row r sits in slot c ^ ((r >> 3) & 7).  The padding
// makes the 16-byte fragment reads of 8 consecutive rows conflict-free, and
// the XOR keeps writes of rows 8 apart (the transposed-B loader) on distinct
// banks.  The MFMA runs with B as its first operand, so each lane ends up
// with 4 consecutive output columns and the epilogue stores 8 bytes at a time.
// B may be stored transposed ([K, N], the FPROP weight copy read by DGRAD):
// the loader transposes R x 8 sub-blocks in registers (byte permutes).
// Grouped (MoE) launches map each workgroup to (group, m-tile) with a scan of
// the device-side group offsets.  Workgroup ids are remapped so that each of
// the 8 XCDs works on a contiguous range of output tiles (L2 locality).

#include "mxq_device.h"
#include "mxq_kernels.h"

namespace mxq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int LDS_ROW = 144;     // bytes per LDS row: 8 chunks of 16 + 16 pad

__device__ __forceinline__ int slot_of(int row, int chunk) { return chunk ^ ((row >> 3) & 7); }

// Raw buffer loads: the hardware range check returns zero for an offset at or
// beyond the buffer size, so tails need neither branches nor selects around
// the loads (branches would make the compiler drain every outstanding load,
// the prefetched stage included, before the LDS stores).  Offsets are 32-bit:
// every operand is below 2^31 bytes (checked by the host), and OOB = 2^31 is
// always out of range.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// ------------------------------------------------------------ FP4 -> FP16
// Eight E2M1 codes (one word, element 2j in the low nibble of byte j) times
// the block scale: four words of packed FP16 pairs.  Both steps are exact.
__device__ __forceinline__ void fp4x8_to_f16(uint32_t w, uint32_t sb_pair, uint32_t out[4]) {
  const h2 s = __builtin_bit_cast(h2, sb_pair);
  // unit scale: the exact code values (the conversion uses only the exponent
  // of its scale operand, so the E4M3 scale is applied by the multiply)
  const h2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const h2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const h2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const h2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  out[0] = __builtin_bit_cast(uint32_t, c0 * s);
  out[1] = __builtin_bit_cast(uint32_t, c1 * s);
  out[2] = __builtin_bit_cast(uint32_t, c2 * s);
  out[3] = __builtin_bit_cast(uint32_t, c3 * s);
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

// Transposes of R x 8 register blocks (R K-rows, 8 N-columns) into the R
// K-values of one column j, packed in K order.
// 16-bit values: row q holds 8 values in 4 words (column j = half j&1 of word j>>1).
template <int R>
__device__ __forceinline__ void transpose16(const uint32_t (*rows)[4], int j, uint32_t* out) {
  const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
  for (int q = 0; q < R / 2; ++q)
    out[q] = __builtin_amdgcn_perm(rows[2 * q + 1][j >> 1], rows[2 * q][j >> 1], sel);
}

// 8-bit values: row q holds 8 bytes in 2 words (column j = byte j&3 of word j>>2).
template <int R>
__device__ __forceinline__ void transpose8(const uint32_t (*rows)[2], int j, uint32_t* out) {
  const int w = j >> 2, b = j & 3;
  const uint32_t sel = (uint32_t)(b | ((4 + b) << 8) | (0x0C << 16) | (0x0C << 24));
#pragma unroll
  for (int q = 0; q < R / 4; ++q) {
    const uint32_t lo = __builtin_amdgcn_perm(rows[4 * q + 1][w], rows[4 * q][w], sel);
    const uint32_t hi = __builtin_amdgcn_perm(rows[4 * q + 3][w], rows[4 * q + 2][w], sel);
    out[q] = lo | (hi << 16);
  }
}

// ------------------------------------------------------------ the kernel
template <int PATH, int BM, int BN, bool BT, int DIST>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int ROWS = BM + BN;
  constexpr int STAGE_BYTES = ROWS * LDS_ROW;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int KSTEP = PATH == P_FP8 ? 128 : 64;          // K elements per stage

  // ---- XCD-aware tile id: workgroup b runs on XCD b % 8; give each XCD a
  // contiguous range of logical tiles.
  const int tiles_n = gridDim.x;
  const int G = gridDim.x * gridDim.y;
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  const int q8 = G >> 3, r8 = G & 7, x = b & 7;
  const int logical = x * q8 + (x < r8 ? x : r8) + (b >> 3);
  const int nt = logical % tiles_n;
  const int mt = logical / tiles_n;

  const TileOrigin to = tile_origin<BM>(p, mt);
  if (!to.active) return;
  const int64_t n0 = (int64_t)nt * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // byte offset of this group's B matrix: FP8 1 B, NVFP4 1/2 B, BF16 2 B per element
  const int64_t gel = (int64_t)to.group * p.b_group_elems;
  const uint8_t* bbase = p.b + (PATH == P_FP8 ? gel : PATH == P_F16 ? (gel >> 1) : gel * 2);
  const uint8_t* bscl = p.b_scales ? p.b_scales + (int64_t)to.group * p.b_group_scales : nullptr;

  // ------------------------------------------------ loader geometry
  // Row-major operands: a lane moves 16 global bytes per chunk.
  //   FP8 / BF16: 16 B = one LDS chunk; 8 chunks per row per stage.
  //   NVFP4: 16 B of codes = 32 values = 4 LDS chunks; 2 per row per stage.
  constexpr int CPR = PATH == P_F16 ? 2 : 8;                 // global chunks per row per stage
  constexpr int A_CH = BM * CPR / 256;
  constexpr int B_CH = BN * CPR / 256;
  // Transposed B: a lane owns R K-rows x 8 N-columns per stage (256 lanes
  // cover KSTEP x BN exactly).
  constexpr int R_BT = KSTEP * BN / 2048;
  const int64_t nk = (p.K + KSTEP - 1) / KSTEP;

  // buffer resources: A (all stored rows), its scales, and this group's B
  constexpr int ESZ_A = PATH == P_BF16 ? 2 : 1;           // bytes per element (NVFP4: 1/2)
  const int64_t a_row_bytes = PATH == P_F16 ? (p.lda >> 1) : p.lda * ESZ_A;
  const int64_t b_row_bytes = PATH == P_F16 ? (p.ldb >> 1) : p.ldb * (PATH == P_BF16 ? 2 : 1);
  const rsrc_t rA = make_rsrc(p.a, p.a_rows * a_row_bytes);
  const rsrc_t rAs = make_rsrc(p.a_scales, p.a_scales ? p.a_rows * (p.K >> (PATH == P_FP8 ? 5 : 4)) : 0);
  const rsrc_t rB = make_rsrc(bbase, (BT ? p.K : p.N) * b_row_bytes);
  const rsrc_t rBs = make_rsrc(bscl, bscl ? p.b_group_scales : 0);

  // per-lane A rows (gather + group bounds resolved once); rows past the
  // tile's end read as zero and their outputs are never stored
  uint32_t a_off[A_CH];
  int a_r[A_CH], a_c[A_CH];
  bool a_ok[A_CH];
  int64_t a_src[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    int id = tid + 256 * i;
    int r = id / CPR, c = id % CPR;
    a_r[i] = r;
    a_c[i] = c;
    int64_t m = to.m0 + r;
    a_ok[i] = m < to.m_end;
    int64_t src = 0;
    if (a_ok[i]) src = p.row_index ? (int64_t)p.row_index[m] : m;
    a_src[i] = src;
    a_off[i] = (uint32_t)(src * a_row_bytes);
  }

  // DIST staging sets in registers: with DIST = 2 the stage being written to
  // LDS and the next one are both in flight.  Set indices are compile-time
  // constants once the K loop is unrolled by two.
  uint4 ra_[DIST][A_CH];
  uint32_t rsa_[DIST][A_CH][2];
  uint4 rb_[DIST][BT ? 1 : B_CH];
  uint32_t rsb_[DIST][BT ? 1 : B_CH][2];
  // transposed staging: FP8 R rows x 8 bytes (2 words); BF16 R rows x 8
  // values (4 words); NVFP4 R rows x 8 codes (1 word) + one 16x16 tile scale
  uint32_t rbt_[DIST][BT ? R_BT : 1][PATH == P_BF16 ? 4 : PATH == P_FP8 ? 2 : 1];
  uint32_t rbt_s_[DIST];
  // MXFP8: the E8M0 bytes each lane feeds its MFMAs, prefetched with the stage
  uint32_t sa_[2][TM][2], sb_[2][TN][2];
  int64_t sa_row[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t m = to.m0 + wm * WM + tm * 32 + (lane & 31);
    sa_row[tm] = m < to.m_end ? (p.row_index ? (int64_t)p.row_index[m] : m) : -1;
  }

  // MXFP8 scale bytes of stage kt into scale set `set` (two sets, by parity):
  // lane (r, h) needs, for each of its MFMA tiles, the E8M0 bytes of blocks
  // 4kt + h and 4kt + 2 + h of its row (one per 64-wide K slice).
  // Out-of-range blocks read 0 (their data are zero too).
  auto load_scales = [&](int64_t kt, int set) {
    if (PATH == P_FP8) {
      const int64_t KB = p.K >> 5;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int64_t kb = kt * 4 + ks * 2 + (lane >> 5);
          const bool ok = sa_row[tm] >= 0 && kb < KB;
          sa_[set][tm][ks] = bload1(rAs, ok ? (uint32_t)scale_offset(sa_row[tm], kb, KB, p.a_mfma_layout) : OOB);
        }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int64_t kb = kt * 4 + ks * 2 + (lane >> 5);
          const int64_t n = n0 + wn * WN + tn * 32 + (lane & 31);
          const bool ok = n < p.N && kb < KB;
          int64_t so;
          if (BT) so = kb * (p.N >> 5) + (n >> 5);                  // stored [K/32, N/32]
          else if (p.b_tile) so = (n >> 5) * KB + kb;
          else so = scale_offset(n, kb, KB, p.b_mfma_layout);
          sb_[set][tn][ks] = bload1(rBs, ok ? (uint32_t)so : OOB);
        }
    }
  };

  auto load_stage = [&](int64_t kt, int set) {
    const int64_t k0 = kt * KSTEP;
    uint4* ra = ra_[set];
    uint32_t (*rsa)[2] = rsa_[set];
    uint4* rb = rb_[set];
    uint32_t (*rsb)[2] = rsb_[set];
    auto& rbt = rbt_[set];
    uint32_t& rbt_s = rbt_s_[set];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      if (PATH == P_F16) {
        // 32 codes = blocks kb, kb+1; K % 16 == 0, so a block is in or out whole
        const int64_t kb = (k0 >> 4) + 2 * a_c[i];
        const bool ok0 = a_ok[i] && kb * 16 < p.K, ok1 = a_ok[i] && (kb + 1) * 16 < p.K;
        const uint2 lo = bload8(rA, ok0 ? a_off[i] + (uint32_t)(kb * 8) : OOB);
        const uint2 hi = bload8(rA, ok1 ? a_off[i] + (uint32_t)(kb * 8 + 8) : OOB);
        ra[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        // scale bytes of blocks kb, kb+1 are adjacent in every layout (kb
        // even); kept raw here and split at the LDS store, so that nothing
        // waits on this load before the next stage's compute
        rsa[i][0] = bload2(rAs, ok0 ? (uint32_t)scale_offset(a_src[i], kb, p.K >> 4, p.a_mfma_layout) : OOB);
      } else {
        const int64_t ke = k0 + a_c[i] * (PATH == P_FP8 ? 16 : 8);
        ra[i] = bload16(rA, (a_ok[i] && ke < p.K) ? a_off[i] + (uint32_t)(ke * ESZ_A) : OOB);
      }
    }
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int id = tid + 256 * i;
        const int r = id / CPR, c = id % CPR;
        const int64_t n = n0 + r;
        const bool rok = n < p.N;
        if (PATH == P_F16) {
          const int64_t kb = (k0 >> 4) + 2 * c;
          const bool ok0 = rok && kb * 16 < p.K, ok1 = rok && (kb + 1) * 16 < p.K;
          const uint32_t ro = (uint32_t)(n * b_row_bytes);
          const uint2 lo = bload8(rB, ok0 ? ro + (uint32_t)(kb * 8) : OOB);
          const uint2 hi = bload8(rB, ok1 ? ro + (uint32_t)(kb * 8 + 8) : OOB);
          rb[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const int64_t nb = p.K >> 4;
          const int64_t so = p.b_tile ? (n >> 4) * nb + kb : scale_offset(n, kb, nb, p.b_mfma_layout);
          rsb[i][0] = bload2(rBs, ok0 ? (uint32_t)so : OOB);
        } else {
          const int64_t ke = k0 + c * (PATH == P_FP8 ? 16 : 8);
          const int64_t boff = n * b_row_bytes + ke * (PATH == P_FP8 ? 1 : 2);
          rb[i] = bload16(rB, (rok && ke < p.K) ? (uint32_t)boff : OOB);
        }
      }
    } else {
      // lane -> (k group, n group of 8), n fastest for coalesced row reads;
      // K and N are multiples of the tile size, so a group is in or out whole.
      const int ng = tid % (BN / 8), kg = tid / (BN / 8);
      const int64_t kr = k0 + (int64_t)kg * R_BT;
      const int64_t n = n0 + (int64_t)ng * 8;
      const bool ok = kr < p.K && n < p.N;
#pragma unroll
      for (int q = 0; q < R_BT; ++q) {
        if (PATH == P_FP8) {
          const uint2 v = bload8(rB, ok ? (uint32_t)((kr + q) * b_row_bytes + n) : OOB);
          rbt[q][0] = v.x;
          rbt[q][1] = v.y;
        } else if (PATH == P_BF16) {
          const uint4 v = bload16(rB, ok ? (uint32_t)((kr + q) * b_row_bytes + n * 2) : OOB);
          rbt[q][0] = v.x; rbt[q][1] = v.y; rbt[q][2] = v.z; rbt[q][3] = v.w;
        } else {
          rbt[q][0] = bload4(rB, ok ? (uint32_t)((kr + q) * b_row_bytes + n / 2) : OOB);
        }
      }
      if (PATH == P_F16) rbt_s = bload1(rBs, ok ? (uint32_t)((kr >> 4) * (p.N >> 4) + (n >> 4)) : OOB);
    }
  };

  // Split the two raw scale bytes of blocks (kb, kb+1); the second is zeroed
  // when block kb+1 lies beyond K (its codes read as zero; a zero scale keeps
  // any byte found there out of the product).
  auto split_scales = [&](uint32_t raw, int64_t kb) -> uint2 {
    return make_uint2(raw & 0xFFu, (kb + 1) * 16 < p.K ? ((raw >> 8) & 0xFFu) : 0u);
  };

  auto store_stage = [&](uint8_t* L, int set, int64_t kt) {
    const int64_t k0s = kt * KSTEP;
    uint8_t* LA = L;
    uint8_t* LB = L + BM * LDS_ROW;
    const uint4* ra = ra_[set];
    const uint32_t (*rsa)[2] = rsa_[set];
    const uint4* rb = rb_[set];
    const uint32_t (*rsb)[2] = rsb_[set];
    const auto& rbt = rbt_[set];
    const uint32_t rbt_s = rbt_s_[set];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int r = a_r[i];
      uint8_t* row = LA + r * LDS_ROW;
      if (PATH == P_F16) {
        const uint32_t w[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
        const uint2 scs = split_scales(rsa[i][0], (k0s >> 4) + 2 * a_c[i]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t sp = e4m3_to_f16_pair(hh ? scs.y : scs.x);
          uint32_t o0[4], o1[4];
          fp4x8_to_f16(w[2 * hh], sp, o0);
          fp4x8_to_f16(w[2 * hh + 1], sp, o1);
          const int c = a_c[i] * 4 + 2 * hh;
          *reinterpret_cast<uint4*>(row + slot_of(r, c) * 16) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
          *reinterpret_cast<uint4*>(row + slot_of(r, c + 1) * 16) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
        }
      } else {
        *reinterpret_cast<uint4*>(row + slot_of(r, a_c[i]) * 16) = ra[i];
      }
    }
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int id = tid + 256 * i;
        const int r = id / CPR, c = id % CPR;
        uint8_t* row = LB + r * LDS_ROW;
        if (PATH == P_F16) {
          const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
          const uint2 scs = split_scales(rsb[i][0], (k0s >> 4) + 2 * c);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const uint32_t sp = e4m3_to_f16_pair(hh ? scs.y : scs.x);
            uint32_t o0[4], o1[4];
            fp4x8_to_f16(w[2 * hh], sp, o0);
            fp4x8_to_f16(w[2 * hh + 1], sp, o1);
            const int cc = c * 4 + 2 * hh;
            *reinterpret_cast<uint4*>(row + slot_of(r, cc) * 16) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
            *reinterpret_cast<uint4*>(row + slot_of(r, cc + 1) * 16) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
          }
        } else {
          *reinterpret_cast<uint4*>(row + slot_of(r, c) * 16) = rb[i];
        }
      }
    } else {
      const int ng = tid % (BN / 8), kg = tid / (BN / 8);
      constexpr int ESZ = PATH == P_FP8 ? 1 : 2;
      const int kbyte = kg * R_BT * ESZ;                     // this lane's K range: 8 or 16 bytes
      if (PATH == P_F16) {
        const uint32_t sp = e4m3_to_f16_pair(rbt_s);
        uint32_t hv[R_BT][4];
#pragma unroll
        for (int q = 0; q < R_BT; ++q) fp4x8_to_f16(rbt[q][0], sp, hv[q]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = ng * 8 + j;
          uint32_t o[R_BT / 2];
          transpose16<R_BT>(hv, j, o);
          uint8_t* dst = LB + r * LDS_ROW + slot_of(r, kbyte >> 4) * 16 + (kbyte & 15);
          if (R_BT == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
          else *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
        }
      } else if (PATH == P_BF16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = ng * 8 + j;
          uint32_t o[R_BT / 2];
          transpose16<R_BT>(reinterpret_cast<const uint32_t(*)[4]>(rbt), j, o);
          uint8_t* dst = LB + r * LDS_ROW + slot_of(r, kbyte >> 4) * 16 + (kbyte & 15);
          if (R_BT == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
          else *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = ng * 8 + j;
          uint32_t o[R_BT / 4];
          transpose8<R_BT>(reinterpret_cast<const uint32_t(*)[2]>(rbt), j, o);
          uint8_t* dst = LB + r * LDS_ROW + slot_of(r, kbyte >> 4) * 16 + (kbyte & 15);
          if (R_BT == 16) *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
          else *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
        }
      }
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto compute = [&](const uint8_t* Lcur, int set) {
    const uint8_t* LA = Lcur + (wm * WM) * LDS_ROW;
    const uint8_t* LB = Lcur + (BM + wn * WN) * LDS_ROW;
    const int r32 = lane & 31, h = lane >> 5;
    if (PATH == P_FP8) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // lane (row r, half h) holds K bytes [16h, 16h+16) of block 0 and
        // [32+16h, 32+16h+16) of block 1 of this 64-wide slice: chunks
        // 4ks + h and 4ks + 2 + h.
        v8i af[TM], bf[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int r = wm * WM + tm * 32 + r32;
          const uint8_t* sp = LA + (tm * 32 + r32) * LDS_ROW;
          uint4 x0 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + h) * 16);
          uint4 x1 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + 2 + h) * 16);
          af[tm] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int r = wn * WN + tn * 32 + r32;
          const uint8_t* sp = LB + (tn * 32 + r32) * LDS_ROW;
          uint4 x0 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + h) * 16);
          uint4 x1 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + 2 + h) * 16);
          bf[tn] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[tn], af[tm], acc[tm][tn], 0, 0, 0, (int)sb_[set][tn][ks], 0, (int)sa_[set][tm][ks]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int chunk = 2 * ks + h;                 // K values [16ks + 8h, +8)
        uint4 af[TM], bf[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int r = wm * WM + tm * 32 + r32;
          af[tm] = *reinterpret_cast<const uint4*>(LA + (tm * 32 + r32) * LDS_ROW + slot_of(r, chunk) * 16);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int r = wn * WN + tn * 32 + r32;
          bf[tn] = *reinterpret_cast<const uint4*>(LB + (tn * 32 + r32) * LDS_ROW + slot_of(r, chunk) * 16);
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            if (PATH == P_F16)
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(v8h, bf[tn]), __builtin_bit_cast(v8h, af[tm]), acc[tm][tn], 0, 0, 0);
            else
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(v8bf, bf[tn]), __builtin_bit_cast(v8bf, af[tm]), acc[tm][tn], 0, 0, 0);
          }
      }
    }
  };

  // Pipeline.  Stage s goes to LDS buffer s % 2 and uses MXFP8 scale set s % 2.
  //  DIST == 2: stage s is staged in register set s % 2; while stage kt is
  //    computed the loads of stages kt+1 and kt+2 are in flight; then stage
  //    kt+1 is written to LDS and stage kt+3 is loaded into the set it freed.
  //  DIST == 1 (large tiles, where two register sets would spill): stage kt+1
  //    is loaded while stage kt is computed, then written to LDS.
  uint8_t* const L0 = lds;
  uint8_t* const L1 = lds + STAGE_BYTES;
  // Loads past the last stage are issued anyway: their offsets are out of
  // range, so they read zeros and touch no memory, and the number of loads
  // in flight is the same on every path (a conditional load would make the
  // compiler drain the whole queue before each LDS store).
  if (DIST == 2) {
    load_stage(0, 0);
    load_scales(0, 0);
    load_stage(1, 1 % DIST);
    load_scales(1, 1);
    store_stage(L0, 0, 0);
    load_stage(2, 0);
    __syncthreads();
    // pairs of stages with no branch inside: stores of stages past the end
    // write zeros into a buffer that is never computed
    int64_t kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      compute(L0, 0);
      store_stage(L1, 1 % DIST, kt + 1);
      load_stage(kt + 3, 1 % DIST);
      load_scales(kt + 2, 0);
      __syncthreads();
      compute(L1, 1);
      store_stage(L0, 0, kt + 2);
      load_stage(kt + 4, 0);
      load_scales(kt + 3, 1);
      __syncthreads();
    }
    if (kt < nk) compute(L0, 0);          // odd stage count: the last stage
  } else {
    load_stage(0, 0);
    store_stage(L0, 0, 0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      uint8_t* const Lc = (kt & 1) ? L1 : L0;
      uint8_t* const Ln = (kt & 1) ? L0 : L1;
      load_stage(kt + 1, 0);
      load_scales(kt, 0);
      compute(Lc, 0);
      store_stage(Ln, 0, kt + 1);
      __syncthreads();
    }
  }

  // ------------------------------------------------ epilogue
  // With B as the MFMA's first operand, lane l holds for its output row
  // m = l % 32 the columns 8g + 4(l / 32) + i, i = 0..3, in acc[4g + i].
  float sbg = 1.0f;
  if (PATH == P_F16) sbg = p.b_gs[to.group];
  const bool vec_ok = ((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 7) == 0);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t m = to.m0 + wm * WM + tm * 32 + (lane & 31);
    if (m >= to.m_end) continue;
    float sa = 1.0f;
    if (PATH == P_F16) sa = p.a_gs_per_row ? p.a_gs[sa_row[tm]] : p.a_gs[0];
    uint16_t* crow = p.c + m * p.ldc;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * WN + tn * 32 + g * 8 + (lane >> 5) * 4;
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[tm][tn][4 * g + i];
          if (PATH == P_F16) v = (v * sa) * sbg;
          o[i] = f32_to_bf16_rne(v);
        }
        if (vec_ok && n + 3 < p.N) {
          *reinterpret_cast<uint2*>(crow + n) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (n + i < p.N) crow[n + i] = (uint16_t)o[i];
        }
      }
    }
  }
}

// ------------------------------------------------------------ launcher
template <int PATH, int BM, int BN, bool BT, int DIST>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  int64_t tiles_n = (a.N + BN - 1) / BN;
  int64_t tiles_m = a.num_groups == 0 ? (a.M + BM - 1) / BM : a.M / BM + a.num_groups;
  if (tiles_m < 1) tiles_m = 1;
  if (tiles_n * tiles_m >= (1ll << 31) || tiles_m > 65535) return hipErrorInvalidValue;
  size_t lds = 2 * (size_t)(BM + BN) * LDS_ROW;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<PATH, BM, BN, BT, DIST>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_kernel<PATH, BM, BN, BT, DIST>), dim3((unsigned)tiles_n, (unsigned)tiles_m),
                     dim3(256), lds, st, a);
  return hipGetLastError();
}

// Tile choice: the largest tile that still gives every CU work.  A 256x256
// tile keeps each wave's MFMA block at 128x128, where fragment traffic is
// about half the LDS bandwidth; 128x128 trades that for occupancy on small
// GEMMs.
static int choose_tile(const GemmArgs& a) {
  const int64_t cus = 256;
  auto tiles = [&](int bm, int bn) {
    int64_t tm = a.num_groups == 0 ? (a.M + bm - 1) / bm : a.M / bm + a.num_groups;
    return tm * ((a.N + bn - 1) / bn);
  };
  if (tiles(256, 256) >= cus) return 2;
  if (tiles(256, 128) >= cus) return 1;
  return 0;
}

template <int PATH, bool BT>
static hipError_t launch_p(const GemmArgs& a, hipStream_t st) {
  int t = choose_tile(a);
  // the FP8 256x256 variant needs more than 512 registers per lane (it would
  // spill), so FP8 stops at 256x128
  if (PATH == P_FP8 && t == 2) t = 1;
  switch (t) {
    case 2: return launch_t<PATH, 256, 256, BT, 1>(a, st);
    case 1: return launch_t<PATH, 256, 128, BT, PATH == P_BF16 ? 2 : 1>(a, st);
    default: return launch_t<PATH, 128, 128, BT, 2>(a, st);
  }
}

hipError_t launch_gemm(int path, bool bt, const GemmArgs& a, hipStream_t st) {
  if (path == P_FP8) return bt ? launch_p<P_FP8, true>(a, st) : launch_p<P_FP8, false>(a, st);
  if (path == P_F16) return bt ? launch_p<P_F16, true>(a, st) : launch_p<P_F16, false>(a, st);
  return bt ? launch_p<P_BF16, true>(a, st) : launch_p<P_BF16, false>(a, st);
}

}  // namespace mxq
