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
// Workgroup: 4 or 8 waves as a WGM x WGN grid; a BM x BN output tile, each wave a
// (BM/WGM) x (BN/WGN) block of 32x32 MFMA tiles.  An LDS row holds 128 bytes
// of K (128 FP8 or 64 FP16/BF16 values) as eight 16-byte chunks, placed by an
// XOR swizzle that keeps the fragment reads and the loader writes free of
// bank conflicts (slot_of).  The MFMA runs with B as its first operand, so each lane ends up
// with 4 consecutive output columns and the epilogue stores 8 bytes at a time.
// B may be stored transposed ([K, N], the FPROP weight copy read by DGRAD):
// the loader transposes R x 8 sub-blocks in registers (byte permutes).
// Grouped (MoE) launches map each workgroup to (group, m-tile) with a scan of
// the device-side group offsets.  Workgroup ids are remapped so that each of
// the 8 XCDs works on a contiguous range of output tiles (L2 locality).

#include "mxq_device.h"
#include "mxq_kernels.h"
#include "nvfp4_device.h"

#include <atomic>
#include <type_traits>

namespace mxq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int LDS_ROW = 128;     // bytes per LDS row: 8 chunks of 16

// LDS bank model of gfx950 (measured with per-pattern bank-conflict counters):
// a 16-byte read serves 16 lanes per cycle over 64 banks of 4 bytes, a
// 16-byte write 8 lanes per cycle over 32 banks (128 bytes; address bit 7
// does not separate them).  A row is 128 bytes, so for reads rows r and r + 1
// use opposite bank halves, for writes the same banks.  Chunk c of row r goes
// to slot c ^ f(r), f(r) = ((r >> 1) ^ (r >> 4) ^ (r & 1)) & 7:
//  * fragment reads (16 consecutive rows from a multiple of 16, one chunk):
//    the 8 even rows get 8 distinct slots, and so do the 8 odd rows;
//  * row-major loader writes, 8 lanes = one row x 8 chunks (FP8, BF16) or
//    rows 2i, 2i + 1 x 4 chunks of one parity (NVFP4's two FP16 slots per
//    code block): f(2i + 1) = f(2i) ^ 1 sends the two rows to opposite
//    parities, so the 8 lanes cover the 32 banks once;
//  * transposed-B writes (lanes on rows 8 apart, so r & 1 is common to all).
__device__ __forceinline__ int slot_of(int row, int chunk) {
  return chunk ^ (((row >> 1) ^ (row >> 4) ^ (row & 1)) & 7);
}

// Raw buffer loads: the hardware range check returns zero for an offset at or
// beyond the buffer size, so tails need neither branches nor selects around
// the loads (branches would make the compiler drain every outstanding load,
// the prefetched stage included, before the LDS stores).  Offsets are 32-bit:
// every operand is below 2^31 bytes (checked by the host), so any offset with
// bit 31 set is out of range.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
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
// The offset itself when ok, else one at or beyond 2^31 (out of range).  Pure
// arithmetic: a select here tends to be turned into a branch around two copies
// of the load, which drains the loads in flight.
__device__ __forceinline__ uint32_t in_range(bool ok, uint32_t off) {
  return off | ((uint32_t)!ok << 31);
}

// 16 bytes of output with the non-temporal hint: a GEMM's output is not read
// again by the kernel, and streaming it past the caches leaves them to the
// operand panels (config-5 NVFP4 GEMMs 0.5-2% faster)
__device__ __forceinline__ void store_nt16(uint16_t* dst, uint4 v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(dst));
}

// ------------------------------------------------------------ FP4 -> FP16
// Eight E2M1 codes (one word, element 2j in the low nibble of byte j) times
// the block scale: four words of packed FP16 pairs.  Both steps are exact.
__device__ __forceinline__ void fp4x8_to_f16(uint32_t w, h2 s, uint32_t out[4]) {
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

// E4M3 byte 0 of v as FP16 (exact: every E4M3 value is an FP16 normal), in
// both halves; the splat folds into the multiply's operand select.  The
// packed conversion (bytes 0 and 1) needs no old value to merge into, unlike
// the single-byte form, which costs a register clear per scale.
__device__ __forceinline__ h2 e4m3_to_h2(uint32_t v) {
  const h2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
  return h2{r.x, r.x};
}

// ------------------------------------------------------------ tile origin
struct TileOrigin {
  int64_t m0, m_end;      // rows [m0, m_end) of C (and of the grouped A row space)
  int group;
  bool active;
};

// Grouped launches: group g owns ceil(rows_g / BM) m-tiles, in group order.
// The offsets are read by the whole wave at once: lane l takes groups
// base + 4l .. base + 4l + 3 of each 256-group chunk (five offsets, one
// round of loads), and a wave prefix sum of the per-lane tile counts places
// the chunk.  Every wave computes the same wave-uniform result.
struct GroupChunk {
  int o[5];        // offsets[base + 4l + u], u = 0..4 (clamped to the last)
  int cnt;         // m-tiles of this lane's (up to) four groups
  int incl;        // inclusive prefix sum of cnt over lanes 0..l
};

template <int BM>
__device__ __forceinline__ GroupChunk group_chunk(const GemmArgs& p, int base, int lane) {
  GroupChunk c;
  const int G = p.num_groups;
  const int g0 = base + 4 * lane;
#pragma unroll
  for (int u = 0; u < 5; ++u) c.o[u] = p.offsets[min(g0 + u, G)];
  c.cnt = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (g0 + u < G) c.cnt += (c.o[u + 1] - c.o[u] + BM - 1) / BM;
  c.incl = c.cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(c.incl, d, 64);
    if (lane >= d) c.incl += y;
  }
  return c;
}

// total m-tiles over all groups (wave-uniform)
template <int BM>
__device__ __forceinline__ int group_mtiles(const GemmArgs& p, int lane) {
  int total = 0;
  for (int base = 0; base < p.num_groups; base += 256)
    total += __shfl(group_chunk<BM>(p, base, lane).incl, 63, 64);
  return __builtin_amdgcn_readfirstlane(total);
}

template <int BM>
__device__ __forceinline__ TileOrigin tile_origin(const GemmArgs& p, int mt, int lane) {
  TileOrigin o;
  if (p.num_groups == 0) {
    o.m0 = (int64_t)mt * BM;
    o.m_end = p.M;
    o.group = 0;
    o.active = o.m0 < p.M;
    return o;
  }
  o.active = false;
  o.group = 0;
  o.m0 = 0;
  o.m_end = 0;
  int acc = 0;                                   // m-tiles of the chunks before
  for (int base = 0; base < p.num_groups; base += 256) {
    const GroupChunk c = group_chunk<BM>(p, base, lane);
    const uint64_t hit = __ballot(mt < acc + c.incl);
    if (hit) {
      const int L = __builtin_ctzll(hit);       // first lane whose groups reach mt
      int t0 = acc + __shfl(c.incl - c.cnt, L, 64);
      int ov[5];
#pragma unroll
      for (int u = 0; u < 5; ++u) ov[u] = __shfl(c.o[u], L, 64);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = (ov[u + 1] - ov[u] + BM - 1) / BM;   // zero past the last group
        if (!o.active && mt < t0 + t) {
          o.group = base + 4 * L + u;
          o.m0 = ov[u] + (int64_t)(mt - t0) * BM;
          o.m_end = ov[u + 1];
          o.active = true;
        }
        t0 += t;
      }
      break;
    }
    acc += __shfl(c.incl, 63, 64);
  }
  o.group = __builtin_amdgcn_readfirstlane(o.group);
  o.m0 = __builtin_amdgcn_readfirstlane((int)o.m0);
  o.m_end = __builtin_amdgcn_readfirstlane((int)o.m_end);
  o.active = __builtin_amdgcn_readfirstlane((int)o.active) != 0;
  return o;
}

// ------------------------------------------------------------ tile order
// XCD-aware tile id: workgroup b runs on XCD b % 8; each XCD gets a
// contiguous range of the G = tiles_m x tiles_n real tiles (a grouped grid is
// sized for the most m-tiles any split of M could need, and each XCD's
// surplus workgroups, the last in its dispatch order, exit: false).  Within
// the range, runs of gm_rows tile rows are walked column by column.
__device__ __forceinline__ bool xcd_tile(int tiles_m, int tiles_n, int gm_rows, int& mt, int& nt) {
  const int G = tiles_m * tiles_n;
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  const int q8 = G >> 3, r8 = G & 7, x = b & 7;
  if ((b >> 3) >= q8 + (x < r8 ? 1 : 0)) return false;
  const int logical = x * q8 + (x < r8 ? x : r8) + (b >> 3);
  const int tgrp = logical / (gm_rows * tiles_n), gin = logical - tgrp * gm_rows * tiles_n;
  const int gm = min(gm_rows, tiles_m - tgrp * gm_rows);
  mt = tgrp * gm_rows + gin % gm;
  nt = gin / gm;
  return true;
}

// Runs of tile rows for the walk above (1: row by row).  Runs of GM tile rows
// walked column by column let the tiles in flight on an XCD form a block that
// shares A and B panels in its L2 (row by row, each row of tiles streams all
// of B again).  GM keeps the block's A and B bytes about equal for the 32-64
// tiles an XCD runs at once: 8 rows of 128-row tiles, 4 of 256-row tiles.
// Measured on MI355X: DGRAD and WGRAD shapes (at most 64 tiles per row) gain
// 3-16%; rows longer than that (an FPROP with N = 24576) run faster in row
// order, where the eight XCDs walk the same B panels together; grouped
// launches keep row order too (neighbouring m-tiles belong to different
// experts), and so do launches whose whole B fits an XCD's 4 MB L2 (there,
// row order lets each XCD read only its own A rows: the 4096x768x2048 NVFP4
// FPROP read 12.8 MB grouped against 11.3 MB, in the same time).
__device__ __forceinline__ int tile_run_rows(const GemmArgs& p, int tiles_n, int bm, int64_t b_bytes) {
  return (p.num_groups || tiles_n > 64 || b_bytes <= ((int64_t)4 << 20)) ? 1 : (bm >= 256 ? 4 : 8);
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
// Template parameters: compute path, output tile BM x BN, transposed B, the
// register prefetch distance (1 or 2 stages), the wave grid WGM x WGN and the
// ping-pong schedule PP.
//
// PP (8 waves, two on each SIMD): waves 0-3 and 4-7 form two groups; group g
// computes output rows [g BM/2, (g+1) BM/2) and loads half of every stage
// (its A rows and half of the B rows).  The groups run one barrier phase
// apart: while one group issues MFMAs, the other converts and stores its half
// of the next stage and issues the global loads of the one after, so the
// matrix cores see one group's MFMAs in every phase.  Phase p (each ends in a
// workgroup barrier): group 0 computes stage p/2 (p even) or stores its half
// of stage p/2 + 1 (p odd); group 1 the reverse.  Stage t lives in LDS buffer
// t % 2, is written in phases 2t-2 and 2t-1 and read in phases 2t and 2t+1.
//
// SDW (MXFP8, K % 128 == 0): a stage's four 32-wide scale blocks of one row
// are four adjacent bytes in every scale layout, so each lane loads them as
// one word, shifts its half's byte to the bottom (byte h, 2 + h) and the MFMA
// selects byte 0 or 2 of that word (its scale byte select) for K step 0 or 1.
// Transposed B keeps byte loads (its blocks are a scale-row apart).
// SDW for NVFP4 (K % 64 == 0, and N % 64 == 0 for transposed B): the byte of
// each chunk's block is read as the aligned word that holds it (a stage's four
// blocks of a row are one word) and shifted down at the LDS store.  A byte
// load kept in flight across the loop back edge is an 8-bit value the
// compiler widens at the loop head, which waits for every load in flight
// (the prefetched stage's too); a word needs no widening.
//
// SS (stages per barrier): the NVFP4 two-set pipeline stages two K steps of
// 64 per barrier (BF16 measured slower with it) (two LDS stages per buffer, register sets per stage), so the
// fixed cost of a barrier phase (LDS latency at its start, the stores and the
// wait at its end) is paid once per 128 of K.
template <int PATH, bool BT, int DIST, bool PP>
constexpr int stages_per_barrier() { return (DIST == 2 && PATH == P_F16 && !BT && !PP) ? 2 : 1; }
//
// BD (B direct; row-major B, two-set pipeline, K % 64 == 0; launched for
// NVFP4 only, see gemm_b_direct):
// B skips LDS.  Each MFMA sums its 16 K values in any order as long as A and
// B agree, so K step ks of a stage takes, in the lane of K half h, the K
// values [32h + 8ks, +8) (all 16-bit paths use this order, so every tile
// gives the same bits): a lane's B values for
// the whole stage are then 32 consecutive K values of its column (one
// 16-byte load of NVFP4 codes plus the stage's scale word, or four 16-byte
// BF16 loads), loaded two stages ahead into registers, and the A fragments
// are read from LDS chunk 4h + ks.  This removes B's LDS writes and reads
// (a third of the LDS traffic of a 128x128 tile) at the cost of converting
// each B column once per wave row.
// B128: blockwise FP8 (MXQ_FMT_FP8_B128): 128-wide power-of-two scale blocks,
// one byte per row (or 128-row tile) and stage; a compile-time choice, since
// even an untaken branch on it in the stage loop slowed MXFP8 by 70%.
// SWI: the MoE gate_up GEMM with SwiGLU in its epilogue (NVFP4, row-major B).
// B holds gate rows [0, I) and up rows [I, 2I) (I = p.swiglu_inter, N = 2I);
// each wave's WN output columns take WN/2 gate rows and the matching WN/2 up
// rows (logical column q WN + j reads gate row q WN/2 + j, or up row
// I + q WN/2 + j - WN/2), so the epilogue pairs them in the wave's own LDS
// slab and writes H [M, I] = SwiGLU(gate, up) from the BF16 products, the
// values the unfused GEMM would store.  Needs I % 64 == 0.
template <int PATH, int BM, int BN, bool BT, int DIST, int WGM, int WGN, bool PP, bool SDW = false,
          bool BD = false, bool B128 = false, bool SWI = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmArgs p) {
  static_assert(!SDW || PATH != P_BF16, "scale words: MXFP8 and NVFP4 only");
  static_assert(!B128 || (PATH == P_FP8 && SDW), "128-wide blocks: FP8 path with scale words");
  static_assert(!SWI || (PATH == P_F16 && !BT), "fused SwiGLU: NVFP4, row-major B");
  static_assert(!BD || (PATH != P_FP8 && !BT && !PP && DIST == 2), "B direct: 16-bit MFMA, row-major B, two sets");
  static_assert(!BD || PATH != P_F16 || SDW, "B direct NVFP4 reads scale words");
  constexpr bool SDWB = SDW && !BT && PATH == P_FP8;
  constexpr bool F16W = SDW && PATH == P_F16;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NT = 64 * WGM * WGN;
  static_assert(!PP || (NT == 512 && DIST == 1 && WGM % 2 == 0), "ping-pong: 8 waves, one staging set");
  constexpr int LT = PP ? NT / 2 : NT;                      // threads loading one share
  constexpr int LBM = PP ? BM / 2 : BM, LBN = PP ? BN / 2 : BN;   // rows of a share
  constexpr int ROWS = BM + (BD ? 0 : BN);                   // B direct keeps no B rows in LDS
  constexpr int STAGE_BYTES = ROWS * LDS_ROW;
  constexpr int SS = stages_per_barrier<PATH, BT, DIST, PP>();
  constexpr int NS = DIST * SS;                               // register staging sets
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && TM >= 1 && TN >= 1, "wave tile");
  constexpr int KSTEP = PATH == P_FP8 ? 128 : 64;          // K elements per stage

  // ---- tile id (XCD-aware, xcd_tile; a grouped grid's real m-tile count
  // comes from the offsets)
  const int lane0 = threadIdx.x & 63;
  const int tiles_n = gridDim.x;
  const int tiles_m = p.num_groups ? group_mtiles<BM>(p, lane0) : (int)gridDim.y;
  const int64_t b_bytes = (int64_t)p.N * p.K * (PATH == P_BF16 ? 2 : 1) / (PATH == P_F16 ? 2 : 1);
  int mt, nt;
  if (!xcd_tile(tiles_m, tiles_n, tile_run_rows(p, tiles_n, BM, b_bytes), mt, nt)) return;

  const TileOrigin to = tile_origin<BM>(p, mt, lane0);
  if (!to.active) return;
  // Every operand is below 2^31 bytes (checked by the host), so K, N, row
  // indices and byte offsets inside A, B and their scales fit 32 bits.
  const int K = (int)p.K, N = (int)p.N;
  const int n0 = nt * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  // B row that feeds logical output column n (the identity unless SWI)
  auto brow = [&](int n) -> int {
    if constexpr (SWI) {
      constexpr int P = (BN / WGN) / 2;
      const int q = n / (2 * P), j = n - q * (2 * P);
      return j < P ? q * P + j : (int)p.swiglu_inter + q * P + (j - P);
    }
    return n;
  };
  // loader: thread within its share, and the share's first A and B row
  const int grp = PP ? (tid >> 8) : 0;
  const int ltid = PP ? (tid & 255) : tid;
  const int la0 = grp * LBM, lb0 = grp * LBN;

  // byte offset of this group's B matrix: FP8 1 B, NVFP4 1/2 B, BF16 2 B per element
  const int64_t gel = (int64_t)to.group * p.b_group_elems;
  const uint8_t* bbase = p.b + (PATH == P_FP8 ? gel : PATH == P_F16 ? (gel >> 1) : gel * 2);
  const uint8_t* bscl = p.b_scales ? p.b_scales + (int64_t)to.group * p.b_group_scales : nullptr;

  // ------------------------------------------------ loader geometry
  // Row-major operands, per lane and chunk:
  //   FP8 / BF16: 16 global bytes = one LDS chunk; 8 chunks per row per stage.
  //   NVFP4: 8 bytes of codes = one 16-value block (one scale byte) = 2 LDS
  //   chunks; 4 per row per stage.  K % 16 == 0, so a block is in or out of
  //   range whole, and an out-of-range block reads zero codes and a zero scale.
  constexpr int CPR = PATH == P_F16 ? 4 : 8;                 // global chunks per row per stage
  constexpr int CW = PATH == P_F16 ? 2 : 4;                  // words per chunk
  constexpr uint32_t CB = 4u * CW;                           // global bytes per chunk
  static_assert((LBM * CPR) % LT == 0 && (LBN * CPR) % LT == 0, "loader split");
  constexpr int A_CH = LBM * CPR / LT;
  constexpr int B_CH = BD ? 0 : LBN * CPR / LT;
  constexpr int B_CHA = B_CH > 0 ? B_CH : 1;                // array extent
  // Transposed B: a lane owns R K-rows x 8 N-columns per stage (LT lanes
  // cover KSTEP x LBN exactly).
  constexpr int R_BT = KSTEP * LBN / (8 * LT);
  static_assert(!BT || (R_BT >= (PATH == P_FP8 ? 4 : 2) && R_BT <= 16), "transposed loader");
  const int nk = (K + KSTEP - 1) / KSTEP;
  // bytes of K advanced per stage in a row-major operand row
  constexpr uint32_t ROW_STEP = PATH == P_F16 ? 32 : 128;

  // buffer resources: A (all stored rows), its scales, and this group's B
  constexpr int ESZ_A = PATH == P_BF16 ? 2 : 1;           // bytes per element (NVFP4: 1/2)
  const int64_t a_row_bytes = PATH == P_F16 ? (p.lda >> 1) : p.lda * ESZ_A;
  const int64_t b_row_bytes = PATH == P_F16 ? (p.ldb >> 1) : p.ldb * (PATH == P_BF16 ? 2 : 1);
  const rsrc_t rA = make_rsrc(p.a, p.a_rows * a_row_bytes);
  // (128-wide blocks: the size rounds up to whole words, since a scale byte is
  // fetched with the aligned word holding it; those bytes never cross a page
  // and are never used)
  const rsrc_t rAs = make_rsrc(p.a_scales, p.a_scales ? (PATH == P_FP8 && B128
                                                             ? (p.a_rows * (p.K >> 7) + 3) & ~int64_t(3)
                                                             : p.a_rows * (p.K >> (PATH == P_FP8 ? 5 : 4)))
                                                      : 0);
  const rsrc_t rB = make_rsrc(bbase, (BT ? p.K : p.N) * b_row_bytes);
  const rsrc_t rBs = make_rsrc(bscl, bscl ? (PATH == P_FP8 && B128 ? (p.b_group_scales + 3) & ~int64_t(3)
                                                                     : p.b_group_scales)
                                         : 0);
  const uint32_t arb = (uint32_t)a_row_bytes, brb = (uint32_t)b_row_bytes;

  // Scale-byte offsets advance by a fixed step per stage: 4 blocks per stage
  // (NVFP4: 64 / 16; MXFP8: 128 / 32), i.e. 4 bytes in a linear layout and
  // one 128-byte chunk in the MFMA layout (blocks 4j..4j+3 of 32 rows).
  // Blockwise FP8 (128-wide blocks): one scale byte per row and stage, the
  // same for both 64-wide K slices and both lane halves.
  const int nb16 = K >> 4, nb32 = K >> 5, nb128 = K >> 7;
  const uint32_t a_sstep = B128 ? 1u : p.a_mfma_layout ? 128u : 4u;

  // per-lane A chunks: row, chunk, byte offset at stage 0, scale offset at stage 0
  int a_c[A_CH], a_r[A_CH];
  bool a_ok[A_CH];
  uint32_t a_off[A_CH], a_soff[A_CH], a_ssh[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int id = ltid + LT * i;
    const int r = la0 + id / CPR, c = id % CPR;
    a_r[i] = r;
    a_c[i] = c;
    const int64_t m = to.m0 + r;
    a_ok[i] = m < to.m_end;
    int src = 0;
    if (a_ok[i]) src = p.row_index ? p.row_index[m] : (int)m;
    a_off[i] = (uint32_t)src * arb + (uint32_t)c * CB;
    a_soff[i] = PATH == P_F16 ? (uint32_t)scale_offset(src, c, nb16, p.a_mfma_layout) : 0u;
    a_ssh[i] = F16W ? 8u * (a_soff[i] & 3u) : 0u;
    if (F16W) a_soff[i] &= ~3u;
  }
  // per-lane B chunks (row-major B)
  int b_c[B_CHA], b_r[B_CHA];
  bool b_ok[B_CHA];
  uint32_t b_off[B_CHA], b_soff[B_CHA], b_ssh[B_CHA];
  const uint32_t b_sstep = (p.b_tile || !p.b_mfma_layout) ? 4u : 128u;
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int id = ltid + LT * i;
    const int r = lb0 + id / CPR, c = id % CPR;
    b_r[i] = r;
    b_c[i] = c;
    const int n = brow(n0 + r);
    b_ok[i] = !BT && n0 + r < N;
    b_off[i] = (uint32_t)n * brb + (uint32_t)c * CB;
    b_soff[i] = 0;
    if (PATH == P_F16 && !BT)
      b_soff[i] = p.b_tile ? (uint32_t)((n >> 4) * nb16 + c)
                           : (uint32_t)scale_offset(n, c, nb16, p.b_mfma_layout);
    b_ssh[i] = F16W ? 8u * (b_soff[i] & 3u) : 0u;
    if (F16W) b_soff[i] &= ~3u;
  }
  // NVFP4 with K % 64 == 0 (scale words): a stage is in or out of range as a
  // whole, so a lane's row offsets carry only its row's validity (bit 31) and
  // each stage adds one uniform term, the stage offset or 2^31 past the last
  // stage.  An invalid row's offset is taken at row 0; adding 2^31 to it
  // wraps to row 0's data, which only feeds that row's discarded outputs.
  constexpr bool KF = F16W && !BT;
  uint32_t a_voff[A_CH], a_svoff[A_CH], b_voff[B_CHA], b_svoff[B_CHA];
  if constexpr (KF) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      a_voff[i] = in_range(a_ok[i], a_off[i]);       // src is row 0 when invalid
      a_svoff[i] = in_range(a_ok[i], a_soff[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int n = b_ok[i] ? brow(n0 + b_r[i]) : 0;
      b_voff[i] = in_range(b_ok[i], (uint32_t)n * brb + (uint32_t)b_c[i] * CB);
      const uint32_t so = p.b_tile ? (uint32_t)((n >> 4) * nb16 + b_c[i])
                                   : (uint32_t)scale_offset(n, b_c[i], nb16, p.b_mfma_layout);
      b_svoff[i] = in_range(b_ok[i], so & ~3u);
    }
  }
  // transposed B: lane -> (k group, n group of 8); K and N are multiples of
  // the tile size, so a group is in or out whole.  Each lane's LDS stores are
  // 8-byte runs (its K range of one column) in rows 8 apart, and a store
  // instruction serves 16 lanes per cycle over 32 banks.  With the n groups
  // fastest, those 16 lanes wrote 8 distinct 16-byte slots at the same half
  // (two-way conflicts); instead each 16 lanes take 8 consecutive n groups
  // (8 distinct slots under slot_of) times two k groups of opposite parity
  // (the two halves of a slot): lane bits 0-2 pick the n group, bit 3 the k
  // parity, the higher bits the rest.  The global loads of a wave still cover
  // the same whole row segments.
  constexpr int NG = LBN / 8;
  const int bt_ng = lb0 / 8 + (NG % 16 == 0 ? (ltid & 7) + 8 * ((ltid >> 4) % (NG / 8)) : ltid % NG);
  const int bt_kg = NG % 16 == 0 ? ((ltid >> 3) & 1) + 2 * ((ltid >> 4) / (NG / 8)) : ltid / NG;
  const bool bt_nok = n0 + bt_ng * 8 < N;
  constexpr int ESZ_BT = PATH == P_FP8 ? 1 : 2;                // bytes per value in LDS
  const uint32_t bt_off = (uint32_t)(bt_kg * R_BT) * brb +
                          (PATH == P_F16 ? (uint32_t)(n0 + bt_ng * 8) / 2 : (uint32_t)(n0 + bt_ng * 8) * ESZ_BT);
  const uint32_t bt_step = (uint32_t)KSTEP * brb;
  const uint32_t bt_sidx = (uint32_t)(((bt_kg * R_BT) >> 4) * (N >> 4) + ((n0 + bt_ng * 8) >> 4));
  const uint32_t bt_soff = F16W ? bt_sidx & ~3u : bt_sidx;
  const uint32_t bt_ssh = F16W ? 8u * (bt_sidx & 3u) : 0u;
  const uint32_t bt_sstep = 4u * (uint32_t)(N >> 4);

  // B direct: lane (column n = l % 32 of each of its TN tiles, K half h) holds
  // the stage's 32 K values [32h, 32h + 32) of column n, by stage parity.
  constexpr int BDW = PATH == P_F16 ? 4 : 16;               // raw words per tile and stage
  uint32_t bdr_[2 * SS][BD ? TN : 1][BD ? BDW : 1];
  uint32_t bds_[2 * SS][BD ? TN : 1];                             // NVFP4: the stage's scale word
  uint32_t bd_off[BD ? TN : 1], bd_soff[BD ? TN : 1];
  bool bd_ok[BD ? TN : 1];
  if constexpr (BD) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = n0 + wn * WN + tn * 32 + (lane & 31);
      bd_ok[tn] = n < N;
      const int nn = bd_ok[tn] ? brow(n) : 0;
      bd_off[tn] = (uint32_t)nn * brb + (uint32_t)(lane >> 5) * (PATH == P_F16 ? 16u : 64u);
      bd_soff[tn] = PATH == P_F16 ? (p.b_tile ? (uint32_t)((nn >> 4) * nb16)
                                              : (uint32_t)scale_offset(nn, 0, nb16, p.b_mfma_layout))
                                  : 0u;
    }
  }
  // stage kt of B into set s (K % 64 == 0: a stage is in or out whole)
  auto load_bd = [&](int kt, int s) {
    if constexpr (BD) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const bool ok = bd_ok[tn] && kt < nk;
        const uint32_t o = bd_off[tn] + (uint32_t)kt * ROW_STEP;
        // with KF: the row's validity bit plus one uniform stage term
        const uint32_t ob = KF ? in_range(bd_ok[tn], bd_off[tn]) + (kt < nk ? (uint32_t)kt * ROW_STEP : 0x80000000u) : 0u;
#pragma unroll
        for (int j = 0; j < BDW / 4; ++j) {
          const uint4 v = bload16(rB, KF ? ob + 16u * j : in_range(ok, o + 16u * j));
          bdr_[s][tn][4 * j] = v.x; bdr_[s][tn][4 * j + 1] = v.y;
          bdr_[s][tn][4 * j + 2] = v.z; bdr_[s][tn][4 * j + 3] = v.w;
        }
        if (PATH == P_F16)
          bds_[s][tn] = bload4(rBs, in_range(bd_ok[tn], bd_soff[tn]) + (kt < nk ? (uint32_t)kt * b_sstep : 0x80000000u));
      }
    }
  };

  // DIST staging sets in registers: with DIST = 2 the stage being written to
  // LDS and the next one are both in flight.  Set indices are compile-time
  // constants once the K loop is unrolled by two.
  uint32_t ra_[NS][A_CH][CW];
  uint32_t rsa_[NS][A_CH];
  uint32_t rb_[NS][BT ? 1 : B_CHA][CW];
  uint32_t rsb_[NS][BT ? 1 : B_CHA];
  // transposed staging: FP8 R rows x 8 bytes (2 words); BF16 R rows x 8
  // values (4 words); NVFP4 R rows x 8 codes (1 word) + one 16x16 tile scale
  uint32_t rbt_[NS][BT ? R_BT : 1][PATH == P_BF16 ? 4 : PATH == P_FP8 ? 2 : 1];
  uint32_t rbt_s_[NS];

  // MXFP8: the E8M0 bytes each lane feeds its MFMAs, prefetched with the
  // stage.  Lane (r, h) needs, for each of its MFMA tiles, the bytes of blocks
  // 4kt + h and 4kt + 2 + h of its row (one per 64-wide K slice).
  uint32_t sa_[2][TM][2], sb_[2][TN][2];
  uint32_t sa_off[TM][2], sb_off[TN][2];
  bool sa_ok[TM], sb_ok[TN];
  int64_t sa_row[TM];
  const int hl = lane >> 5;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t m = to.m0 + wm * WM + tm * 32 + (lane & 31);
    sa_row[tm] = m < to.m_end ? (p.row_index ? (int64_t)p.row_index[m] : m) : -1;
    sa_ok[tm] = sa_row[tm] >= 0;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      sa_off[tm][ks] = (PATH == P_FP8 && sa_ok[tm])
                           ? (B128 ? (uint32_t)(sa_row[tm] * nb128)
                                       : (uint32_t)scale_offset(sa_row[tm], ks * 2 + hl, nb32, p.a_mfma_layout))
                           : 0u;
  }
  uint32_t sb_step = 4u;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int n = n0 + wn * WN + tn * 32 + (lane & 31);
    sb_ok[tn] = n < N;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kb = ks * 2 + hl;
      uint32_t so = 0;
      if (PATH == P_FP8) {
        if (B128) {
          if (BT) so = (uint32_t)(n >> 7);                              // stored [K/128, N/128]
          else if (p.b_tile) so = (uint32_t)((n >> 7) * nb128);
          else so = (uint32_t)(n * nb128);
        } else if (BT) so = (uint32_t)(kb * (N >> 5) + (n >> 5));       // stored [K/32, N/32]
        else if (p.b_tile) so = (uint32_t)((n >> 5) * nb32 + kb);
        else so = (uint32_t)scale_offset(n, kb, nb32, p.b_mfma_layout);
      }
      sb_off[tn][ks] = so;
    }
  }
  if (PATH == P_FP8)
    sb_step = B128 ? (BT ? (uint32_t)(N >> 7) : 1u)
                       : BT ? 4u * (uint32_t)(N >> 5) : (p.b_tile || !p.b_mfma_layout) ? 4u : 128u;

  auto load_scales = [&](int kt, int set) {
    if (PATH == P_FP8) {
      // (the word of blocks 4kt..4kt+3 starts hl bytes before block 4kt + hl)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        if constexpr (B128) {
          // 128-wide blocks: the stage's one byte, replicated into the bytes
          // the two K slices select
          const uint32_t o = sa_off[tm][0] + (uint32_t)kt;
          const bool ok = sa_ok[tm] && kt < nb128;
          sa_[set][tm][0] = ((bload4(rAs, in_range(ok, o & ~3u)) >> (8 * (o & 3u))) & 0xFFu) * 0x01010101u;
        } else if constexpr (SDW) {
          const bool ok = sa_ok[tm] && kt * 4 < nb32;
          sa_[set][tm][0] = bload4(rAs, in_range(ok, sa_off[tm][0] - hl + (uint32_t)kt * a_sstep)) >> (8 * hl);
        } else {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bool ok = sa_ok[tm] && kt * 4 + ks * 2 + hl < nb32;
            sa_[set][tm][ks] = bload1(rAs, in_range(ok, sa_off[tm][ks] + (uint32_t)kt * a_sstep));
          }
        }
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        if constexpr (B128 && SDWB) {
          const uint32_t o = sb_off[tn][0] + (uint32_t)kt * sb_step;
          const bool ok = sb_ok[tn] && kt < nb128;
          sb_[set][tn][0] = ((bload4(rBs, in_range(ok, o & ~3u)) >> (8 * (o & 3u))) & 0xFFu) * 0x01010101u;
        } else if constexpr (SDWB) {
          const bool ok = sb_ok[tn] && kt * 4 < nb32;
          sb_[set][tn][0] = bload4(rBs, in_range(ok, sb_off[tn][0] - hl + (uint32_t)kt * sb_step)) >> (8 * hl);
        } else if constexpr (B128) {
          // transposed B: the same byte for both K slices, from its aligned word
          const uint32_t o = sb_off[tn][0] + (uint32_t)kt * sb_step;
          const bool ok = sb_ok[tn] && kt < nb128;
          sb_[set][tn][0] = sb_[set][tn][1] = bload4(rBs, in_range(ok, o & ~3u)) >> (8 * (o & 3u));
        } else {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bool ok = sb_ok[tn] && kt * 4 + ks * 2 + hl < nb32;
            sb_[set][tn][ks] = bload1(rBs, in_range(ok, sb_off[tn][ks] + (uint32_t)kt * sb_step));
          }
        }
      }
    }
  };

  auto load_stage = [&](int kt, int set) {
    const int k0 = kt * KSTEP;
    auto& ra = ra_[set];
    uint32_t* rsa = rsa_[set];
    auto& rb = rb_[set];
    uint32_t* rsb = rsb_[set];
    auto& rbt = rbt_[set];
    uint32_t& rbt_s = rbt_s_[set];
    // one chunk into w[CW]; values per chunk: NVFP4 16, FP8 16, BF16 8
    auto chunk = [&](rsrc_t r, uint32_t off, uint32_t* w) {
      if (PATH == P_F16) {
        const uint2 v = bload8(r, off);
        w[0] = v.x; w[1] = v.y;
      } else {
        const uint4 v = bload16(r, off);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      }
    };
    constexpr int VPC = PATH == P_BF16 ? 8 : 16;
    if constexpr (KF) {
      const bool kin = kt < nk;
      const uint32_t kso = kin ? (uint32_t)kt * ROW_STEP : 0x80000000u;
      const uint32_t ksa = kin ? (uint32_t)kt * a_sstep : 0x80000000u;
      const uint32_t ksb = kin ? (uint32_t)kt * b_sstep : 0x80000000u;
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        chunk(rA, a_voff[i] + kso, ra[i]);
        rsa[i] = bload4(rAs, a_svoff[i] + ksa);
      }
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        chunk(rB, b_voff[i] + kso, rb[i]);
        rsb[i] = bload4(rBs, b_svoff[i] + ksb);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const bool ok = a_ok[i] && k0 + a_c[i] * VPC < K;
      chunk(rA, in_range(ok, a_off[i] + (uint32_t)kt * ROW_STEP), ra[i]);
      // the block's scale byte, kept raw until the LDS store so that nothing
      // waits on this load before the next stage's compute
      if (PATH == P_F16) {
        const uint32_t so = in_range(ok, a_soff[i] + (uint32_t)kt * a_sstep);
        rsa[i] = F16W ? bload4(rAs, so) : bload1(rAs, so);
      }
    }
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const bool ok = b_ok[i] && k0 + b_c[i] * VPC < K;
        chunk(rB, in_range(ok, b_off[i] + (uint32_t)kt * ROW_STEP), rb[i]);
        if (PATH == P_F16) {
          const uint32_t so = in_range(ok, b_soff[i] + (uint32_t)kt * b_sstep);
          rsb[i] = F16W ? bload4(rBs, so) : bload1(rBs, so);
        }
      }
    } else {
      const bool ok = bt_nok && k0 + bt_kg * R_BT < K;
      const uint32_t o = bt_off + (uint32_t)kt * bt_step;
#pragma unroll
      for (int q = 0; q < R_BT; ++q) {
        const uint32_t oq = in_range(ok, o + (uint32_t)q * brb);
        if (PATH == P_FP8) {
          const uint2 v = bload8(rB, oq);
          rbt[q][0] = v.x;
          rbt[q][1] = v.y;
        } else if (PATH == P_BF16) {
          const uint4 v = bload16(rB, oq);
          rbt[q][0] = v.x; rbt[q][1] = v.y; rbt[q][2] = v.z; rbt[q][3] = v.w;
        } else {
          rbt[q][0] = bload4(rB, oq);
        }
      }
      if (PATH == P_F16) {
        const uint32_t so = in_range(ok, bt_soff + (uint32_t)kt * bt_sstep);
        rbt_s = F16W ? bload4(rBs, so) : bload1(rBs, so);
      }
    }
  };

  // LDS store of a transposed column run of NW words (4, 8 or 16 bytes)
  auto store_run = [](uint8_t* dst, const uint32_t* o, int nw) {
    if (nw == 4) *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    else if (nw == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
    else *reinterpret_cast<uint32_t*>(dst) = o[0];
  };

  // One chunk -> LDS.  NVFP4: 16 codes of one block times its scale -> two
  // FP16 chunks (slots 2c, 2c + 1); otherwise the 16 bytes as they are.
  auto store_chunk = [&](uint8_t* row, int r, int c, const uint32_t* w, uint32_t sraw) {
    if (PATH == P_F16) {
      const h2 sp = e4m3_to_h2(sraw);
      uint32_t o0[4], o1[4];
      fp4x8_to_f16(w[0], sp, o0);
      fp4x8_to_f16(w[1], sp, o1);
      *reinterpret_cast<uint4*>(row + slot_of(r, 2 * c) * 16) = make_uint4(o0[0], o0[1], o0[2], o0[3]);
      *reinterpret_cast<uint4*>(row + slot_of(r, 2 * c + 1) * 16) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    } else {
      *reinterpret_cast<uint4*>(row + slot_of(r, c) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  auto store_stage = [&](uint8_t* L, int set) {
    uint8_t* LA = L;
    uint8_t* LB = L + BM * LDS_ROW;
    const auto& ra = ra_[set];
    const uint32_t* rsa = rsa_[set];
    const auto& rb = rb_[set];
    const uint32_t* rsb = rsb_[set];
    const auto& rbt = rbt_[set];
    const uint32_t rbt_s = rbt_s_[set];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) store_chunk(LA + a_r[i] * LDS_ROW, a_r[i], a_c[i], ra[i], rsa[i] >> a_ssh[i]);
    if (!BT) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) store_chunk(LB + b_r[i] * LDS_ROW, b_r[i], b_c[i], rb[i], rsb[i] >> b_ssh[i]);
    } else {
      const int kbyte = bt_kg * R_BT * ESZ_BT;         // this lane's K range: 4, 8 or 16 bytes
      if constexpr (PATH == P_F16) {
        const h2 sp = e4m3_to_h2(rbt_s >> bt_ssh);
        uint32_t hv[R_BT][4];
#pragma unroll
        for (int q = 0; q < R_BT; ++q) fp4x8_to_f16(rbt[q][0], sp, hv[q]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = bt_ng * 8 + j;
          uint32_t o[R_BT >= 2 ? R_BT / 2 : 1];
          transpose16<R_BT>(hv, j, o);
          store_run(LB + r * LDS_ROW + slot_of(r, kbyte >> 4) * 16 + (kbyte & 15), o, R_BT / 2);
        }
      } else if constexpr (PATH == P_BF16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = bt_ng * 8 + j;
          uint32_t o[R_BT >= 2 ? R_BT / 2 : 1];
          transpose16<R_BT>(reinterpret_cast<const uint32_t(*)[4]>(rbt), j, o);
          store_run(LB + r * LDS_ROW + slot_of(r, kbyte >> 4) * 16 + (kbyte & 15), o, R_BT / 2);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = bt_ng * 8 + j;
          uint32_t o[R_BT >= 4 ? R_BT / 4 : 1];
          transpose8<R_BT>(reinterpret_cast<const uint32_t(*)[2]>(rbt), j, o);
          store_run(LB + r * LDS_ROW + slot_of(r, kbyte >> 4) * 16 + (kbyte & 15), o, R_BT / 4);
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

  // One stage of MFMAs.  Fragment reads are software-pipelined: the reads of
  // K step ks + 1 are issued before the MFMAs of step ks (two register sets),
  // and scheduling barriers keep the compiler from folding the two back into
  // a read-wait-multiply chain that would expose the LDS latency every step.
  // Wave tiles with 8 or more MFMAs per K step keep one set (registers are
  // short there, and the step's MFMAs already outlast the next reads' latency
  // of the other wave on the SIMD).
  constexpr int FS = TM * TN >= 8 ? 1 : 2;
  auto compute = [&](const uint8_t* Lcur, int set) {
    const uint8_t* LA = Lcur + (wm * WM) * LDS_ROW;
    const uint8_t* LB = Lcur + (BM + wn * WN) * LDS_ROW;
    const int r32 = lane & 31, h = lane >> 5;
    if constexpr (PATH == P_FP8) {
      // lane (row r, half h) holds K bytes [16h, 16h+16) of block 0 and
      // [32+16h, 32+16h+16) of block 1 of each 64-wide slice: chunks
      // 4ks + h and 4ks + 2 + h.
      v8i af[FS][TM], bf[FS][TN];
      auto read = [&](int ks, int q) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int r = wm * WM + tm * 32 + r32;
          const uint8_t* sp = LA + (tm * 32 + r32) * LDS_ROW;
          uint4 x0 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + h) * 16);
          uint4 x1 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + 2 + h) * 16);
          af[q][tm] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int r = wn * WN + tn * 32 + r32;
          const uint8_t* sp = LB + (tn * 32 + r32) * LDS_ROW;
          uint4 x0 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + h) * 16);
          uint4 x1 = *reinterpret_cast<const uint4*>(sp + slot_of(r, 4 * ks + 2 + h) * 16);
          bf[q][tn] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
      };
      if (FS == 2) read(0, 0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int q = FS == 2 ? (ks & 1) : 0;
        if (FS == 1) read(ks, 0);
        else if (ks + 1 < 2) read(ks + 1, (ks + 1) & 1);
        if (FS == 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
          {
            const int sbv = (int)sb_[set][tn][SDWB ? 0 : ks], sav = (int)sa_[set][tm][SDW ? 0 : ks];
            if (ks == 0)
              acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bf[q][tn], af[q][tm], acc[tm][tn], 0, 0, 0, sbv, 0, sav);
            else
              acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bf[q][tn], af[q][tm], acc[tm][tn], 0, 0, SDWB ? 2 : 0, sbv, SDW ? 2 : 0, sav);
          }
        if (FS == 2) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // FH fragment sets: 1 (read each K step right before its MFMAs), 2 (the
      // next step's reads ahead of this step's MFMAs) or 4 (all four steps'
      // reads issued at once, so one LDS latency per stage, not per step).
      // 4 is taken where it measured faster: NVFP4 with small wave tiles in
      // the two-set pipeline, where the scheduler then also spreads the next
      // stage's FP4 -> FP16 conversion between the MFMAs (BF16 and the
      // ping-pong schedule measured slower with it).
      constexpr int FH = (PATH == P_F16 && !PP && !BT && TM * TN <= 2) ? 4 : FS;
      uint4 af[FH][TM], bf[FH][TN];
      auto read = [&](int ks, int q) {
        // K values [32h + 8ks, +8) of the stage (the order B direct needs;
        // every 16-bit path uses it so that all tiles sum alike)
        const int chunk = 4 * h + ks;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const int r = wm * WM + tm * 32 + r32;
          af[q][tm] = *reinterpret_cast<const uint4*>(LA + (tm * 32 + r32) * LDS_ROW + slot_of(r, chunk) * 16);
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          if constexpr (BD) {
            if constexpr (PATH == P_F16) {
              // block 2h + ks / 2 of the stage: byte 2h + ks / 2 of the scale word
              const h2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bds_[set][tn] >> (16 * h), 1.0f, false);
              const h2 sp = (ks >> 1) ? h2{s01.y, s01.y} : h2{s01.x, s01.x};
              uint32_t o[4];
              fp4x8_to_f16(bdr_[set][tn][ks], sp, o);
              bf[q][tn] = make_uint4(o[0], o[1], o[2], o[3]);
            } else {
              bf[q][tn] = make_uint4(bdr_[set][tn][4 * ks], bdr_[set][tn][4 * ks + 1],
                                     bdr_[set][tn][4 * ks + 2], bdr_[set][tn][4 * ks + 3]);
            }
          } else {
            const int r = wn * WN + tn * 32 + r32;
            bf[q][tn] = *reinterpret_cast<const uint4*>(LB + (tn * 32 + r32) * LDS_ROW + slot_of(r, chunk) * 16);
          }
        }
      };
      if (FH == 4) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) read(ks, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (FH == 2) read(0, 0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int q = FH == 4 ? ks : FH == 2 ? (ks & 1) : 0;
        if (FH == 1) read(ks, 0);
        else if (FH == 2 && ks + 1 < 4) read(ks + 1, (ks + 1) & 1);
        if (FH == 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            if constexpr (PATH == P_F16)
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(v8h, bf[q][tn]), __builtin_bit_cast(v8h, af[q][tm]), acc[tm][tn], 0, 0, 0);
            else
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(v8bf, bf[q][tn]), __builtin_bit_cast(v8bf, af[q][tm]), acc[tm][tn], 0, 0, 0);
          }
        if (FH == 2) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Pipeline.  Stage s goes to LDS buffer s % 2 and uses MXFP8 scale set s % 2.
  //  DIST == 2: stage s is staged in register set s % 2; while stage kt is
  //    computed the loads of stages kt+1 and kt+2 are in flight; then stage
  //    kt+1 is written to LDS.  The loop runs two stages per iteration so
  //    that every register-set index is a compile-time constant, and its
  //    loads are unconditional (past the end they are range-checked to zero),
  //    so the compiler can keep the other set's loads outstanding across the
  //    LDS stores instead of draining them.
  //  DIST == 1: the next stage's loads (and MXFP8 scales) are in flight
  //    during the compute.
  uint8_t* const L0 = lds;
  uint8_t* const L1 = lds + SS * STAGE_BYTES;
  if constexpr (PP) {
    // NVFP4: the group issuing MFMAs runs at a raised wave priority, so that
    // on each SIMD its instructions win the issue arbitration against the
    // other group's FP4 -> FP16 conversions and stores (a per-wave priority
    // inside the kernel; measured on the config-5 GEMMs: FPROP and WGRAD
    // 4-5% faster; the MXFP8 kernels, which convert nothing, 2% slower).
    auto compute_pp = [&](const uint8_t* L, int set) {
      if constexpr (PATH == P_F16) __builtin_amdgcn_s_setprio(1);
      compute(L, set);
      if constexpr (PATH == P_F16) __builtin_amdgcn_s_setprio(0);
    };
    // prologue: both halves of stage 0 in buffer 0, stage 1 staged in
    // registers, MXFP8 scale sets 0 and 1 for stages 0 and 1
    load_stage(0, 0);
    load_scales(0, 0);
    load_scales(1, 1);
    store_stage(L0, 0);
    load_stage(1, 0);
    __syncthreads();
    // Stage loop, unrolled by two so that buffer and scale-set indices are
    // constants.  The barrier count is the same for both groups (two per
    // stage); past the last stage the loads read zeros and the stores write
    // them into the idle buffer.
    if (grp == 0) {
      for (int kt = 0; kt < nk; kt += 2) {
        compute_pp(L0, 0);                      // C(kt)
        __syncthreads();
        store_stage(L1, 0);                  // M: stage kt+1 -> buffer 1
        load_stage(kt + 2, 0);
        load_scales(kt + 2, 0);
        __syncthreads();
        if (kt + 1 < nk) {
          compute_pp(L1, 1);                    // C(kt+1)
          __syncthreads();
          store_stage(L0, 0);                // M: stage kt+2 -> buffer 0
          load_stage(kt + 3, 0);
          load_scales(kt + 3, 1);
          __syncthreads();
        }
      }
    } else {
      for (int kt = 0; kt < nk; kt += 2) {
        store_stage(L1, 0);                  // M: stage kt+1 -> buffer 1
        load_stage(kt + 2, 0);
        load_scales(kt + 1, 1);
        __syncthreads();
        compute_pp(L0, 0);                      // C(kt)
        __syncthreads();
        if (kt + 1 < nk) {
          store_stage(L0, 0);                // M: stage kt+2 -> buffer 0
          load_stage(kt + 3, 0);
          load_scales(kt + 2, 0);
          __syncthreads();
          compute_pp(L1, 1);                    // C(kt+1)
          __syncthreads();
        }
      }
    }
  } else if (DIST == 2) {
    // super-stage u = stages u*SS .. u*SS + SS - 1, in LDS buffer u % 2 and
    // register sets (u % 2)*SS + j; past the last stage loads read zeros, so
    // a partial last super-stage adds zero products
    auto load_su = [&](int u, int s) {
#pragma unroll
      for (int j = 0; j < SS; ++j) load_stage(u * SS + j, s * SS + j);
    };
    auto scales_su = [&](int u, int s) {
#pragma unroll
      for (int j = 0; j < SS; ++j) load_scales(u * SS + j, s * SS + j);
    };
    auto bd_su = [&](int u, int s) {
#pragma unroll
      for (int j = 0; j < SS; ++j) load_bd(u * SS + j, s * SS + j);
    };
    auto store_su = [&](uint8_t* L, int s) {
#pragma unroll
      for (int j = 0; j < SS; ++j) store_stage(L + j * STAGE_BYTES, s * SS + j);
    };
    auto compute_su = [&](const uint8_t* L, int s) {
#pragma unroll
      for (int j = 0; j < SS; ++j) compute(L + j * STAGE_BYTES, s * SS + j);
    };
    const int nu = (nk + SS - 1) / SS;
    bd_su(0, 0);
    bd_su(1, 1);
    load_su(0, 0);
    scales_su(0, 0);
    load_su(1, 1);
    scales_su(1, 1);
    store_su(L0, 0);
    load_su(2, 0);
    __syncthreads();
    int u = 0;
    for (; u + 1 < nu; u += 2) {
      compute_su(L0, 0);
      bd_su(u + 2, 0);
      store_su(L1, 1);
      load_su(u + 3, 1);
      scales_su(u + 2, 0);
      __syncthreads();
      compute_su(L1, 1);
      bd_su(u + 3, 1);
      store_su(L0, 0);
      load_su(u + 4, 0);
      scales_su(u + 3, 1);
      __syncthreads();
    }
    if (u < nu) compute_su(L0, 0);          // odd super-stage count: the last one
  } else {
    // one register staging set; unrolled by two so that the MXFP8 scale set
    // of stage s (s % 2) is loaded a stage ahead, not right before its MFMAs
    load_stage(0, 0);
    load_scales(0, 0);
    store_stage(L0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      load_stage(kt + 1, 0);
      load_scales(kt + 1, 1);
      compute(L0, 0);
      store_stage(L1, 0);
      __syncthreads();
      if (kt + 1 < nk) {
        load_stage(kt + 2, 0);
        load_scales(kt + 2, 0);
        compute(L1, 1);
        store_stage(L0, 0);
        __syncthreads();
      }
    }
  }

  // ------------------------------------------------ epilogue
  // With B as the MFMA's first operand, lane l holds for its output row
  // m = l % 32 the columns 8g + 4(l / 32) + i, i = 0..3, in acc[4g + i].
  // Each wave stages one 32-row slab of its tile at a time in its own LDS
  // region (BF16, rows padded by 8 bytes), then reads it back row-wise so
  // that 8 lanes store one contiguous 128-byte run of C.
  __syncthreads();                       // every wave is past its last LDS read
  constexpr int EROW = WN * 2 + 8;       // bytes per staged row
  constexpr int ECH = WN / 8;            // 16-byte chunks per row
  constexpr int ERI = 64 / ECH;          // rows per read-back instruction
  static_assert((NT / 64) * 32 * EROW <= 2 * SS * STAGE_BYTES, "epilogue staging");
  uint8_t* const E = lds + wave * (32 * EROW);
  float sbg = 1.0f;
  if (PATH == P_F16) sbg = p.b_gs[to.group];
  const bool vec16 = ((p.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    float sa = 1.0f;
    if (PATH == P_F16) {
      const int64_t srow = sa_row[tm];
      sa = srow >= 0 ? (p.a_gs_per_row ? p.a_gs[srow] : p.a_gs[0]) : 0.0f;
    }
    uint8_t* const er = E + (lane & 31) * EROW + (lane >> 5) * 8;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = acc[tm][tn][4 * g + i];
          if (PATH == P_F16) v[i] = (v[i] * sa) * sbg;
        }
        *reinterpret_cast<uint2*>(er + (tn * 32 + g * 8) * 2) =
            make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
      }
    if constexpr (SWI) {
      // gate chunk cc and up chunk cc + ECH/2 of a staged row -> 8 values of H
      // (the wave's block of 2P logical columns is whole: 2I % WN == 0)
      constexpr int ECH2 = ECH / 2, ERI2 = 64 / ECH2;
      const bool wave_in = n0 + wn * WN < N;
#pragma unroll
      for (int it = 0; it < 32 / ERI2; ++it) {
        const int rr = it * ERI2 + lane / ECH2, cc = lane % ECH2;
        const uint4 gv = *reinterpret_cast<const uint4*>(E + rr * EROW + cc * 16);
        const uint4 uv = *reinterpret_cast<const uint4*>(E + rr * EROW + (cc + ECH2) * 16);
        const int64_t m = to.m0 + wm * WM + tm * 32 + rr;
        const int hc = ((n0 + wn * WN) >> 1) + cc * 8;
        if (wave_in && m < to.m_end) {
          const uint4 hv = make_uint4(swiglu_bf16x2(gv.x, uv.x), swiglu_bf16x2(gv.y, uv.y),
                                      swiglu_bf16x2(gv.z, uv.z), swiglu_bf16x2(gv.w, uv.w));
          uint16_t* const dst = p.c + m * p.ldc + hc;
          if (vec16) {
            *reinterpret_cast<uint4*>(dst) = hv;
          } else {
            const uint32_t w[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int it = 0; it < 32 / ERI; ++it) {
      const int rr = it * ERI + lane / ECH, cc = lane % ECH;
      const uint4 val = *reinterpret_cast<const uint4*>(E + rr * EROW + cc * 16);
      const int64_t m = to.m0 + wm * WM + tm * 32 + rr;
      const int n = n0 + wn * WN + cc * 8;
      if (m < to.m_end) {
        uint16_t* const dst = p.c + m * p.ldc + n;
        if (vec16 && n + 7 < N) {
          *reinterpret_cast<uint4*>(dst) = val;
        } else {
          const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (n + i < N) dst[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
        }
      }
    }
  }
}

// ------------------------------------------------------------ FP8, direct to LDS
// A second FP8 kernel for dense launches with row-major B and K % 128 == 0
// (FPROP with the weight tile copy, DGRAD with its transposed copy, WGRAD with
// the columnwise copies).  It serves blockwise FP8 with power-of-two scales;
// MXFP8 takes its successor below, which loads whole cache lines.  The register-staged kernel above spends most of its
// time moving data: its 256x128 tile writes 48 KB into LDS per 128 of K from
// registers, and in a stage without loads and stores (a timing-only ablation)
// it already runs 36% faster, while without its MFMAs only 18% faster.  Here:
//  * the global loads write LDS themselves (buffer_load_dwordx4 ... lds: lane
//    l of a wave's load lands at the instruction's LDS base + 16 l; checked on
//    the chip), so there are no staging registers and no LDS store
//    instructions; out-of-range rows read zeros through the buffer range
//    check, as in the kernel above;
//  * that frees the registers for a 256x256 tile on 4 waves (one per SIMD),
//    each wave 128x128: 16 MFMAs per 64 of K against 8 fragment reads, so LDS
//    reads per MFMA halve and global bytes per MFMA halve against 256x128;
//  * stages of 64 K (32 KB: 256 A rows and 256 B rows of 64 bytes) in four
//    LDS buffers; the loads of stage s + 3 are issued while stage s is
//    computed, and one barrier per stage orders them: at the barrier of stage
//    s every wave has waited for its share of stage s + 1 and has finished
//    reading stage s - 1, whose buffer the next loads overwrite;
//  * fragments are read a stage ahead (two register sets): the reads of
//    stage s + 1 run under the MFMAs of stage s;
//  * the E8M0 scale words travel the same way: a stage pair's words (2 KB)
//    are loaded into LDS with its even stage and read once per pair.
// Measured when it still served MXFP8 (8192x24576x4096 FPROP, and DGRAD /
// WGRAD of the same layer): 1311 / 1140 / 1272 us for the kernel above,
// 963-989 / 815-845 / 854-885 us here.  Timing-only ablations of this kernel: without its loads
// 698 / 546 / 538 us, without its waits for them no faster (the prefetch
// hides the latency), every tile loading the same data 10% faster (little is
// bound by HBM), without its barriers 8% faster.
// A row's 64 bytes are four 16-byte chunks, chunk c in slot c ^ ((r >> 2) & 3):
// the fragment reads (16 consecutive rows, one chunk) then cover all 64 banks.
// A DMA instruction fills 16 consecutive rows; lane l takes row l / 4, slot
// l % 4 and so loads chunk (l % 4) ^ ((row >> 2) & 3) of that row.
// Each lane feeds its MFMAs the same K bytes and scale bytes as the kernel
// above (chunks h and 2 + h of a 64-wide slice), so both give the same bits.
constexpr int DMA_BM = 256, DMA_BN = 256;
constexpr int DMA_ROW = 64;                                 // LDS bytes per row and stage
constexpr int DMA_DATA = (DMA_BM + DMA_BN) * DMA_ROW;       // 32 KB of A and B rows
constexpr int DMA_SC = 2048;                                // a stage pair's scale words (A, then B)
constexpr int DMA_STAGE = DMA_DATA + DMA_SC;
constexpr int DMA_NBUF = 4;

typedef unsigned srd_t __attribute__((ext_vector_type(4)));   // a buffer descriptor in SGPRs

// A raw buffer descriptor as four scalar words (base, stride 0, size in
// bytes, the same flags as make_rsrc).
__device__ __forceinline__ srd_t make_srd(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return srd_t{(uint32_t)b, (uint32_t)(b >> 32) & 0xFFFFu, (uint32_t)bytes, 0x00020000u};
}

// Loads into LDS: lane l's 16 (or 4) bytes at voff land at LDS address
// m0 + 16 l (4 l).  Written as assembly so that the compiler, which cannot
// tell these LDS writes from the fragment reads of other buffers, does not
// wait for every load in flight before each LDS read; the kernel waits for
// them itself (wait_vmcnt), counting every vector-memory instruction it
// issues, and issues no other vector-memory loads in its main loop.
__device__ __forceinline__ void dma16(const srd_t& srd, uint32_t lds_addr, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(srd), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4(const srd_t& srd, uint32_t lds_addr, uint32_t voff) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(srd), "{m0}"(lds_addr) : "memory");
}
// The same with a wave-uniform byte offset soff added by the instruction
// (its SGPR offset), so that a per-stage offset costs no VALU add.  soff must
// keep every in-range lane inside its row; lanes whose voff is out of range
// (bit 31 set) stay out of range.
__device__ __forceinline__ void dma16s(const srd_t& srd, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(srd), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}
__device__ __forceinline__ void dma4s(const srd_t& srd, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(srd), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Blockwise FP8 (128-wide power-of-two blocks, linear scales): a row's one
// scale byte per stage pair, fetched with the aligned word holding it and
// replicated into all four bytes (both K slices and lane halves take it).
__global__ __launch_bounds__(256) void gemm_fp8_dma_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tiles_n = gridDim.x, tiles_m = gridDim.y;
  int mt, nt;
  // runs of 4 tile rows whatever the row length (FPROP 8192x24576x4096: 963
  // against 1038 us in row order; DGRAD and WGRAD shapes the same or better)
  if (!xcd_tile(tiles_m, tiles_n, p.N * p.K <= ((int64_t)4 << 20) ? 1 : 4, mt, nt)) return;
  const int K = (int)p.K, N = (int)p.N, M = (int)p.M;
  const int m0 = mt * DMA_BM, n0 = nt * DMA_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (the loads' LDS base)
  const int wm = w >> 1, wn = w & 1;                        // wave tile: rows wm*128, columns wn*128
  const int h = lane >> 5, r32 = lane & 31;
  const int nk = K / 64;
  const int nb128 = K >> 7;
  const uint32_t lbase = (uint32_t)reinterpret_cast<uintptr_t>(lds);

  const srd_t sA = make_srd(p.a, p.a_rows * p.lda);
  const srd_t sB = make_srd(p.b, p.N * p.ldb);
  const srd_t sAs = make_srd(p.a_scales, (p.a_rows * nb128 + 3) & ~int64_t(3));
  const srd_t sBs = make_srd(p.b_scales, (p.b_group_scales + 3) & ~int64_t(3));
  const uint32_t arb = (uint32_t)p.lda, brb = (uint32_t)p.ldb;

  // Data: wave w fills rows (4w + i) * 16 .. + 16 of A and of B.
  uint32_t a_dv[4], b_dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (4 * w + i) * 16 + (lane >> 2);
    const uint32_t c = (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
    const bool aok = m0 + r < M, bok = n0 + r < N;
    a_dv[i] = in_range(aok, (uint32_t)(aok ? m0 + r : 0) * arb + c * 16u);
    b_dv[i] = in_range(bok, (uint32_t)(bok ? n0 + r : 0) * brb + c * 16u);
  }
  // E8M0 scale words: the word of blocks 4q .. 4q + 3 of a row covers stage
  // pair q (stages 2q, 2q + 1).  A pair's words ride with its even stage:
  // entry E = 32 half + r (16 bytes) holds the words of rows 128 half + r +
  // 32 t, t = 0..3, so a lane reads its four tiles' words at once.  Wave w
  // loads A entries 16w .. 16w + 15 and B entries likewise (lane l: entry
  // 16w + l / 4, tile l % 4).
  uint32_t a_sv, b_sv;
  {
    const int E = 16 * w + (lane >> 2), t = lane & 3;
    const int r = (E >> 5) * 128 + (E & 31) + 32 * t;
    const bool aok = m0 + r < M, bok = n0 + r < N;
    const int n = n0 + r;
    // the byte of pair 0 (the load takes the aligned word of pair q's byte)
    a_sv = in_range(aok, aok ? (uint32_t)((m0 + r) * nb128) : 0u);
    b_sv = in_range(bok, bok ? (uint32_t)((p.b_tile ? (n >> 7) : n) * nb128) : 0u);
  }

  // stage s (in range or not) into buffer s % 4, with pair s / 2's scale
  // words when s is even; stages past the end read zeros, never computed
  // part i of stage s: A rows (i < 4) or B rows (i >= 4) of this wave
  auto dma_part = [&](int s, int i) {
    const uint32_t L = lbase + (uint32_t)((s & (DMA_NBUF - 1)) * DMA_STAGE);
    const uint32_t ko = s < nk ? (uint32_t)s * 64u : 0x80000000u;
    if (i < 4) dma16(sA, L + (uint32_t)((4 * w + i) * 1024), a_dv[i] + ko);
    else dma16(sB, L + (uint32_t)(DMA_BM * DMA_ROW + (4 * w + i - 4) * 1024), b_dv[i - 4] + ko);
  };
  auto dma_sc = [&](int s) {          // the scale words of pair s / 2 (s even)
    const uint32_t L = lbase + (uint32_t)((s & (DMA_NBUF - 1)) * DMA_STAGE);
    const int q = s >> 1;
    const bool qin = s < nk;
    dma4(sAs, L + DMA_DATA + (uint32_t)(w * 256), qin ? (a_sv + (uint32_t)q) & ~3u : 0x80000000u);
    dma4(sBs, L + DMA_DATA + 1024u + (uint32_t)(w * 256), qin ? (b_sv + (uint32_t)q) & ~3u : 0x80000000u);
  };
  auto dma = [&](int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma_part(s, i);
    if ((s & 1) == 0) dma_sc(s);
  };

  // fragment reads: tile t of A (rows wm*128 + 32t + r) and of B
  const int ra = wm * 128 + r32, rb = wn * 128 + r32;           // (r >> 2) & 3 is the same for r + 32t
  const uint32_t fa0 = (uint32_t)(ra * DMA_ROW + ((h ^ ((ra >> 2) & 3)) << 4));
  const uint32_t fa1 = (uint32_t)(ra * DMA_ROW + (((2 + h) ^ ((ra >> 2) & 3)) << 4));
  const uint32_t fb0 = (uint32_t)(DMA_BM * DMA_ROW + rb * DMA_ROW + ((h ^ ((rb >> 2) & 3)) << 4));
  const uint32_t fb1 = (uint32_t)(DMA_BM * DMA_ROW + rb * DMA_ROW + (((2 + h) ^ ((rb >> 2) & 3)) << 4));
  const uint32_t fsa = (uint32_t)(DMA_DATA + (wm * 32 + r32) * 16);
  const uint32_t fsb = (uint32_t)(DMA_DATA + 1024 + (wn * 32 + r32) * 16);
  v8i fa[2][4], fb[2][4];
  // part k of stage s's fragments: A tile k (k < 4) or B tile k - 4
  auto read_part = [&](int s, int set, int k) {
    const uint8_t* L = lds + (s & (DMA_NBUF - 1)) * DMA_STAGE;
    const int t = k & 3;
    const uint32_t o0 = k < 4 ? fa0 : fb0, o1 = k < 4 ? fa1 : fb1;
    const uint4 x0 = *reinterpret_cast<const uint4*>(L + o0 + t * 32 * DMA_ROW);
    const uint4 x1 = *reinterpret_cast<const uint4*>(L + o1 + t * 32 * DMA_ROW);
    const v8i v = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    if (k < 4) fa[set][t] = v;
    else fb[set][t] = v;
  };
  auto read = [&](int s, int set) {
#pragma unroll
    for (int k = 0; k < 8; ++k) read_part(s, set, k);
  };
  // a stage pair's scale bytes: the row's byte of the pair, in all four bytes
  struct Sc { uint32_t a[4], b[4]; };
  // byte position of pair 0's byte in its word, per tile row of the lane
  uint32_t a_b3[4], b_b3[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a_b3[t] = (uint32_t)((m0 + ra + 32 * t) * nb128) & 3u;
    b_b3[t] = (uint32_t)((p.b_tile ? ((n0 + rb + 32 * t) >> 7) : (n0 + rb + 32 * t)) * nb128) & 3u;
  }
  auto read_sc = [&](int s) {
    const uint8_t* L = lds + (s & (DMA_NBUF - 1)) * DMA_STAGE;
    const uint4 va = *reinterpret_cast<const uint4*>(L + fsa);
    const uint4 vb = *reinterpret_cast<const uint4*>(L + fsb);
    Sc v;
    const uint32_t q = (uint32_t)(s >> 1);
    const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v.a[t] = ((wa[t] >> (8 * ((a_b3[t] + q) & 3u))) & 0xFFu) * 0x01010101u;
      v.b[t] = ((wb[t] >> (8 * ((b_b3[t] + q) & 3u))) & 0xFFu) * 0x01010101u;
    }
    return v;
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Vector-memory instructions a lane issues: 8 per stage loaded, plus 2
  // scale loads with every even stage.  At the top of stage s the loads of
  // stage s + 1 (with its scales) must be done; issued after them: those of
  // stage s + 2, with scales when s + 2 is even: 10 after an even s, 8 after
  // an odd one.
  dma(0);
  dma(1);
  dma(2);
  wait_vmcnt<18>();                  // stage 0 and its scales landed (this lane's share)
  asm volatile("s_barrier" ::: "memory");
  read(0, 0);
  Sc cur = read_sc(0), nxt;

  // Two stages per iteration (K % 128 == 0: nk is even): stage 2j uses
  // fragment set 0 and scale byte 0 of pair j, stage 2j + 1 set 1 and byte 2.
  for (int s = 0; s < nk; s += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 0) wait_vmcnt<10>();  // stage s + u + 1 landed (this lane's share)
      else wait_vmcnt<8>();
      asm volatile("s_barrier" ::: "memory");
      // Each MFMA is followed by a slice of the other work, so that the
      // matrix pipe is fed while the LDS reads and the loads drain: after
      // MFMAs 0-7 two of the next stage's 16 fragment reads each, after MFMAs
      // 8-15 one of this wave's 8 loads of stage s + 3 (a wave that issued
      // them all at once stalled behind the full load queue before its first
      // MFMA).  Scheduling barriers keep this order.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tm = i >> 2, tn = i & 3;
        if (u == 0)
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[0][tn], fa[0][tm], acc[tm][tn], 0, 0, 0, (int)cur.b[tn], 0, (int)cur.a[tm]);
        else
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[1][tn], fa[1][tm], acc[tm][tn], 0, 0, 2, (int)cur.b[tn], 2, (int)cur.a[tm]);
        if (i < 8) {
          read_part(s + u + 1, u ^ 1, i);
          if (u == 1 && i == 7) nxt = read_sc(s + 2);
        } else {
          dma_part(s + u + 3, i - 8);
          if (u == 1 && i == 15) dma_sc(s + u + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
  }

  // ------------------------------------------------ epilogue (as in gemm_kernel)
  wait_vmcnt<0>();                     // no load still writing LDS
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int WN = 128;
  constexpr int EROW = WN * 2 + 8;
  constexpr int ECH = WN / 8;
  constexpr int ERI = 64 / ECH;
  uint8_t* const E = lds + w * (32 * EROW);
  const bool vec16 = ((p.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    uint8_t* const er = E + r32 * EROW + h * 8;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(er + (tn * 32 + g * 8) * 2) =
            make_uint2(f32x2_to_bf16x2(acc[tm][tn][4 * g], acc[tm][tn][4 * g + 1]),
                       f32x2_to_bf16x2(acc[tm][tn][4 * g + 2], acc[tm][tn][4 * g + 3]));
#pragma unroll
    for (int it = 0; it < 32 / ERI; ++it) {
      const int rr = it * ERI + lane / ECH, cc = lane % ECH;
      const uint4 val = *reinterpret_cast<const uint4*>(E + rr * EROW + cc * 16);
      const int64_t m = m0 + wm * 128 + tm * 32 + rr;
      const int n = n0 + wn * WN + cc * 8;
      if (m < M) {
        uint16_t* const dst = p.c + m * p.ldc + n;
        if (vec16 && n + 7 < N) {
          store_nt16(dst, val);
        } else {
          const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (n + i < N) dst[i] = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
        }
      }
    }
  }
}

static hipError_t launch_fp8_dma(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles_n = (a.N + DMA_BN - 1) / DMA_BN, tiles_m = (a.M + DMA_BM - 1) / DMA_BM;
  if (tiles_n * tiles_m >= (1ll << 31) || tiles_m > 65535) return hipErrorInvalidValue;
  const size_t lds = (size_t)DMA_NBUF * DMA_STAGE;
  static std::atomic<uint32_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit((const void*)gemm_fp8_dma_kernel, (int)lds, lds_set); e != hipSuccess)
    return e;
  hipLaunchKernelGGL(gemm_fp8_dma_kernel, dim3((unsigned)tiles_n, (unsigned)tiles_m), dim3(256), lds, st, a);
  return hipGetLastError();
}

// MXFP8 (32-wide E8M0 blocks) on whole cache lines.  The kernel above loads
// 64 bytes of each row per stage, half of a 128-byte line: its counters at
// 8192x24576x4096 showed the load path (texture addresser and L1) busy 84% of
// the time on one request per half line, a third of them for per-pair scale
// words.  This kernel loads stage pairs (128 K: a row's whole line) and the
// scale words in groups of four pairs:
//  * two pair buffers of 64 KB (rows of 128 bytes, chunk c of row r in slot
//    c ^ ((r >> 1) & 7), so the fragment reads of 16 consecutive rows cover
//    all banks); a DMA instruction fills 8 rows, lane l taking row l / 8 and
//    slot l % 8;
//  * pair P + 2's loads are issued during stage 2P + 1 (one after each
//    MFMA) into the buffer pair P has left; at the top of every odd stage the
//    wave waits for all its loads and the workgroup meets at a barrier (pair
//    P + 1 landed, pair P's buffer free): one barrier per pair;
//  * scale words: a two-slot ring of 8 KB groups, group g (pairs 4g .. 4g + 3)
//    as [row][pair] words, A's 256 rows then B's.  Lane l of a group load
//    takes the word of pair l % 4 of row 16 k + l / 4 (k: the load's part),
//    so a row's four words (16 contiguous bytes in the linear and tile
//    layouts) are one request.  Part p of group g rides with odd stage
//    8g - 9 + 2p: after the last read of group g - 2 in the same slot (pair
//    4g - 5, read in stage 8g - 11) and before the first read of group g
//    (pair 4g, read in stage 8g - 1).
// Each lane feeds its MFMAs the same K bytes and scale bytes as the kernels
// above, so all give the same bits.
constexpr int FP8P_ROW = 128;                                // LDS bytes per row and stage pair
constexpr int FP8P_DATA = (DMA_BM + DMA_BN) * FP8P_ROW;      // 64 KB of A and B rows
constexpr int FP8P_SG = 2 * FP8P_DATA;                       // the scale-group ring
constexpr int FP8P_SGS = 8192;                               // one group: 256 A rows, 256 B rows, 16 bytes each
constexpr int FP8P_LDS = FP8P_SG + 2 * FP8P_SGS;             // 144 KB

__global__ __launch_bounds__(256) void gemm_fp8_pair_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tiles_n = gridDim.x, tiles_m = gridDim.y;
  int mt, nt;
  if (!xcd_tile(tiles_m, tiles_n, p.N * p.K <= ((int64_t)4 << 20) ? 1 : 4, mt, nt)) return;
  const int K = (int)p.K, N = (int)p.N, M = (int)p.M;
  const int m0 = mt * DMA_BM, n0 = nt * DMA_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (the loads' LDS base)
  const int wm = w >> 1, wn = w & 1;                        // wave tile: rows wm*128, columns wn*128
  const int h = lane >> 5, r32 = lane & 31;
  const int np = K / 128;                                   // stage pairs
  const int nb32 = K >> 5;
  const uint32_t lbase = (uint32_t)reinterpret_cast<uintptr_t>(lds);

  const srd_t sA = make_srd(p.a, p.a_rows * p.lda);
  const srd_t sB = make_srd(p.b, p.N * p.ldb);
  const srd_t sAs = make_srd(p.a_scales, p.a_rows * nb32);
  const srd_t sBs = make_srd(p.b_scales, p.b_group_scales);
  const uint32_t arb = (uint32_t)p.lda, brb = (uint32_t)p.ldb;

  // Data: wave w fills rows 64 w + 8 i .. + 8 of A and of B (i = 0..7)
  uint32_t a_dv[8], b_dv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 64 * w + 8 * i + (lane >> 3);
    const uint32_t c = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    const bool aok = m0 + r < M, bok = n0 + r < N;
    a_dv[i] = in_range(aok, (uint32_t)(aok ? m0 + r : 0) * arb + c * 16u);
    b_dv[i] = in_range(bok, (uint32_t)(bok ? n0 + r : 0) * brb + c * 16u);
  }
  // Scale groups.  Part k's rows lie 16 k below part 0's: a wave-uniform
  // step in every layout, added through the instruction's SGPR offset; a
  // lane's rows past the operand's end are marked in a 4-bit mask.
  const uint32_t a_sstep = p.a_mfma_layout ? 128u : 4u;      // a word's step per pair
  const uint32_t b_sstep = (p.b_tile || !p.b_mfma_layout) ? 4u : 128u;
  uint32_t a_gv, b_gv, a_gm = 0, b_gm = 0;
  {
    const int R = 64 * w + (lane >> 2), q = lane & 3;
    const int n = n0 + R;
    a_gv = (uint32_t)scale_offset(m0 + R, 0, nb32, p.a_mfma_layout) + (uint32_t)q * a_sstep;
    b_gv = (p.b_tile ? (uint32_t)((n >> 5) * nb32) : (uint32_t)scale_offset(n, 0, nb32, p.b_mfma_layout)) +
           (uint32_t)q * b_sstep;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a_gm |= (uint32_t)(m0 + R + 16 * k >= M) << k;
      b_gm |= (uint32_t)(n + 16 * k >= N) << k;
    }
  }
  // part k's step from part 0: (k / 2) 32-row chunks, plus 16 rows when k is odd
  const uint32_t a_g2 = p.a_mfma_layout ? (uint32_t)(nb32 >> 2) * 128u : (uint32_t)(32 * nb32);
  const uint32_t a_g1 = p.a_mfma_layout ? 64u : (uint32_t)(16 * nb32);
  const uint32_t b_g2 = p.b_tile ? (uint32_t)nb32 : p.b_mfma_layout ? (uint32_t)(nb32 >> 2) * 128u : (uint32_t)(32 * nb32);
  const uint32_t b_g1 = p.b_tile ? 0u : p.b_mfma_layout ? 64u : (uint32_t)(16 * nb32);

  // load i (0..15) of pair P: A rows (i < 8) or B rows of this wave.  The
  // pair's K offset rides in the SGPR offset (it keeps every lane inside its
  // row); pairs past the end load through descriptors of zero size.
  srd_t cA = sA, cB = sB;
  auto dma_part = [&](int P, int i) {
    const uint32_t L = lbase + (uint32_t)((P & 1) * FP8P_DATA);
    const bool pin = P < np;
    if (i == 0) {
      cA[2] = pin ? sA[2] : 0u;
      cB[2] = pin ? sB[2] : 0u;
    }
    const uint32_t ko = pin ? (uint32_t)P * 128u : 0u;
    if (i < 8) dma16s(cA, L + (uint32_t)((64 * w + 8 * i) * FP8P_ROW), a_dv[i], ko);
    else dma16s(cB, L + (uint32_t)(DMA_BM * FP8P_ROW + (64 * w + 8 * (i - 8)) * FP8P_ROW), b_dv[i - 8], ko);
  };
  // part k of scale group G: this wave's A and B words of rows 64 w + 16 k + (0..15)
  auto dma_grp = [&](int G, int k) {
    const uint32_t L = lbase + FP8P_SG + (uint32_t)((G & 1) * FP8P_SGS + (64 * w + 16 * k) * 16);
    const bool gin = 4 * G < np;
    srd_t gA = sAs, gB = sBs;
    gA[2] = gin ? sAs[2] : 0u;
    gB[2] = gin ? sBs[2] : 0u;
    // lanes of pairs past the last (a partial last group) load nothing either:
    // the SGPR offset escapes the range check, so every in-range lane's whole
    // address must lie inside the operand's scales
    const uint32_t pk = (uint32_t)(4 * G + (lane & 3) >= np) << 31;
    const uint32_t av = a_gv | (((a_gm >> k) & 1u) << 31) | pk, bv = b_gv | (((b_gm >> k) & 1u) << 31) | pk;
    const uint32_t ak = (uint32_t)(k >> 1) * a_g2 + (uint32_t)(k & 1) * a_g1;
    const uint32_t bk = (uint32_t)(k >> 1) * b_g2 + (uint32_t)(k & 1) * b_g1;
    dma4s(gA, L, av, gin ? (uint32_t)(4 * G) * a_sstep + ak : 0u);
    dma4s(gB, L + 4096u, bv, gin ? (uint32_t)(4 * G) * b_sstep + bk : 0u);
  };

  // fragment reads: tile t of A (rows wm*128 + 32t + r) and of B, stage e of
  // a pair: chunks 4e + h and 4e + 2 + h ((r >> 1) & 7 is the same for r + 32t)
  const int ra = wm * 128 + r32, rb = wn * 128 + r32;
  const uint32_t swa = (uint32_t)((ra >> 1) & 7), swb = (uint32_t)((rb >> 1) & 7);
  const uint32_t cra = (uint32_t)(ra * FP8P_ROW), crb = (uint32_t)(DMA_BM * FP8P_ROW + rb * FP8P_ROW);
  v8i fa[2][4], fb[2][4];
  // part k of stage e of pair P's fragments: A tile k (k < 4) or B tile k - 4
  auto read_part = [&](int P, int e, int set, int k) {
    const uint8_t* L = lds + (P & 1) * FP8P_DATA;
    const int t = k & 3;
    const uint32_t base = (k < 4 ? cra : crb) + (uint32_t)(t * 32 * FP8P_ROW);
    const uint32_t sw = k < 4 ? swa : swb;
    const uint4 x0 = *reinterpret_cast<const uint4*>(L + base + (((uint32_t)(4 * e + h) ^ sw) << 4));
    const uint4 x1 = *reinterpret_cast<const uint4*>(L + base + (((uint32_t)(4 * e + 2 + h) ^ sw) << 4));
    const v8i v = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    if (k < 4) fa[set][t] = v;
    else fb[set][t] = v;
  };
  // pair P's scale words (lane half h: its block's byte to byte 0/2)
  struct Sc { uint32_t a[4], b[4]; };
  auto read_sc = [&](int P) {
    const uint8_t* G = lds + FP8P_SG + ((P >> 2) & 1) * FP8P_SGS + (P & 3) * 4;
    Sc v;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v.a[t] = *reinterpret_cast<const uint32_t*>(G + (ra + 32 * t) * 16) >> (8 * h);
      v.b[t] = *reinterpret_cast<const uint32_t*>(G + 4096 + (rb + 32 * t) * 16) >> (8 * h);
    }
    return v;
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Prologue: pair 0, scale group 0, part 0 of group 1, pair 1.  Then wait
  // for pair 0 and group 0 (18 loads of this lane issued after them).
#pragma unroll
  for (int i = 0; i < 16; ++i) dma_part(0, i);
#pragma unroll
  for (int k = 0; k < 4; ++k) dma_grp(0, k);
  dma_grp(1, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) dma_part(1, i);
  wait_vmcnt<18>();
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int k = 0; k < 8; ++k) read_part(0, 0, 0, k);
  Sc cur = read_sc(0), nxt;

  for (int P = 0; P < np; ++P) {
    // stage 2P: fragment set 0, scale bytes 0; the reads of stage 2P + 1
    // (same pair) after the first eight MFMAs, two each
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tm = i >> 2, tn = i & 3;
      acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fb[0][tn], fa[0][tm], acc[tm][tn], 0, 0, 0, (int)cur.b[tn], 0, (int)cur.a[tm]);
      if (i < 8) read_part(P, 1, 1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage 2P + 1: every load of this wave landed (pair P + 1 and the scale
    // parts issued with it), and every wave is done with pair P's buffer
    wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tm = i >> 2, tn = i & 3;
      acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fb[1][tn], fa[1][tm], acc[tm][tn], 0, 0, 2, (int)cur.b[tn], 2, (int)cur.a[tm]);
      if (i < 8) read_part(P + 1, 0, 0, i);
      if (i == 7) nxt = read_sc(P + 1);
      dma_part(P + 2, i);
      if (i == 15) dma_grp((P + 5) >> 2, (P + 5) & 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    cur = nxt;
  }

  // ------------------------------------------------ epilogue (as in gemm_kernel)
  wait_vmcnt<0>();                     // no load still writing LDS
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int WN = 128;
  constexpr int EROW = WN * 2 + 8;
  constexpr int ECH = WN / 8;
  constexpr int ERI = 64 / ECH;
  uint8_t* const E = lds + w * (32 * EROW);
  const bool vec16 = ((p.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    uint8_t* const er = E + r32 * EROW + h * 8;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(er + (tn * 32 + g * 8) * 2) =
            make_uint2(f32x2_to_bf16x2(acc[tm][tn][4 * g], acc[tm][tn][4 * g + 1]),
                       f32x2_to_bf16x2(acc[tm][tn][4 * g + 2], acc[tm][tn][4 * g + 3]));
#pragma unroll
    for (int it = 0; it < 32 / ERI; ++it) {
      const int rr = it * ERI + lane / ECH, cc = lane % ECH;
      const uint4 val = *reinterpret_cast<const uint4*>(E + rr * EROW + cc * 16);
      const int64_t m = m0 + wm * 128 + tm * 32 + rr;
      const int n = n0 + wn * WN + cc * 8;
      if (m < M) {
        uint16_t* const dst = p.c + m * p.ldc + n;
        if (vec16 && n + 7 < N) {
          store_nt16(dst, val);
        } else {
          const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (n + i < N) dst[i] = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
        }
      }
    }
  }
}

static hipError_t launch_fp8_pair(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles_n = (a.N + DMA_BN - 1) / DMA_BN, tiles_m = (a.M + DMA_BM - 1) / DMA_BM;
  if (tiles_n * tiles_m >= (1ll << 31) || tiles_m > 65535) return hipErrorInvalidValue;
  static std::atomic<uint32_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit((const void*)gemm_fp8_pair_kernel, FP8P_LDS, lds_set); e != hipSuccess)
    return e;
  hipLaunchKernelGGL(gemm_fp8_pair_kernel, dim3((unsigned)tiles_n, (unsigned)tiles_m), dim3(256), FP8P_LDS, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ NVFP4, direct to LDS
// The NVFP4 counterpart of the FP8 direct-to-LDS kernels above, for dense
// launches with row-major B and K % 128 == 0 (FPROP with the 16x16 weight
// copy, DGRAD with its transposed copy, WGRAD with the columnwise copies).
// LDS holds the operands as they are stored, FP4 codes and E4M3 scale bytes,
// loaded straight into it; each wave converts the fragments it feeds its
// MFMAs (hardware FP4 -> FP16 with unit scale, times the block scale: exact,
// as in the register-staged kernel).  Its stages load half lines (64 code
// bytes of a row), like the first FP8 kernel: with four times the MFMA work
// per loaded byte of FP8, its load path is 25-36% busy at the config-5
// shapes, not its bound.
// Against staging FP16 tiles through LDS this moves a quarter of the LDS
// bytes and drops the LDS store instructions, at the cost of converting each
// A and B value twice (the two waves that share a row or column of tiles).
//  * 256x256 tile on 4 waves (one per SIMD), each 128x128: per 16 of K,
//    16 MFMAs (v_mfma_f32_32x32x16_f16) and 8 fragment conversions.
//  * Stages of 128 K: 256 A rows and 256 B rows of 64 code bytes (chunk c of
//    a row in slot c ^ ((r >> 2) & 3), as in the first FP8 kernel), then the
//    rows' scale words (two per row and stage: blocks 8s .. 8s + 3 and
//    8s + 4 .. 8s + 7), in four LDS buffers of 36 KB; the loads of stage
//    s + 3 are issued while stage s computes; one barrier per stage.
//  * A lane (row r, K half h) reads, per 64 K, the 16 code bytes of K
//    [32h, 32h + 32) of its row for each of its 8 tiles, a 64-K step ahead;
//    K step ks (16 K) takes codes [32h + 8ks, +8) (one word), the order every
//    16-bit path uses, so the bits equal the other tiles'.  Conversions run a
//    K step ahead of the MFMAs.
// Scale words in LDS: entry E = 32 half + r (32 bytes) holds, for tiles
// t = 0..3 (rows 128 half + r + 32t), the stage's two words of each.
constexpr int NVD_ROW = 64;                                // code bytes per row and stage (128 K)
constexpr int NVD_DATA = (DMA_BM + DMA_BN) * NVD_ROW;      // 32 KB
constexpr int NVD_SC = (DMA_BM + DMA_BN) * 8;              // 4 KB of scale words
constexpr int NVD_STAGE = NVD_DATA + NVD_SC;
constexpr int NVD_NBUF = 4;

// NW = 4: waves 2x2, each 128x128 (one wave per SIMD); NW = 8: waves 2x4,
// each 128x64 (two per SIMD, so one wave's conversions and loads can issue
// while the other's MFMAs run, at 6 conversions per 8 MFMAs instead of 8 per
// 16).  GRP: grouped (MoE) launches, tiles placed as in gemm_kernel, A rows
// gathered through the row index, B and its scales and S per group.  SWI:
// the gate_up GEMM with SwiGLU in the epilogue (as in gemm_kernel: each
// wave's WN logical columns read WN/2 gate rows and the matching up rows).
template <int NW, bool GRP = false, bool SWI = false>
__global__ __launch_bounds__(64 * NW) void gemm_nvfp4_dma_kernel(GemmArgs p) {
  constexpr int WGN = NW / 2;                               // waves across N
  constexpr int WN = DMA_BN / WGN;                          // 128 or 64 columns per wave
  constexpr int TM = 4, TN = WN / 32;                       // 32x32 tiles per wave
  constexpr int NF = TM + TN;                               // fragments per K step
  constexpr int CI = 16 / NW;                               // 1 KB code loads per operand and wave
  constexpr int SI = 8 / NW;                                // scale-word loads per operand and wave
  constexpr int NV = 2 * CI + 2 * SI;                       // vector-memory instructions per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int tiles_n = gridDim.x;
  const int tiles_m = GRP ? group_mtiles<DMA_BM>(p, lane) : (int)gridDim.y;
  int mt, nt;
  if (!xcd_tile(tiles_m, tiles_n, (GRP || (p.N * p.K / 2) <= ((int64_t)4 << 20)) ? 1 : 4, mt, nt)) return;
  const TileOrigin to = tile_origin<DMA_BM>(p, mt, lane);
  if (!to.active) return;
  const int K = (int)p.K, N = (int)p.N;
  const int m0 = (int)to.m0, m_end = (int)to.m_end, grp = to.group;
  const int n0 = nt * DMA_BN;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WGN, wn = w % WGN;
  // A row behind output row m, B row behind logical column n
  auto arow = [&](int m) -> int { return p.row_index ? p.row_index[m] : m; };
  auto brow = [&](int n) -> int {
    if constexpr (SWI) {
      constexpr int P = WN / 2;
      const int q = n / (2 * P), j = n - q * (2 * P);
      return j < P ? q * P + j : (int)p.swiglu_inter + q * P + (j - P);
    }
    return n;
  };
  const int h = lane >> 5, r32 = lane & 31;
  const int nk = K / 128;
  const int nb16 = K >> 4;
  const uint32_t lbase = (uint32_t)reinterpret_cast<uintptr_t>(lds);

  const uint32_t arb = (uint32_t)(p.lda >> 1), brb = (uint32_t)(p.ldb >> 1);   // code bytes per row
  const uint8_t* bbase = p.b + (int64_t)grp * (p.b_group_elems >> 1);
  const uint8_t* bsbase = p.b_scales + (int64_t)grp * p.b_group_scales;
  const srd_t sA = make_srd(p.a, p.a_rows * (int64_t)arb);
  const srd_t sB = make_srd(bbase, p.N * (int64_t)brb);
  const srd_t sAs = make_srd(p.a_scales, p.a_rows * nb16);
  const srd_t sBs = make_srd(bsbase, p.b_group_scales);

  // codes: wave w fills rows (CI w + i) * 16 .. + 16 of A and of B
  uint32_t a_dv[CI], b_dv[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    const int r = (CI * w + i) * 16 + (lane >> 2);
    const uint32_t c = (uint32_t)((lane & 3) ^ ((r >> 2) & 3));
    const bool aok = m0 + r < m_end, bok = n0 + r < N;
    a_dv[i] = in_range(aok, (uint32_t)(aok ? arow(m0 + r) : 0) * arb + c * 16u);
    b_dv[i] = in_range(bok, (uint32_t)(bok ? brow(n0 + r) : 0) * brb + c * 16u);
  }
  // scale words: entry E (32 bytes) = 32 half + r holds, for tiles t = 0..3
  // (rows 128 half + r + 32t), the stage's two words; wave w loads entries
  // 8 (SI w + i) .. + 8 of A and of B; lane l: entry + l / 8, tile (l % 8) / 2,
  // word l % 2
  uint32_t a_sv[SI], b_sv[SI];
#pragma unroll
  for (int i = 0; i < SI; ++i) {
    const int E = 8 * (SI * w + i) + (lane >> 3), t = (lane & 7) >> 1, sub = lane & 1;
    const int r = (E >> 5) * 128 + (E & 31) + 32 * t;
    const bool aok = m0 + r < m_end, bok = n0 + r < N;
    a_sv[i] = in_range(aok, aok ? (uint32_t)scale_offset(arow(m0 + r), 4 * sub, nb16, p.a_mfma_layout) : 0u);
    const int n = bok ? brow(n0 + r) : 0;
    b_sv[i] = in_range(bok, bok ? (p.b_tile ? (uint32_t)((n >> 4) * nb16 + 4 * sub)
                                            : (uint32_t)scale_offset(n, 4 * sub, nb16, p.b_mfma_layout))
                                : 0u);
  }
  const uint32_t a_sst = p.a_mfma_layout ? 256u : 8u;
  const uint32_t b_sst = (p.b_tile || !p.b_mfma_layout) ? 8u : 256u;

  // part i of stage s: A code rows (i < CI), B code rows, A scale words, B
  // scale words.  The stage's K offset rides in the instruction's SGPR
  // offset; a stage past the end loads through descriptors of zero size
  // (zeros, no memory traffic).  Part 0 of a stage comes first.
  srd_t cA = sA, cB = sB, cAs = sAs, cBs = sBs;
  auto dma_part = [&](int s, int i) {
    const uint32_t L = lbase + (uint32_t)((s & (NVD_NBUF - 1)) * NVD_STAGE);
    const bool sin = s < nk;
    if (i == 0) {
      // the descriptors' sizes: zero from the first stage past the end
      cA[2] = sin ? sA[2] : 0u;
      cB[2] = sin ? sB[2] : 0u;
      cAs[2] = sin ? sAs[2] : 0u;
      cBs[2] = sin ? sBs[2] : 0u;
    }
    const uint32_t ko = sin ? (uint32_t)s * 64u : 0u;
    if (i < CI) {
      dma16s(cA, L + (uint32_t)((CI * w + i) * 1024), a_dv[i], ko);
    } else if (i < 2 * CI) {
      const int j = i - CI;
      dma16s(cB, L + (uint32_t)(DMA_BM * NVD_ROW + (CI * w + j) * 1024), b_dv[j], ko);
    } else if (i < 2 * CI + SI) {
      const int j = i - 2 * CI;
      dma4s(cAs, L + NVD_DATA + (uint32_t)((8 * (SI * w + j)) * 32), a_sv[j], sin ? (uint32_t)s * a_sst : 0u);
    } else {
      const int j = i - 2 * CI - SI;
      dma4s(cBs, L + NVD_DATA + 2048u + (uint32_t)((8 * (SI * w + j)) * 32), b_sv[j],
            sin ? (uint32_t)s * b_sst : 0u);
    }
  };
  auto dma = [&](int s) {
#pragma unroll
    for (int i = 0; i < NV; ++i) dma_part(s, i);
  };

  // Raw code chunks: 16 bytes of K [32h, 32h + 32) of one 64-K half of a
  // stage, for the wave's A tiles (f < TM) and B tiles (f >= TM).  One set:
  // each half is read right after the conversions of the previous one are
  // issued.
  const int ra = wm * 128 + r32, rb = wn * WN + r32;
  const uint32_t cra = (uint32_t)(ra * NVD_ROW), crb = (uint32_t)(DMA_BM * NVD_ROW + rb * NVD_ROW);
  const uint32_t swa = (uint32_t)((ra >> 2) & 3), swb = (uint32_t)((rb >> 2) & 3);
  uint4 raw[NF];
  auto read_raw = [&](int s, int half, int f) {
    const uint8_t* L = lds + (s & (NVD_NBUF - 1)) * NVD_STAGE;
    const uint32_t c = (uint32_t)(2 * half + h);
    const uint32_t o = f < TM ? cra + (uint32_t)(f * 32 * NVD_ROW) + ((c ^ swa) << 4)
                              : crb + (uint32_t)((f - TM) * 32 * NVD_ROW) + ((c ^ swb) << 4);
    raw[f] = *reinterpret_cast<const uint4*>(L + o);
  };
  // block scales of a stage as FP16 pairs: per fragment and 64-K half, the
  // lane's two blocks (K [32h, 32h + 16) and [32h + 16, 32h + 32)) (exact:
  // E4M3 values are FP16 normals).  The stage's scale words are read into scw
  // and converted per fragment (cvt_sc).
  h2 sc[NF][2];
  uint32_t scw[NF][2];
  auto read_scw = [&](int s) {
    const uint8_t* L = lds + (s & (NVD_NBUF - 1)) * NVD_STAGE + NVD_DATA;
    const uint4* ea = reinterpret_cast<const uint4*>(L + (wm * 32 + r32) * 32);
    const uint4 a0 = ea[0], a1 = ea[1];
    scw[0][0] = a0.x; scw[0][1] = a0.y; scw[1][0] = a0.z; scw[1][1] = a0.w;
    scw[2][0] = a1.x; scw[2][1] = a1.y; scw[3][0] = a1.z; scw[3][1] = a1.w;
    // B: rows wn WN + r + 32t lie in half (wn WN) / 128, tiles from (wn WN % 128) / 32
    const int eb = ((wn * WN) >> 7) * 32 + r32, tb = ((wn * WN) & 127) >> 5;
    const uint4* pb = reinterpret_cast<const uint4*>(L + 2048 + eb * 32 + tb * 8);
    const uint4 b0 = pb[0];
    scw[TM][0] = b0.x; scw[TM][1] = b0.y; scw[TM + 1][0] = b0.z; scw[TM + 1][1] = b0.w;
    if constexpr (TN == 4) {
      const uint4 b1 = pb[1];
      scw[TM + 2][0] = b1.x; scw[TM + 2][1] = b1.y; scw[TM + 3][0] = b1.z; scw[TM + 3][1] = b1.w;
    }
  };
  // the lane's two bytes of each word (lane half h) moved to the low half
  auto shift_scw = [&](int f) {
    const uint32_t sh = 16u * (uint32_t)h;
    scw[f][0] >>= sh;
    scw[f][1] >>= sh;
  };
  auto cvt_sc = [&](int f, int hf) { sc[f][hf] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scw[f][hf], 1.0f, false); };
  auto read_sc = [&](int s) {
    read_scw(s);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      shift_scw(f);
      cvt_sc(f, 0);
      cvt_sc(f, 1);
    }
  };
  // FP16 operands of one K step, two sets (packed FP16 pairs)
  uint4 cv[2][NF];
  // part 0: values 0..3 of the lane's 8 (code bytes 0, 1), part 1: values 4..7
  auto convert_part = [&](const uint4& r, h2 s01, int ks, int part, uint4& dst) {
    const h2 sp = (ks >> 1) ? h2{s01.y, s01.y} : h2{s01.x, s01.x};
    const uint32_t word = ks == 0 ? r.x : ks == 1 ? r.y : ks == 2 ? r.z : r.w;
    if (part == 0) {
      dst.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sp);
      dst.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sp);
    } else {
      dst.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sp);
      dst.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sp);
    }
  };
  auto convert = [&](const uint4& r, h2 s01, int ks, uint4& dst) {
    convert_part(r, s01, ks, 0, dst);
    convert_part(r, s01, ks, 1, dst);
  };
  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mfma = [&](int set, int tm, int tn) {
    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, cv[set][TM + tn]),
                                                         __builtin_bit_cast(v8h, cv[set][tm]), acc[tm][tn], 0, 0, 0);
  };

  // Vector-memory instructions per lane and stage: NV.  At the top of stage
  // s the loads of stage s + 1 must be done; issued after them: stage s + 2's.
  dma(0);
  dma(1);
  dma(2);
  wait_vmcnt<2 * NV>();
  asm volatile("s_barrier" ::: "memory");
  read_sc(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) read_raw(0, 0, f);
#pragma unroll
  for (int f = 0; f < NF; ++f) convert(raw[f], sc[f][0], 0, cv[0][f]);

  constexpr int NM = TM * TN;
  static_assert(NV <= NM, "slots");
  for (int s = 0; s < nk; ++s) {
    wait_vmcnt<NV>();                                      // stage s + 1 landed (this lane's share)
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int set = kk & 1;
      const int nkk = (kk + 1) & 7;                        // next K step (of this stage or the next)
      const int nhalf = nkk >> 2, nks = nkk & 3;
      // After MFMA i of a K step: the half conversions j = i, i + NM, ... of
      // the next K step (half j: part j % 2 of fragment j / 2; two
      // conversions and two multiplies, four VALU instructions, about what
      // one 32-cycle MFMA hides; 4 waves: one half per MFMA, 8 waves: one or
      // two).  In K step 2 the raw read of fragment f of this stage's second
      // half right after its last half conversion from the first half; in K
      // steps 4 and 5 the loads of stage s + 3, half in each; in K step 6
      // the scale words of the next stage (after MFMA 0, shifted into place
      // after MFMAs 4, 5, ...) and the raw reads of its first half, placed
      // as in K step 2; in K step 7 each fragment's two block scales are
      // converted, one before each of its half conversions.
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        mfma(set, i / TN, i % TN);
#pragma unroll
        for (int j = i; j < 2 * NF; j += NM) {
          const int f = j >> 1, part = j & 1;
          if (kk == 7) cvt_sc(f, part);
          convert_part(raw[f], sc[f][nhalf], nks, part, cv[set ^ 1][f]);
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          // slot of fragment f's second half; its raw chunk is reread after it
          const int last = (2 * f + 1) % NM;
          if (last + 1 == i || (last == NM - 1 && i == NM - 1)) {
            if (kk == 2) read_raw(s, 1, f);
            if (kk == 6) read_raw(s + 1, 0, f);
          }
        }
        if (kk == 4 && i < NV / 2) dma_part(s + 3, i);
        if (kk == 5 && i < NV - NV / 2) dma_part(s + 3, NV / 2 + i);
        if (kk == 6 && i == 0) read_scw(s + 1);
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (kk == 6 && (4 + f < NM ? 4 + f : NM - 1) == i) shift_scw(f);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ------------------------------------------------ epilogue (as in gemm_kernel)
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int EROW = WN * 2 + 8;
  constexpr int ECH = WN / 8;
  constexpr int ERI = 64 / ECH;
  uint8_t* const E = lds + w * (32 * EROW);
  const bool vec16 = ((p.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 15) == 0);
  const float sbg = p.b_gs[grp];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int mrow = m0 + wm * 128 + tm * 32 + r32;
    const float sa = mrow < m_end ? (p.a_gs_per_row ? p.a_gs[arow(mrow)] : p.a_gs[0]) : 0.0f;
    uint8_t* const er = E + r32 * EROW + h * 8;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (acc[tm][tn][4 * g + i] * sa) * sbg;
        *reinterpret_cast<uint2*>(er + (tn * 32 + g * 8) * 2) =
            make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
      }
    if constexpr (SWI) {
      // gate chunk cc and up chunk cc + ECH / 2 of a staged row -> 8 values of H
      constexpr int ECH2 = ECH / 2, ERI2 = 64 / ECH2;
      const bool wave_in = n0 + wn * WN < N;
#pragma unroll
      for (int it = 0; it < 32 / ERI2; ++it) {
        const int rr = it * ERI2 + lane / ECH2, cc = lane % ECH2;
        const uint4 gv = *reinterpret_cast<const uint4*>(E + rr * EROW + cc * 16);
        const uint4 uv = *reinterpret_cast<const uint4*>(E + rr * EROW + (cc + ECH2) * 16);
        const int64_t m = m0 + wm * 128 + tm * 32 + rr;
        const int hc = ((n0 + wn * WN) >> 1) + cc * 8;
        if (wave_in && m < m_end) {
          const uint4 hv = make_uint4(swiglu_bf16x2(gv.x, uv.x), swiglu_bf16x2(gv.y, uv.y),
                                      swiglu_bf16x2(gv.z, uv.z), swiglu_bf16x2(gv.w, uv.w));
          uint16_t* const dst = p.c + m * p.ldc + hc;
          if (vec16) {
            store_nt16(dst, hv);
          } else {
            const uint32_t wv[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int it = 0; it < 32 / ERI; ++it) {
      const int rr = it * ERI + lane / ECH, cc = lane % ECH;
      const uint4 val = *reinterpret_cast<const uint4*>(E + rr * EROW + cc * 16);
      const int64_t m = m0 + wm * 128 + tm * 32 + rr;
      const int n = n0 + wn * WN + cc * 8;
      if (m < m_end) {
        uint16_t* const dst = p.c + m * p.ldc + n;
        if (vec16 && n + 7 < N) {
          store_nt16(dst, val);
        } else {
          const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (n + i < N) dst[i] = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
        }
      }
    }
  }
}

template <int NW, bool GRP = false, bool SWI = false>
static hipError_t launch_nvfp4_dma(const GemmArgs& a, hipStream_t st) {
  const int64_t tiles_n = (a.N + DMA_BN - 1) / DMA_BN;
  int64_t tiles_m = GRP ? a.M / DMA_BM + a.num_groups : (a.M + DMA_BM - 1) / DMA_BM;
  if (tiles_m < 1) tiles_m = 1;
  if (tiles_n * tiles_m >= (1ll << 31) || tiles_m > 65535) return hipErrorInvalidValue;
  const size_t lds = (size_t)NVD_NBUF * NVD_STAGE;
  auto kern = gemm_nvfp4_dma_kernel<NW, GRP, SWI>;
  static std::atomic<uint32_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit((const void*)kern, (int)lds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles_n, (unsigned)tiles_m), dim3(64 * NW), lds, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ launcher
template <int PATH, int BM, int BN, bool BT, int DIST, int WGM, int WGN, bool PP = false, bool SWI = false>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st);

template <int PATH, int BM, int BN, bool BT, int DIST, int WGM, int WGN, bool PP, bool SDW, bool BD = false,
          bool B128 = false, bool SWI = false>
static hipError_t launch_k(const GemmArgs& a, hipStream_t st) {
  int64_t tiles_n = (a.N + BN - 1) / BN;
  int64_t tiles_m = a.num_groups == 0 ? (a.M + BM - 1) / BM : a.M / BM + a.num_groups;
  if (tiles_m < 1) tiles_m = 1;
  if (tiles_n * tiles_m >= (1ll << 31) || tiles_m > 65535) return hipErrorInvalidValue;
  size_t lds = 2 * (size_t)stages_per_barrier<PATH, BT, DIST, PP>() * (BM + (BD ? 0 : BN)) * LDS_ROW;
  auto kern = gemm_kernel<PATH, BM, BN, BT, DIST, WGM, WGN, PP, SDW, BD, B128, SWI>;
  static std::atomic<uint32_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit((const void*)kern, (int)lds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles_n, (unsigned)tiles_m), dim3(64 * WGM * WGN), lds, st, a);
  return hipGetLastError();
}

// B direct (see gemm_kernel): NVFP4 only.  For BF16 it measured slower
// (4096x2048x768: 34 us against 20 us through LDS; its B needs four 16-byte
// loads per lane and stage and BF16 is bound by LDS, not by the conversion).
static constexpr bool gemm_b_direct() { return true; }

template <int PATH, int BM, int BN, bool BT, int DIST, int WGM, int WGN, bool PP, bool SWI>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  if constexpr (SWI) {
    // NVFP4, row-major B (the gate_up weight), K % 64 == 0 (checked on the host)
    if constexpr (!PP && DIST == 2)
      if (gemm_b_direct()) return launch_k<PATH, BM, BN, BT, DIST, WGM, WGN, PP, true, true, false, true>(a, st);
    return launch_k<PATH, BM, BN, BT, DIST, WGM, WGN, PP, true, false, false, true>(a, st);
  } else if constexpr (PATH == P_FP8) {
    // one scale word per row and stage (128-wide blocks, K % 128 == 0: their
    // one byte, replicated)
    if (a.a_b128) return launch_k<PATH, BM, BN, BT, DIST, WGM, WGN, PP, true, false, true>(a, st);
    if ((a.K >> 5) % 4 == 0) return launch_k<PATH, BM, BN, BT, DIST, WGM, WGN, PP, true>(a, st);
  } else if constexpr (PATH == P_F16) {
    if constexpr (!BT && !PP && DIST == 2)
      if (a.K % 64 == 0 && gemm_b_direct()) return launch_k<PATH, BM, BN, BT, DIST, WGM, WGN, PP, true, true>(a, st);
    if (a.K % 64 == 0 && (!BT || a.N % 64 == 0)) return launch_k<PATH, BM, BN, BT, DIST, WGM, WGN, PP, true>(a, st);
  }
  return launch_k<PATH, BM, BN, BT, DIST, WGM, WGN, PP, false>(a, st);
}

static int64_t tile_count(const GemmArgs& a, int bm, int bn) {
  int64_t tm = a.num_groups == 0 ? (a.M + bm - 1) / bm : a.M / bm + a.num_groups;
  return tm * ((a.N + bn - 1) / bn);
}

// Forced tile configuration (the case numbers of launch_p), or -1 for the
// measured choice.  Per host thread (set through mx_gemm_set_tile), so a
// tuning thread never changes the tiles of another thread's calls.
static thread_local int g_tile_override = -1;

void gemm_set_tile(int tile) { g_tile_override = tile; }

// Tile choice: the largest tile that still gives every CU work.  Larger wave
// tiles need fewer LDS fragment bytes per MFMA; 8-wave workgroups put two
// waves on each SIMD.
template <int PATH, bool BT, bool SWI = false>
static hipError_t launch_p(const GemmArgs& a, hipStream_t st) {
  const int64_t cus = 256;
  int t = g_tile_override;
  if constexpr (PATH == P_FP8 && !BT && !SWI) {
    // MXFP8 and blockwise FP8 take the direct-to-LDS 256x256 kernel
    // (configuration 7) once its tiles fill the CUs, where it applies: dense,
    // row-major B, K % 128 == 0
    const bool dma_ok = a.num_groups == 0 && !a.row_index && a.K % 128 == 0;
    if (dma_ok && (t == 7 || (t < 0 && tile_count(a, 256, 256) >= cus)))
      return a.a_b128 ? launch_fp8_dma(a, st) : launch_fp8_pair(a, st);
  }
  if constexpr (PATH == P_F16 && !BT) {
    // NVFP4 likewise takes its direct-to-LDS kernel on 4 waves (7) for
    // launches with row-major B and K % 128 == 0 that fill the CUs, dense or
    // grouped, with or without the fused SwiGLU; 8 is the same kernel on 8
    // waves (measured no faster; dense only)
    const bool dma_ok = a.K % 128 == 0;
    // grouped launches only with K >= 2048: the MoE down GEMM (K = 768, six
    // stages per tile) measured 300 against 278 us on the ping-pong kernel,
    // the gate_up (K = 2048) 461 against 473 us
    if (dma_ok && (t == 7 || (t < 0 && tile_count(a, 256, 256) >= cus && (a.num_groups == 0 || a.K >= 2048)))) {
      if (a.num_groups) return launch_nvfp4_dma<4, true, SWI>(a, st);
      return launch_nvfp4_dma<4, false, SWI>(a, st);
    }
    if constexpr (!SWI)
      if (dma_ok && t == 8 && a.num_groups == 0) return launch_nvfp4_dma<8>(a, st);
  }
  if (t >= 7) t = -1;                    // configurations 7, 8 where they do not apply: the measured choice
  if (t < 0) {
    // measured on MI355X (8192^3, 8192x24576x4096, 8192x28672x4096,
    // 8192x1536x2048, 4096x768x2048, 4096x2048x768, grouped 128 x 512 rows):
    // the ping-pong 256x256 tile runs a tile in about 2.5x the time of the
    // 8-wave 128x128 tile for 4x the work, so NVFP4 takes it whenever its
    // rounds of tiles over the CUs cost less (5 * rounds <= 2 * rounds of
    // 128x128), transposed B included; BF16 takes it once it fills the CUs,
    // else ping-pong 256x128 / 128x128 (for 4096x2048x768 the 128x128 tile is
    // faster on warm repeated launches, 256x128 inside the step with cold
    // inputs: 21.7 against 23.0 us); MXFP8 takes ping-pong 256x128 once
    // that fills the CUs, else the 8-wave 128x128 tile.
    const int64_t r6 = (tile_count(a, 256, 256) + cus - 1) / cus;
    const int64_t r1 = (tile_count(a, 128, 128) + cus - 1) / cus;
    const bool big = tile_count(a, 256, 256) >= cus, mid = tile_count(a, 256, 128) >= cus;
    if (PATH == P_F16) t = 5 * r6 <= 2 * r1 ? 6 : 1;
    else if (PATH == P_BF16) t = big ? 6 : mid ? 5 : 4;
    else t = mid ? 5 : 1;
  }
  switch (t) {
    case 6: return launch_t<PATH, 256, 256, BT, 1, 4, 2, true, SWI>(a, st);
    case 5: return launch_t<PATH, 256, 128, BT, 1, 4, 2, true, SWI>(a, st);
    case 4: return launch_t<PATH, 128, 128, BT, 1, 4, 2, true, SWI>(a, st);
    case 3: return launch_t<PATH, 256, 256, BT, 1, 2, 4, false, SWI>(a, st);
    case 2: return launch_t<PATH, 256, 128, BT, 1, 4, 2, false, SWI>(a, st);
    case 1: return launch_t<PATH, 128, 128, BT, 2, 2, 4, false, SWI>(a, st);
    default: return launch_t<PATH, 128, 128, BT, 2, 2, 2, false, SWI>(a, st);
  }
}

// ------------------------------------------------------------ MoE gate_up with Q(H) in the epilogue
// The experts' gate_up GEMM with the SwiGLU and the per-token NVFP4
// requantization of H in its epilogue: the codes, E4M3 block scales and
// per-token S that nvfp4_quantize (1x16 blocks, per-token S, RNE) gives for
// H, byte for byte, and optionally H itself, without H's round trip through
// HBM ("Miles Blackwell RL ...", section "Um Quantizador Compartilhado É o
// Verdadeiro Mecanismo": one shared quantizer emitting packed FP4, block
// scales and token scales).  S needs the amax of a token's whole H row, so a
// workgroup owns whole rows: 32 tokens x all 2 inter gate_up columns, on 8
// waves (two per SIMD), wave q holding the 32 rows x (P gate + P up) columns
// of H columns [q P, q P + P), P = inter / 8.
//  * Stages of 64 K.  B's 2 inter code rows sit in LDS in the order the
//    waves read them (wave q: its P gate rows, then its P up rows), 64 bytes
//    a row for a pair of stages; each wave loads and reads only its own rows,
//    so it reloads them (the next pair) as soon as it has read the pair's
//    second stage.  A's 32 code rows and the rows' scale words (a row's 4
//    block scales of a stage), B's, then A's, sit in two stage buffers,
//    stage s + 1 loaded as stage s begins.  Everything is loaded straight
//    into LDS; before a stage's last K step every wave waits for its own
//    loads and a barrier makes stage s + 1 visible, whose fragments are then
//    read and converted under that K step's MFMAs.  (Measured at the
//    Qwen3-30B-A3B MoE shape the kernel is bound by L2 requests: a B row's
//    64 bytes per pair are one request, and the weights' scale words in the
//    MFMA layout put 32 rows' words of a stage in one line.)
//  * The K steps are those of the direct-to-LDS NVFP4 kernel (lane half h:
//    K [32h + 8 ks, + 8) of a 64-K block), so H has the bits mx_gemm_swiglu
//    gives.
//  * Epilogue: H (the products' BF16 values through the shared SwiGLU) staged
//    in LDS as whole rows; 16 threads per row take the row's amax and S =
//    amax / 2688, then each its blocks through the quantizer's own block
//    scale and encoder (nvfp4_device.h).
constexpr int QH_BM = 32;                                   // tokens per workgroup
constexpr int QH_ROW = 32;                                  // code bytes per row and stage (64 K)

template <int P>
struct QhLayout {
  static constexpr int INTER = 8 * P;
  static constexpr int NB = 2 * INTER;                      // B rows (gate_up columns)
  // B codes of a stage pair (128 K, 64 bytes a row), one region: each wave
  // reads and reloads only its own rows
  static constexpr int B_CODES = 0;
  static constexpr int B_ROW = 2 * QH_ROW;
  // then two buffers of a stage's A codes and the scale words
  static constexpr int BUF = NB * B_ROW;
  static constexpr int A_CODES = 0;                         // offsets within a buffer
  static constexpr int B_SC = A_CODES + QH_BM * QH_ROW;
  static constexpr int A_SC = B_SC + NB * 4;
  static constexpr int STAGE = A_SC + 256;                  // A's words: one 64-lane load, lanes 32+ write zeros
  static constexpr int LDS = BUF + 2 * STAGE;
  static constexpr int BC_PW = 2 * P / 16;                  // 1 KB code loads per wave and stage pair (16 rows each)
  static constexpr int BS_PW = 2 * P / 64;                  // 256-byte scale-word loads per wave
  static constexpr int HROW = INTER * 2 + 16;               // a staged H row (bytes)
  static_assert(P % 32 == 0 && QH_BM * HROW <= LDS, "layout");
};

struct QhOut {
  uint8_t* codes;
  int64_t ld_codes;                                        // bytes
  uint8_t* scales;
  float* gs;                                               // per-token S
  int mfma;                                                // scale layout of the Q(H) copy
};

// A's 32-byte code rows: the two 16-byte halves sit in slots h ^ ((r >> 3) &
// 1); B's 64-byte rows (a stage pair): chunk c in slot c ^ ((r >> 2) & 3).
// The 16 rows of one LDS read pass then cover all 64 banks.
__device__ __forceinline__ int qh_slot(int r, int h) { return h ^ ((r >> 3) & 1); }
__device__ __forceinline__ int qh_bslot(int r, int c) { return c ^ ((r >> 2) & 3); }

template <int P>
__global__ __launch_bounds__(512) void gemm_nvfp4_swiglu_q_kernel(GemmArgs p, QhOut o) {
  using Lay = QhLayout<P>;
  constexpr int INTER = Lay::INTER;
  constexpr int TN = 2 * P / 32;                            // 32x32 tiles per wave (gate, then up)
  constexpr int NF = 1 + TN;                                // fragments per K step (A, then B)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = p.num_groups ? group_mtiles<QH_BM>(p, lane) : (int)gridDim.x;
  int mt, nt;
  if (!xcd_tile(tiles_m, 1, 1, mt, nt)) return;
  const TileOrigin to = tile_origin<QH_BM>(p, mt, lane);
  if (!to.active) return;
  const int K = (int)p.K;
  const int m0 = (int)to.m0, m_end = (int)to.m_end, grp = to.group;
  auto arow = [&](int m) -> int { return p.row_index ? p.row_index[m] : m; };
  // B row (gate_up column) behind LDS row n: wave q = n / 2P reads gate rows
  // q P .. q P + P, then the matching up rows
  auto brow = [&](int n) -> int {
    const int q = n / (2 * P), j = n - q * (2 * P);
    return j < P ? q * P + j : INTER + q * P + (j - P);
  };
  const int h = lane >> 5, r32 = lane & 31;
  const int nk = K / 64;
  const int nb16 = K >> 4;
  const uint32_t lbase = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  const uint32_t arb = (uint32_t)(p.lda >> 1), brb = (uint32_t)(p.ldb >> 1);   // code bytes per row
  const uint8_t* bbase = p.b + (int64_t)grp * (p.b_group_elems >> 1);
  const uint8_t* bsbase = p.b_scales + (int64_t)grp * p.b_group_scales;
  const srd_t sA = make_srd(p.a, p.a_rows * (int64_t)arb);
  const srd_t sB = make_srd(bbase, 2 * (int64_t)INTER * brb);
  const srd_t sAs = make_srd(p.a_scales, p.a_rows * nb16);
  const srd_t sBs = make_srd(bsbase, p.b_group_scales);
  const uint32_t a_sst = p.a_mfma_layout ? 128u : 4u;                          // a word's step per stage
  const uint32_t b_sst = (p.b_tile || !p.b_mfma_layout) ? 4u : 128u;

  // This wave's loads: the code rows and scale words of its own 2P B rows
  // (LDS rows 2P w ..), the codes per stage pair in 1 KB parts (lane l: row
  // 16k + l / 4, slot l % 4, which holds chunk qh_bslot of the row's 64
  // bytes: one 64-byte request per row) and the words per stage in 256-byte
  // parts (lane l: row 64k + l); wave 0 loads A's codes, wave 1 A's scale
  // words (lanes below 32), per stage.
  uint32_t bc_off[Lay::BC_PW], bs_off[Lay::BS_PW], a_off;
#pragma unroll
  for (int k = 0; k < Lay::BC_PW; ++k) {
    const int n = 2 * P * w + 16 * k + (lane >> 2);
    bc_off[k] = (uint32_t)brow(n) * brb + (uint32_t)qh_bslot(n, lane & 3) * 16u;
  }
#pragma unroll
  for (int k = 0; k < Lay::BS_PW; ++k) {
    const int n = brow(2 * P * w + 64 * k + lane);
    bs_off[k] = p.b_tile ? (uint32_t)((n >> 4) * nb16) : (uint32_t)scale_offset(n, 0, nb16, p.b_mfma_layout);
  }
  if (w == 0) {
    const int r = lane >> 1;
    const bool ok = m0 + r < m_end;
    a_off = in_range(ok, (uint32_t)(ok ? arow(m0 + r) : 0) * arb + (uint32_t)qh_slot(r, lane & 1) * 16u);
  } else {
    const bool ok = lane < 32 && m0 + lane < m_end;
    a_off = in_range(ok, ok ? (uint32_t)scale_offset(arow(m0 + lane), 0, nb16, p.a_mfma_layout) : 0u);
  }
  auto issue = [&](int s) {                                 // stage s's A codes and words into buffer s % 2
    const uint32_t L = lbase + (uint32_t)(Lay::BUF + (s & 1) * Lay::STAGE);
#pragma unroll
    for (int k = 0; k < Lay::BS_PW; ++k)
      dma4(sBs, L + (uint32_t)(Lay::B_SC + (2 * P * w + 64 * k) * 4), bs_off[k] + (uint32_t)s * b_sst);
    if (w == 0) dma16(sA, L + (uint32_t)Lay::A_CODES, a_off + (uint32_t)s * 32u);
    else if (w == 1) dma4(sAs, L + (uint32_t)Lay::A_SC, a_off + (uint32_t)s * a_sst);
  };
  auto issue_b = [&](int q) {                               // this wave's B codes of stages 2q, 2q + 1
#pragma unroll
    for (int k = 0; k < Lay::BC_PW; ++k)
      dma16(sB, lbase + (uint32_t)(Lay::B_CODES + (2 * P * w + 16 * k) * Lay::B_ROW), bc_off[k] + (uint32_t)q * 64u);
  };

  // fragments of a stage: A (f = 0) and B tile f - 1 (LDS rows w 2P + 32(f - 1) + r)
  uint4 raw[NF];
  h2 sc[NF];
  uint32_t co[2][NF], so[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int row = f == 0 ? r32 : w * 2 * P + 32 * (f - 1) + r32;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      co[t][f] = f == 0 ? (uint32_t)(Lay::BUF + Lay::A_CODES + row * QH_ROW + qh_slot(row, h) * 16)
                        : (uint32_t)(Lay::B_CODES + row * Lay::B_ROW + qh_bslot(row, 2 * t + h) * 16);
    so[f] = (uint32_t)(Lay::BUF + (f == 0 ? Lay::A_SC : Lay::B_SC) + row * 4);
  }
  auto read = [&](int s) {
    const uint32_t t = (uint32_t)(s & 1);
    const uint8_t* L = lds + t * Lay::STAGE;                // A and the words: buffer s % 2
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      raw[f] = *reinterpret_cast<const uint4*>(f == 0 ? L + co[0][0] : lds + (t ? co[1][f] : co[0][f]));
      // blocks 2h and 2h + 1 of the stage (K [32h, 32h + 32)) as FP16
      sc[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(*reinterpret_cast<const uint32_t*>(L + so[f]) >> (16 * h),
                                                       1.0f, false);
    }
  };
  v8h cv[2][NF];
  auto convert = [&](int f, int ks, v8h& dst) {
    const h2 s01 = sc[f];
    const h2 sp = (ks >> 1) ? h2{s01.y, s01.y} : h2{s01.x, s01.x};
    const uint32_t word = ks == 0 ? raw[f].x : ks == 1 ? raw[f].y : ks == 2 ? raw[f].z : raw[f].w;
    uint32_t q[4];
    fp4x8_to_f16(word, sp, q);
    dst = __builtin_bit_cast(v8h, make_uint4(q[0], q[1], q[2], q[3]));
  };

  v16f acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  issue_b(0);
  issue(0);
  wait_vmcnt<0>();
  asm volatile("s_barrier" ::: "memory");
  read(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) convert(f, 0, cv[0][f]);

  for (int s = 0; s < nk; ++s) {
    const bool more = s + 1 < nk;
    // buffer (s + 1) % 2 last held stage s - 1, read during stage s - 2
    if (more) issue(s + 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int set = ks & 1;
      if (ks == 3 && more) {
        // this wave's share of stage s + 1 (and, s even, of the pair's B codes)
        wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
        read(s + 1);
        if ((s & 1) == 0 && s + 2 < nk) {
          // the pair's last reads of this wave's B rows are done: load the
          // next pair (needed at the last K step of stage s + 1)
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          issue_b(s / 2 + 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cv[set][1 + i], cv[set][0], acc[i], 0, 0, 0);
        // the conversions of the next K step (of this stage, or stage s + 1's first)
        if (ks < 3 || more) {
          convert(i, (ks + 1) & 3, cv[set ^ 1][i]);
          if (i == TN - 1) convert(TN, (ks + 1) & 3, cv[set ^ 1][TN]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ------------------------------------------------ epilogue
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  uint8_t* const E = lds;                                   // 32 staged H rows
  {
    const float sbg = p.b_gs[grp];
    const int mrow = m0 + r32;
    const float sa = mrow < m_end ? (p.a_gs_per_row ? p.a_gs[arow(mrow)] : p.a_gs[0]) : 0.0f;
    uint8_t* const er = E + r32 * Lay::HROW + (w * P) * 2 + h * 8;
#pragma unroll
    for (int t = 0; t < TN / 2; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float gv[4], uv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[i] = (acc[t][4 * g + i] * sa) * sbg;
          uv[i] = (acc[t + TN / 2][4 * g + i] * sa) * sbg;
        }
        const uint32_t h01 = swiglu_bf16x2(f32x2_to_bf16x2(gv[0], gv[1]), f32x2_to_bf16x2(uv[0], uv[1]));
        const uint32_t h23 = swiglu_bf16x2(f32x2_to_bf16x2(gv[2], gv[3]), f32x2_to_bf16x2(uv[2], uv[3]));
        *reinterpret_cast<uint2*>(er + (t * 32 + g * 8) * 2) = make_uint2(h01, h23);
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // 16 threads per token row, each INTER / 16 consecutive H values (whole
  // 16-value blocks)
  constexpr int PER = INTER / 16, NBLK = PER / 16;
  const int rr = tid >> 4, part = tid & 15;
  const int64_t m = m0 + rr;
  uint4 v[2 * NBLK];
#pragma unroll
  for (int c = 0; c < 2 * NBLK; ++c)
    v[c] = *reinterpret_cast<const uint4*>(E + rr * Lay::HROW + (part * PER + 8 * c) * 2);
  uint32_t mb = 0;
#pragma unroll
  for (int c = 0; c < 2 * NBLK; ++c) mb = umax(mb, amax8_bits(v[c]));
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) mb = umax(mb, lane_xor_u32(mb, x));
  const float S = __uint_as_float(mb) / 2688.0f;
  if (m < m_end) {
    if (part == 0) o.gs[m] = S;
    with_frame(S, [&](auto tiny) {
      constexpr bool TINY = decltype(tiny)::value;
      const u32x4 none = {0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const uint32_t ab = umax(amax8_bits(v[2 * b]), amax8_bits(v[2 * b + 1]));
        const BlockScale bs = nv_block_scale(__uint_as_float(ab), S);
        const uint32_t q0 = nv_encode8<false, TINY>(v[2 * b], bs.r, none);
        const uint32_t q1 = nv_encode8<false, TINY>(v[2 * b + 1], bs.r, none);
        const int blk = part * NBLK + b;
        *reinterpret_cast<uint2*>(o.codes + m * o.ld_codes + blk * 8) = make_uint2(q0, q1);
        o.scales[scale_offset(m, blk, INTER / 16, o.mfma)] = (uint8_t)bs.code;
      }
    });
    if (p.c) {
#pragma unroll
      for (int c = 0; c < 2 * NBLK; ++c)
        *reinterpret_cast<uint4*>(p.c + m * p.ldc + part * PER + 8 * c) = v[c];
    }
  }
}

template <int P>
static hipError_t launch_swiglu_q_p(const GemmArgs& a, const QhOut& o, hipStream_t st) {
  using Lay = QhLayout<P>;
  int64_t tiles_m = a.num_groups ? a.M / QH_BM + a.num_groups : (a.M + QH_BM - 1) / QH_BM;
  if (tiles_m < 1) tiles_m = 1;
  if (tiles_m >= (1ll << 31)) return hipErrorInvalidValue;
  const size_t lds = (size_t)Lay::LDS;
  static std::atomic<uint32_t> lds_set{0};
  if (hipError_t e = ensure_lds_limit((const void*)gemm_nvfp4_swiglu_q_kernel<P>, (int)lds, lds_set); e != hipSuccess)
    return e;
  hipLaunchKernelGGL(gemm_nvfp4_swiglu_q_kernel<P>, dim3((unsigned)tiles_m), dim3(512), lds, st, a, o);
  return hipGetLastError();
}

hipError_t launch_gemm_swiglu_q(const GemmArgs& a, uint8_t* codes, int64_t ld_codes, uint8_t* scales, float* gs,
                                bool mfma, hipStream_t st) {
  const QhOut o = {codes, ld_codes, scales, gs, (int)mfma};
  switch (a.swiglu_inter) {
    case 256: return launch_swiglu_q_p<32>(a, o, st);
    case 512: return launch_swiglu_q_p<64>(a, o, st);
    case 768: return launch_swiglu_q_p<96>(a, o, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int path, bool bt, const GemmArgs& a, hipStream_t st) {
  if (a.swiglu_inter) return launch_p<P_F16, false, true>(a, st);
  if (path == P_FP8) return bt ? launch_p<P_FP8, true>(a, st) : launch_p<P_FP8, false>(a, st);
  if (path == P_F16) return bt ? launch_p<P_F16, true>(a, st) : launch_p<P_F16, false>(a, st);
  return bt ? launch_p<P_BF16, true>(a, st) : launch_p<P_BF16, false>(a, st);
}

}  // namespace mxq
