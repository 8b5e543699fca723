/*
 * mxq.h -- C ABI of the microscaling quantization library for MI355X (gfx950).
 *
 * What it computes (sources are the web pages this library is written from):
 *
 *  - MXFP8: blocks of 32 E4M3 values sharing one E8M0 power-of-two scale
 *    ("Miles Blackwell RL Troca a Uniformidade BF16 por MXFP8 e NVFP4
 *    Nativos", section "O Suporte Miles Blackwell Agora Abrange Todo o Loop
 *    de RL"; "End-to-End MXFP8 Reinforcement Learning on Blackwell",
 *    Table 10 F6: an E8M0 scale keeps only an exponent), plus a 32x32 tile
 *    variant for weights read in both orientations.
 *  - NVFP4: blocks of 16 E2M1 values with an E4M3 block scale under a second
 *    FP32 scale that is per token (same Miles page, same section; "NVFP4 RL
 *    training", baseline-recipe section) or per tensor, with 16x16 weight
 *    blocks shared by FPROP and DGRAD, RNE for weights/activations and
 *    stochastic rounding for gradients ("Train models faster with JAX and
 *    MaxText using NVFP4 on NVIDIA Blackwell", section "NVFP4 pretraining
 *    recipe").
 *  - BF16 dequantization DQ(Q(x)) for the dequantized backward ("NVFP4 RL
 *    training", section on the dequantized backward).
 *  - FPROP / DGRAD / WGRAD GEMMs on the quantized operands with BF16 output
 *    (NVFP4 MaxText page, "NVFP4 pretraining recipe"), dense or grouped per
 *    MoE expert.
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no device memory, never synchronizes, and keeps no pointer
 *    after a call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it; results are ready when the stream reaches that point.
 *  - BF16 values are passed as their uint16_t bit patterns; matrices are
 *    row-major with an explicit leading dimension (elements, unless stated).
 *  - Arguments are validated on the host before anything is launched.  On any
 *    error nothing is written, no kernel is launched, the status says why, and
 *    mxq_last_error() (thread-local) gives a message.  No C++ exception ever
 *    crosses this interface.
 *  - Inputs must be finite.  Non-finite inputs give unspecified codes.
 *  - Calls may run concurrently on different streams when their output
 *    buffers do not overlap.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_VERSION 1

typedef enum {
  MXQ_OK = 0,
  MXQ_EINVAL = 1,        /* null pointer, negative size, bad enum value        */
  MXQ_ESHAPE = 2,        /* a size is not a multiple of what the format needs  */
  MXQ_EALIGN = 3,        /* pointer or leading dimension not 16-byte aligned   */
  MXQ_EUNSUPPORTED = 4,  /* a valid but unsupported combination (never emulated) */
  MXQ_EHIP = 5           /* the HIP runtime reported an error at launch        */
} mxq_status;

typedef enum {
  MXQ_FMT_MXFP8 = 0,     /* E4M3 codes (1 byte) + E8M0 scales                  */
  MXQ_FMT_NVFP4 = 1,     /* E2M1 codes (2 per byte) + E4M3 scales + FP32 scale */
  MXQ_FMT_BF16 = 2,      /* plain BF16 (GEMM operands only)                    */
  MXQ_FMT_FP8_B128 = 3,  /* DeepSeek-style blockwise FP8: E4M3 codes (1 byte)
                          * + E8M0 power-of-two scales per 1x128 row block or
                          * 128x128 tile, linear layout (fp8bw_quantize)       */
  MXQ_FMT_FP8_B128_F32 = 4 /* the same blocks with binary32 scales (an operand's
                          * scales pointer then points to 4-byte aligned
                          * floats; fp8bw_quantize_f32)                        */
} mxq_format;

typedef enum {
  /* Blocks along the contiguous dimension: 1x32 (MXFP8) or 1x16 (NVFP4). */
  MXQ_BLOCK_ROW = 0,
  /* Blocks along rows: 32x1 or 16x1.  The copy is stored TRANSPOSED,
   * [cols, rows], so that its blocks are contiguous again (the copy a WGRAD
   * GEMM reads). */
  MXQ_BLOCK_COL = 1,
  /* One scale per 32x32 (MXFP8) or 16x16 (NVFP4) tile; the same codes and
   * scales read transposed serve the transposed GEMM operand. */
  MXQ_BLOCK_TILE = 2,
  /* MXFP8 only: ROW and COL copies from one read of the input. */
  MXQ_BLOCK_DUAL = 3,
  /* BF16 operands: no blocks. */
  MXQ_BLOCK_NONE = 4
} mxq_block;

typedef enum {
  MXQ_GS_NONE = 0,       /* MXFP8 / BF16: no second-level scale                 */
  MXQ_GS_PER_ROW = 1,    /* NVFP4: one FP32 scale per row (per token)           */
  MXQ_GS_PER_TENSOR = 2, /* NVFP4: one FP32 scale for the whole tensor          */
  MXQ_GS_GIVEN = 3       /* NVFP4: the caller supplies the per-tensor scale     */
} mxq_gscale;

typedef enum {
  MXQ_ROUND_RNE = 0,     /* round to nearest, ties to even                      */
  MXQ_ROUND_SR = 1,      /* stochastic rounding (NVFP4 elements only)           */
  /* NVFP4 ROW and TILE copies: RNE with the Four-Over-Six block-scale choice
   * ("NVFP4 RL training" / "The 4-bitter Lesson", section on Four-Over-Six
   * for RL weights and activations).  Each block (or 16x16 tile) is encoded
   * under s6 = E4M3(fl(a_b / fl(6*S))) and s4 = E4M3(fl(a_b / fl(4*S)))
   * (both RNE, saturating at 448) and keeps s4 iff the binary32 sum of its
   * squared dequantization errors e = fl(x - fl(fl(value(code)*s_b)*S)),
   * squared with one rounding each, is strictly smaller.  The sum is a
   * pairwise tree in element order (neighbours first); a tile sums each
   * row's 16 squares by that tree and then the 16 row sums by it.  Ties keep
   * s6.  The stored copy is plain NVFP4 (the chosen s_b is its block scale),
   * so mx_dequantize and mx_gemm read it unchanged. */
  MXQ_ROUND_RNE_4OVER6 = 2
} mxq_round;

typedef enum {
  /* Scale grid row-major: [rows, cols/B] for 1D blocks, [rows/B, cols/B] for
   * tiles (B = block size; for a COL copy "rows" are the input's columns). */
  MXQ_LAYOUT_LINEAR = 0,
  /* 1D blocks only: chunks of 32 rows x 4 consecutive blocks, 128 bytes each,
   * stored chunk-row-major; inside a chunk row r%32 owns bytes 4*(r%32)..+3
   * (its 4 blocks in order).  Byte offset of (row r, block b), with
   * B = blocks per row:  ((r/32)*(B/4) + b/4)*128 + (r%32)*4 + b%4.
   * Needs rows % 32 == 0 and B % 4 == 0.  This is the order in which the GEMM
   * kernels fetch scales, one 128-byte line per 32-row MFMA tile. */
  MXQ_LAYOUT_MFMA = 1
} mxq_scale_layout;

/*
 * mx_quantize -- MXFP8 quantization of a BF16 matrix x [rows, cols].
 *
 * Format: 32 E4M3 values share one E8M0 scale ("Miles Blackwell RL Troca a
 * Uniformidade BF16 por MXFP8 e NVFP4 Nativos", section "O Suporte Miles
 * Blackwell Agora Abrange Todo o Loop de RL"; "End-to-End MXFP8 Reinforcement
 * Learning on Blackwell", Table 10 F6: the scale keeps only an exponent).
 * Rowwise and columnwise copies are both made from the original values
 * (Miles page, section "Um Quantizador Compartilhado É o Verdadeiro
 * Mecanismo"), which is what DUAL does from one read.
 *
 * Block rule (the pages give none; this is the plainest reading of "no block
 * overflows after scaling"): the block's E8M0 exponent e is the smallest
 * integer in [-127, 127] with max|x| <= 448 * 2^e (all-zero block: e = -127,
 * code 0x00); each code is E4M3 round-to-nearest-even of x * 2^-e, which is an
 * exact scaling and never saturates.
 *
 *   x, ld_x            input, row-major, ld_x >= cols (elements)
 *   block              ROW: codes [rows, cols] (ld_codes), scales per layout
 *                      COL: codes [cols, rows] (ld_codes), scales [cols, rows/32]
 *                      TILE: codes [rows, cols], scales [rows/32, cols/32] LINEAR;
 *                            with codes_col non-NULL also the transposed copy:
 *                            codes_col [cols, rows] (ld_codes_col) and
 *                            scales_col [cols/32, rows/32] LINEAR.  A 32x32
 *                            block's scale serves its rows and its columns, so
 *                            that copy is exactly the TILE quantization of x^T
 *                            (the weight for DGRAD, read untransposed).
 *                      DUAL: ROW copy into codes/scales AND COL copy into
 *                            codes_col/scales_col (ld_codes_col)
 *   layout             LINEAR or MFMA (MFMA: ROW/COL/DUAL only)
 *   codes_col, scales_col, ld_codes_col   DUAL (required) and TILE (optional
 *                      transposed copy), else ignored (may be NULL)
 * Shapes: cols % 32 == 0; rows % 32 == 0 for COL, TILE, DUAL.
 * Alignment: x, codes, codes_col 16-byte aligned; ld_x*2, ld_codes and
 * ld_codes_col multiples of 16.
 */
mxq_status mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                       mxq_block block, mxq_scale_layout layout,
                       uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                       uint8_t* codes_col, int64_t ld_codes_col, uint8_t* scales_col,
                       void* stream);

/*
 * nvfp4_quantize -- NVFP4 quantization of a BF16 matrix x [rows, cols].
 *
 * Format and recipe: 16 E2M1 values share an E4M3 block scale under a second
 * FP32 scale computed online per token, and one fused op yields packed FP4,
 * block scales and token scales ("Miles Blackwell RL ...", sections "O
 * Suporte Miles Blackwell Agora Abrange Todo o Loop de RL" and "Um
 * Quantizador Compartilhado É o Verdadeiro Mecanismo"); per-tensor second
 * scales, 16x16 weight blocks, 1x16 activation and gradient blocks, RNE for
 * weights and activations and stochastic rounding for gradients ("Train
 * models faster with JAX and MaxText using NVFP4 on NVIDIA Blackwell",
 * section "NVFP4 pretraining recipe").
 *
 * Steps, each fl() one binary32 IEEE operation (round-to-nearest-even,
 * subnormals kept, no fused multiply-add):
 *   S   = fl(A / 2688), A = max|x| over the row (PER_ROW) or tensor
 *         (PER_TENSOR); GIVEN reads S from gscales[0].  A = 0 gives S = 0.
 *   s_b = E4M3 RNE (saturating) of fl(a_b / fl(6*S)), a_b = block max|x|.
 *   code: s_b == 0 -> signed zero; else E2M1 of fl(x * fl(1 / fl(s_b*S))),
 *         RNE or stochastic (saturating at 6).
 * Stochastic rounding draws 16 bits per element from Philox4x32-10 with key
 * (seed lo, seed hi) and counter (n lo, n hi, stream_id, tensor_tag),
 * n = idx / 8, idx = row*cols + col of the element in x; element idx takes
 * output word (idx%8)/2, low half if idx is even, high half if odd; it rounds
 * up iff draw * 2^-16 < the fraction of the way to the next grid point.
 *
 *   block   ROW (1x16): codes [rows, cols/2] bytes (ld_codes_bytes),
 *                        block_scales per layout, gscales [rows] (PER_ROW) or [1]
 *           COL (16x1): transposed copy, codes [cols, rows/2] bytes,
 *                        block_scales [cols, rows/16]; PER_TENSOR or GIVEN only
 *           TILE (16x16): codes [rows, cols/2], block_scales [rows/16, cols/16]
 *                        LINEAR; PER_TENSOR or GIVEN only
 *   gs      PER_ROW (ROW only), PER_TENSOR, GIVEN
 *   rnd     RNE, SR, or RNE_4OVER6 (ROW and TILE; COL gives MXQ_EUNSUPPORTED)
 *   codes   two E2M1 codes per byte, even element in the low nibble
 *   gscales PER_ROW/PER_TENSOR: written; GIVEN: read (caller's S >= 0)
 * With PER_TENSOR the call enqueues an extra read pass over x for A, using
 * gscales[0] as its accumulator (between the two kernels it holds A tagged
 * with bit 31; once the call's work completes it holds S); gscales must not
 * alias x, codes or scales.
 * Shapes: cols % 16 == 0 (ROW); rows % 16 == 0 and cols % 16 == 0 (COL,
 * TILE).  Alignment: x, codes 16-byte aligned, ld_x*2 and ld_codes_bytes
 * multiples of 16; gscales 4-byte aligned.
 * When S < 2^-64 the element step is taken with x and S scaled by 2^64
 * (exact): code = E2M1 of fl(fl(x*2^64) * fl(1 / fl(s_b*fl(S*2^64)))), which
 * equals the unscaled step wherever s_b*S is a binary32 normal and keeps it
 * finite for every finite BF16 input.
 */
mxq_status nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          mxq_block block, mxq_gscale gs, mxq_round rnd,
                          uint64_t seed, uint32_t stream_id, uint32_t tensor_tag,
                          mxq_scale_layout layout,
                          uint8_t* codes, int64_t ld_codes_bytes,
                          uint8_t* block_scales, float* gscales,
                          void* stream);

/*
 * nvfp4_quantize_dq -- nvfp4_quantize with block TILE (16x16, the weight
 * copy) that also writes, in the same pass, the dequantized BF16 copy
 * dq[r, c] = bf16_RNE(fl(fl(value(code) * s_b) * S)) -- exactly what
 * mx_dequantize returns for that copy -- for the dequantized backward, whose
 * BF16 GEMMs read DQ(Q(w)) ("NVFP4 RL training" / "The 4-bitter Lesson",
 * section on the dequantized backward).  Saves the dequantizer's launch and
 * its re-read of the codes.
 *   gs      PER_TENSOR or GIVEN;  rnd  RNE or RNE_4OVER6 (SR: MXQ_EUNSUPPORTED)
 *   dq      BF16 [rows, cols], ld_dq elements (16-byte aligned, ld_dq*2 % 16 == 0)
 *   other arguments, shapes and errors as nvfp4_quantize with block TILE,
 *   LINEAR scale layout.
 */
mxq_status nvfp4_quantize_dq(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                             mxq_gscale gs, mxq_round rnd, uint8_t* codes, int64_t ld_codes_bytes,
                             uint8_t* block_scales, float* gscales, uint16_t* dq, int64_t ld_dq,
                             void* stream);

/*
 * nvfp4_quantize_rowcol -- the two NVFP4 copies a linear layer needs of an
 * activation or output gradient x [rows, cols]: the rowwise copy with a
 * per-token second scale (FPROP / DGRAD operand) and the columnwise copy with
 * a per-tensor second scale (WGRAD operand), both made from x ("Miles
 * Blackwell RL ...", section "Um Quantizador Compartilhado É o Verdadeiro
 * Mecanismo": rowwise and columnwise copies from the high-precision
 * original; "Train models faster with JAX and MaxText using NVFP4 on NVIDIA
 * Blackwell", section "NVFP4 pretraining recipe": 1x16 blocks, SR for
 * gradients).  Exactly what nvfp4_quantize returns for block ROW with
 * PER_ROW and for block COL with PER_TENSOR, but in two passes instead of
 * three: the rowwise pass also accumulates the tensor amax that the
 * columnwise copy's S needs.  Stochastic rounding (rnd SR) draws with
 * stream_id 0 for the rowwise copy and 1 for the columnwise copy.
 *   rnd        RNE or SR (RNE_4OVER6: MXQ_EUNSUPPORTED)
 *   codes, block_scales, gscales        the ROW copy (codes [rows, cols/2]
 *              bytes, scales per layout, gscales [rows])
 *   codes_col, block_scales_col, gscale_col   the COL copy (codes [cols,
 *              rows/2] bytes, scales [cols, rows/16] per layout, gscale_col
 *              [1]; between the two passes gscale_col[0] holds the tagged
 *              amax; it must not alias gscales)
 *   layout     LINEAR or MFMA for both copies (MFMA: rows, cols % 64 == 0)
 * Shapes: rows % 16 == 0, cols % 16 == 0.  Alignment as nvfp4_quantize for
 * each copy.
 */
mxq_status nvfp4_quantize_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                 mxq_round rnd, uint64_t seed, uint32_t tensor_tag, mxq_scale_layout layout,
                                 uint8_t* codes, int64_t ld_codes_bytes, uint8_t* block_scales,
                                 float* gscales, uint8_t* codes_col, int64_t ld_codes_col_bytes,
                                 uint8_t* block_scales_col, float* gscale_col, void* stream);

/*
 * nvfp4_quantize_tile_t -- nvfp4_quantize with block TILE (16x16, the weight
 * copy) that also writes, in the same pass, the transposed copy: the 16x16
 * quantization of x^T.  A 16x16 tile's scale serves its rows and its columns,
 * so FPROP and DGRAD share the tile scales ("Train models faster with JAX and
 * MaxText using NVFP4 on NVIDIA Blackwell", section "NVFP4 pretraining
 * recipe"), and the transposed copy is exactly the codes transposed and the
 * scale grid transposed.  DGRAD (dX = dY W) then reads it row-major as B
 * (transposed = 0) instead of transposing the weight on its way into the GEMM.
 *   codes_t         [cols, rows/2] bytes (ld_codes_t_bytes), two codes per
 *                   byte, even row index in the low nibble; 8-byte aligned,
 *                   ld_codes_t_bytes % 8 == 0
 *   block_scales_t  [cols/16, rows/16] E4M3, LINEAR
 *   other arguments, shapes and errors as nvfp4_quantize with block TILE,
 *   LINEAR scale layout (any rounding: the codes are transposed as encoded).
 */
mxq_status nvfp4_quantize_tile_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                 mxq_gscale gs, mxq_round rnd, uint64_t seed, uint32_t stream_id,
                                 uint32_t tensor_tag, uint8_t* codes, int64_t ld_codes_bytes,
                                 uint8_t* block_scales, uint8_t* codes_t, int64_t ld_codes_t_bytes,
                                 uint8_t* block_scales_t, float* gscales, void* stream);

/*
 * nvfp4_quantize_rht -- columnwise NVFP4 copy (COL, 16x1 blocks, stored
 * transposed) of the random Hadamard transform of x [rows, cols].  The NVFP4
 * pretraining recipe applies this transform to the two inputs of the WGRAD
 * GEMM only ("Train models faster with JAX and MaxText using NVFP4 on NVIDIA
 * Blackwell", section "NVFP4 pretraining recipe"); FPROP and DGRAD operands
 * use nvfp4_quantize.
 *
 * Each 16-row block v of every column becomes y = (1/4) H16 D v, H16 the
 * Sylvester Hadamard matrix (entry (i,j) = (-1)^popcount(i & j)), D the
 * diagonal with -1 where bit i of sign_mask is set and +1 elsewhere.  The
 * matrix is orthogonal: quantize both WGRAD operands (dY and X, rows = tokens)
 * with the SAME mask and dY^T X is unchanged before rounding.  The caller
 * draws the mask (the transform's randomness) and may redraw it per step.
 * Binary32: sign flips, then the butterfly over strides 1, 2, 4, 8 (each
 * (a, b) -> (a + b, a - b), one rounded operation), then the exact scaling
 * by 1/4.  y is then quantized exactly as nvfp4_quantize quantizes a COL
 * copy of a binary32 input: A = max|y| over the tensor (PER_TENSOR, one extra
 * read pass over x that computes the transform too) or S given (GIVEN), block
 * scales from the 16-value block max|y|, RNE or stochastic rounding with the
 * draw of element (row, col) of y.
 *
 *   sign_mask  bits 0..15 (higher bits: MXQ_EINVAL)
 *   gs         PER_TENSOR or GIVEN (PER_ROW: MXQ_EUNSUPPORTED)
 *   outputs    as nvfp4_quantize with block COL: codes [cols, rows/2] bytes
 *              (ld_codes_bytes), block_scales per layout ([cols, rows/16]
 *              LINEAR; MFMA needs cols % 32 == 0 and rows % 64 == 0), gscales[0]
 * Shapes: rows % 16 == 0, cols % 16 == 0.  Alignment as nvfp4_quantize.  x
 * must be finite.
 */
mxq_status nvfp4_quantize_rht(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              uint32_t sign_mask, mxq_gscale gs, mxq_round rnd,
                              uint64_t seed, uint32_t stream_id, uint32_t tensor_tag,
                              mxq_scale_layout layout,
                              uint8_t* codes, int64_t ld_codes_bytes,
                              uint8_t* block_scales, float* gscales,
                              void* stream);

/*
 * fp8bw_quantize -- DeepSeek-style blockwise FP8 of a BF16 matrix x [rows,
 * cols], with power-of-two scales.  The blockwise FP8 recipe quantizes
 * weights in [128, 128] blocks and input activations and output gradients in
 * [1, 128] blocks ("NVIDIA NeMo RL agora roda treino ... FP8 ponta a ponta",
 * section "FP8 nas camadas lineares"); on Blackwell that recipe's learner is
 * restricted to power-of-two scales ("End-to-End MXFP8 Reinforcement Learning
 * on Blackwell", Table 1), which is also what the scaled MFMA takes here.
 * Rule: the MXFP8 rule over a 128-value block (or a 128x128 tile): e is the
 * smallest integer in [-127, 127] with amax <= 448 * 2^e (-127 for a zero
 * block), stored as the E8M0 byte e + 127; codes are E4M3 RNE of x * 2^-e.
 *
 *   block   ROW  (1x128):  codes [rows, cols] (ld_codes), scales [rows, cols/128]
 *           COL  (128x1):  transposed copy, codes [cols, rows], scales [cols, rows/128]
 *           TILE (128x128): codes [rows, cols], scales [rows/128, cols/128];
 *                           with codes_col/scales_col also the transposed copy
 *                           ([cols, rows], scales [cols/128, rows/128]), the
 *                           same codes transposed (DGRAD reads it untransposed)
 *           DUAL: ROW into codes/scales and COL into codes_col/scales_col
 * Shapes: cols % 128 == 0; rows % 128 == 0 except for ROW.  Alignment: x and
 * codes 16-byte aligned, ld_x*2 and ld_codes multiples of 16.  The scales are
 * always in the linear layout; the GEMM takes them as MXQ_FMT_FP8_B128.
 */
mxq_status fp8bw_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          mxq_block block, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                          uint8_t* codes_col, int64_t ld_codes_col, uint8_t* scales_col,
                          void* stream);

/*
 * fp8bw_quantize_f32 -- blockwise FP8 with binary32 block scales, the
 * DeepSeek-V3 recipe itself and the FP32-scale arm of the blockwise
 * comparison ("End-to-End MXFP8 Reinforcement Learning on Blackwell",
 * Table 1).  Same blocks, layouts, shapes and alignment as fp8bw_quantize;
 * the scales are floats (4-byte aligned).
 * Rule: s = amax / 448 in binary32 (one correctly rounded division; amax over
 * the 128 values or the 128x128 tile); codes are E4M3 RNE of the binary32
 * quotient x / s clamped to [-448, 448] (the quotient of the block maximum
 * can exceed 448 by an ulp and then encodes as 448).  A zero block stores
 * s = 0 and zero codes.  The GEMM takes the copies as MXQ_FMT_FP8_B128_F32.
 */
mxq_status fp8bw_quantize_f32(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              mxq_block block, uint8_t* codes, int64_t ld_codes, float* scales,
                              uint8_t* codes_col, int64_t ld_codes_col, float* scales_col,
                              void* stream);

/*
 * mx_dequantize -- DQ(Q(x)) of one stored copy to BF16, the operand of the
 * dequantized backward, whose BF16 GEMMs read DQ(Q(w)) ("NVFP4 RL training" /
 * "The 4-bitter Lesson", section on the dequantized backward).  (rows, cols) is the shape of the STORED copy (for a
 * COL copy that is [input cols, input rows]); block says how its scales are
 * laid out (ROW for a COL copy too, since the stored copy is row-blocked).
 *   MXFP8, FP8_B128: bf16_RNE(value(c) * 2^e)  (exact unless beyond the BF16 range)
 *   FP8_B128_F32: bf16_RNE(fl32(value(c) * s))
 *   NVFP4: bf16_RNE(fl(fl(value(c) * s_b) * S))
 *   ld_codes  elements for MXFP8 and FP8_B128, BYTES for NVFP4; ld_out elements.
 *   gscales   NVFP4 only ([rows] for PER_ROW, [1] otherwise); may be NULL otherwise.
 *   FP8_B128, FP8_B128_F32: LINEAR scales, gs NONE, cols % 128 (and rows %
 *   128 for TILE); FP8_B128_F32 scales are 4-byte aligned floats.
 */
mxq_status mx_dequantize(mxq_format fmt, const uint8_t* codes, int64_t ld_codes,
                         const uint8_t* scales, const float* gscales,
                         int64_t rows, int64_t cols, mxq_block block, mxq_gscale gs,
                         mxq_scale_layout layout, uint16_t* out, int64_t ld_out,
                         void* stream);

/*
 * A GEMM operand: one stored copy made by the quantizers above, or BF16.
 *
 * A is logically [M, K], B logically [N, K]; both are normally stored with K
 * contiguous (rowwise blocks along K).  B with transposed != 0 is stored
 * [K, N] (N contiguous) and must be tile-blocked (MXFP8 32x32, NVFP4 16x16)
 * or BF16: that is how a DGRAD reads the FPROP weight copy.
 *   data     codes (MXFP8: 1 B/elem; NVFP4: packed, 2 elem/B) or BF16 values
 *   ld       leading dimension of the stored matrix in ELEMENTS (even for NVFP4)
 *   scales   block scales of the stored copy (NULL for BF16)
 *   gscales  NVFP4 second-level scales (per row of A, or per tensor; for a
 *            grouped B one per group); NULL otherwise
 *   block    ROW (1D along K), TILE (2D), NONE (BF16)
 *   gs       PER_ROW (A only), PER_TENSOR / GIVEN (same meaning here), NONE
 *   layout   scale layout (MFMA allowed for ROW blocks)
 * Grouped B: num_groups matrices stored back to back, group g at
 *   data + g*N*ld elements, scales + g*(N*K/B) bytes, gscales + g.
 */
typedef struct {
  mxq_format fmt;
  const void* data;
  const uint8_t* scales;
  const float* gscales;
  mxq_block block;
  mxq_gscale gs;
  mxq_scale_layout layout;
  int64_t ld;
  int32_t transposed;
} mxq_operand;

/*
 * mx_gemm -- C[M, N] = sum_k A[m, k] * B[n, k], FP32 accumulation, BF16 out:
 * the FPROP, DGRAD and WGRAD GEMMs of a linear layer on its quantized
 * operands, with BF16 outputs ("Train models faster with JAX and MaxText
 * using NVFP4 on NVIDIA Blackwell", section "NVFP4 pretraining recipe"; MXFP8
 * on every GEMM: "Miles Blackwell RL ...", section "O Suporte Miles Blackwell
 * Agora Abrange Todo o Loop de RL"), dense or grouped per MoE expert with the
 * routed rows gathered ("Miles Blackwell RL ...", same section: the routed
 * experts run in NVFP4).  a_rows extends the call beyond the four-argument
 * shape (M, N, K): with a gather index the rows of A are not the rows of C,
 * so the library needs A's own row count to bound its loads.
 *   FPROP  Y  = X  * W^T : A = rowwise X,  B = W (rowwise or tile)
 *   DGRAD  dX = dY * W   : A = rowwise dY, B = W tile copy with transposed=1
 *   WGRAD  dW = dY^T * X : A = columnwise dY copy, B = columnwise X copy
 * A and B must have the same format (MXFP8 x MXFP8 or FP8_B128 x FP8_B128
 * on the scaled MFMA, NVFP4 x NVFP4 dequantized exactly to FP16 for the FP16
 * MFMA, or BF16 x BF16); mixed formats give MXQ_EUNSUPPORTED.
 * FP8_B128_F32 x FP8_B128_F32 (binary32 block scales): each 128-wide K
 * block's partial sums come from the scaled MFMA with unit scales and are
 * accumulated as fma(s_a(m, kb) * s_b(n, kb), P_kb, acc) in binary32.  Dense
 * only (num_groups 0, no gather), operands as stored (transposed = 0: DGRAD
 * reads the weight's transposed TILE copy), ROW or TILE scales for either.
 *   c, ldc              BF16 output, row-major
 *   num_groups          0 for a dense GEMM; else grouped (MoE experts)
 *   group_row_offsets   device int32 [num_groups+1], non-decreasing, from 0 to
 *                       M; rows [off[g], off[g+1]) of C use B group g
 *   a_row_index         device int32 [M] or NULL: row r of C reads A row
 *                       a_row_index[r] (gather), every entry in [0, a_rows)
 *   a_rows              rows stored in A (== M when a_row_index is NULL)
 * Shapes: K % 32 (MXFP8), K % 128 (FP8_B128, FP8_B128_F32), K % 16 (NVFP4), K % 8 (BF16); a transposed B needs
 * N and K multiples of its tile size.  M, N any positive size.
 * Offsets and indices are read on the device and are NOT validated: values
 * outside the stated ranges give undefined results.
 */
mxq_status mx_gemm(const mxq_operand* a, const mxq_operand* b,
                   int64_t M, int64_t N, int64_t K, int64_t a_rows,
                   uint16_t* c, int64_t ldc,
                   int32_t num_groups, const int32_t* group_row_offsets,
                   const int32_t* a_row_index, void* stream);

/*
 * mx_gemm_set_tile -- force the workgroup tile of the later mx_gemm and
 * mx_gemm_swiglu calls made FROM THE CALLING HOST THREAD (a tuning and test
 * aid; the default is the measured choice).  The setting is thread-local, the
 * one piece of state the library keeps besides the thread-local error text;
 * other threads are unaffected.
 *   tile  -1  the measured choice per path and shape (default)
 *          0  128x128, 4 waves (2x2), two staging sets
 *          1  128x128, 8 waves (2x4), two staging sets
 *          2  256x128, 8 waves (4x2), one staging set
 *          3  256x256, 8 waves (2x4), one staging set
 *          4  128x128, 8 waves in two ping-pong groups
 *          5  256x128, 8 waves in two ping-pong groups
 *          6  256x256, 8 waves in two ping-pong groups
 *          7  MXFP8 and NVFP4: 256x256, 4 waves, operands loaded straight
 *             into LDS (dense launches with row-major B; K % 128 == 0; any
 *             other call under 7 or 8 takes the measured choice)
 *          8  NVFP4: the same on 8 waves
 * Every configuration computes the same result bit for bit (the K order of
 * the accumulation does not depend on the tile).  Returns MXQ_EINVAL outside
 * [-1, 8].  It applies to calls made after it returns; launches already
 * queued keep their tile.
 */
mxq_status mx_gemm_set_tile(int32_t tile);

/*
 * mx_swiglu -- h = silu(g) * u for a [rows, 2*inter] BF16 gate_up output
 * (gate = first inter columns, up = last inter columns), computed in binary32
 * with silu(g) = g / (1 + exp(-g)), stored as BF16 RNE [rows, inter].
 * This sits between the grouped gate_up and down GEMMs of the MoE experts
 * (SwiGLU experts: "Miles Blackwell RL ...", section "Um Quantizador
 * Compartilhado É o Verdadeiro Mecanismo").  inter % 8 == 0; 16-byte aligned.
 */
mxq_status mx_swiglu(const uint16_t* gu, int64_t rows, int64_t inter, int64_t ld_gu,
                     uint16_t* h, int64_t ld_h, void* stream);

/*
 * mx_gemm_swiglu -- the MoE gate_up GEMM with the SwiGLU fused into its
 * epilogue: H[M, inter] = silu(G) * U with [G | U] = A * B^T, computed exactly
 * as mx_swiglu(mx_gemm(...)) computes it (the GEMM's BF16 products, then the
 * same binary32 SwiGLU), without the [M, 2*inter] BF16 round trip through HBM.
 * The pages attribute part of NVFP4's training cost to the unfused steps
 * around the expert GEMMs ("Miles Blackwell RL ...", section "Um Quantizador
 * Compartilhado É o Verdadeiro Mecanismo").
 *   a, b      NVFP4 operands as for mx_gemm; b holds, per group, the gate rows
 *             [0, inter) then the up rows [inter, 2*inter) (row-major, not
 *             transposed; ROW or TILE blocks)
 *   h, ldh    BF16 output [M, inter], row-major
 *   other arguments as for mx_gemm (grouped launch, gather index)
 * Shapes: inter % 64 == 0, K % 64 == 0.  Other formats or a transposed B give
 * MXQ_EUNSUPPORTED.  The per-token requantization of H is either a separate
 * call (nvfp4_quantize) or fused, in mx_gemm_swiglu_nvfp4.
 */
mxq_status mx_gemm_swiglu(const mxq_operand* a, const mxq_operand* b, int64_t M, int64_t inter,
                          int64_t K, int64_t a_rows, uint16_t* h, int64_t ldh, int32_t num_groups,
                          const int32_t* group_row_offsets, const int32_t* a_row_index,
                          void* stream);

/*
 * mx_gemm_swiglu_nvfp4 -- the MoE gate_up GEMM with the SwiGLU and the
 * per-token NVFP4 requantization of H fused into its epilogue: the FP4
 * codes, E4M3 block scales and FP32 token scales that
 * nvfp4_quantize(H, ROW, PER_ROW, RNE) writes for H = mx_gemm_swiglu(...),
 * byte for byte, without H's trip through HBM; H itself too when h is given.
 * The pages describe the shared quantizer as one fused operation emitting
 * packed FP4, block scales and token scales ("Miles Blackwell RL Troca a
 * Uniformidade BF16 por MXFP8 e NVFP4 Nativos", section "Um Quantizador
 * Compartilhado É o Verdadeiro Mecanismo").
 *   a, b, M, inter, K, a_rows, num_groups, group_row_offsets, a_row_index
 *                 as for mx_gemm_swiglu
 *   codes         device, [M, inter / 2] bytes, row stride ld_codes (a
 *                 multiple of 16, rows 16-byte aligned), two codes a byte
 *                 (even column in the low nibble)
 *   block_scales  device, M * inter / 16 E4M3 bytes, in `layout` (LINEAR:
 *                 row-major [M, inter / 16]; MFMA: as nvfp4_quantize's MFMA
 *                 layout, M % 32 == 0)
 *   gscales       device, M floats: S of each token row (amax(H row) / 2688)
 *   h, ldh        optional BF16 H [M, inter] (NULL: not written)
 * Shapes: inter in {256, 512, 768} (a workgroup holds 32 whole rows of H),
 * K % 64 == 0.  Errors as for mx_gemm_swiglu; MXQ_EALIGN for misaligned
 * outputs.  Nothing is written on an error.
 */
mxq_status mx_gemm_swiglu_nvfp4(const mxq_operand* a, const mxq_operand* b, int64_t M, int64_t inter,
                                int64_t K, int64_t a_rows, uint8_t* codes, int64_t ld_codes,
                                uint8_t* block_scales, int32_t layout, float* gscales, uint16_t* h,
                                int64_t ldh, int32_t num_groups, const int32_t* group_row_offsets,
                                const int32_t* a_row_index, void* stream);

const char* mxq_status_str(mxq_status s);
const char* mxq_last_error(void);
int mxq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
