/*
 * mxgg.h -- C ABI of the grouped block-scaled (MX) GEMM library for MoE expert
 * layers on AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are the public pull-request pages this library is
 * built from; each is named by its title):
 *
 *  - "Triton mxfp4 (and a8w4) grouped GEMM kernel": a persistent grouped MXFP4
 *    GEMM in three passes -- forward (TN), input gradient (dgrad, NN) and
 *    variable-K weight gradient (wgrad, NT) -- fed by a row operand
 *    (data (N, K/2) + UE8M0 scales, one per 32 along K) and, for wgrad, a column operand
 *    whose expert segments are padded (the segment-padded layout below). The
 *    same page requires split validation: no negative split, one split per
 *    expert, splits summing to the row count of every row-split operand.
 *  - "route te.GroupedLinear through #723; a8w4 fwd-only": the a8w4 forward
 *    (E4M3 activations with UE8M0 block-32 scales x E2M1 weights), empty
 *    batches that launch nothing, caller-provided output buffers, and the
 *    tiny-scale rule (the shared exponent clamps at -127 and is applied before
 *    rounding).
 *  - "Grouped MXFP8 GEMMs with HipKittens": one launch over all experts with a
 *    binary-search (upper_bound) tile-to-expert lookup, at most 512 experts,
 *    contiguous packed expert weights.
 *  - "Add ROCm Triton blockwise FP8 grouped GEMM": the blockwise FP8 variant
 *    (1x128 activation scales, 128x128 weight scales, segment-padded 1x128
 *    column scales, power-of-two scales), variable-K wgrad with in-place
 *    accumulation, and the rule that every output element is owned by exactly
 *    one tile (no wrapped tail tiles).
 *
 * MX scale layout: block-major with a padded block stride. The UE8M0 scales
 * of an operand with R rows and B blocks of 32 along its contraction axis are
 * stored as u8 [B, R4], R4 = mxgg_mx_scale_stride(R) = R rounded up to a
 * multiple of 4: the scale of row r, block b is byte b*R4 + r; the padding
 * rows hold 0 as written by the quantizers and are never used (the page on
 * hipBLASLt MXFP4 support describes pre-arranged scale layouts; this one lets
 * a GEMM stage move the scales of four consecutive rows with one aligned
 * 4-byte load). Blockwise fp32 scales are row-major as listed below.
 *
 * Formats (OCP MX v1.0 and OCP FP8):
 *   MXGG_MXFP4        E2M1 elements, 2 per byte (even element in bits 3:0),
 *                     one UE8M0 scale byte per 32 elements along the
 *                     contraction axis (value 2^(byte-127)).
 *   MXGG_MXFP8        E4M3 ("FN", max 448) elements, one byte each, UE8M0
 *                     scale per 32 elements.
 *   MXGG_FP8_1x128    E4M3 elements, one fp32 scale per 128 elements along the
 *                     contraction axis (activations, wgrad column operands);
 *                     the scales block-major like MX ones: f32 [blocks, rows],
 *                     so a GEMM tile's rows of one block are one contiguous
 *                     run.
 *   MXGG_FP8_128x128  E4M3 elements, one fp32 scale per 128x128 block
 *                     (weights).
 *                     Blockwise E4M3 codes of an operand with L bytes per row
 *                     are stored in 64-byte blocks along the row, u8 [L/64,
 *                     rows, 64]: byte j of row r at ((j/64)*rows + r)*64 +
 *                     j%64, so the 64 bytes a GEMM stage needs from each of a
 *                     tile's rows are one contiguous run.
 *   MXGG_FP8_1x128_P2, MXGG_FP8_128x128_P2
 *                     The same layouts with every scale a power of two (what
 *                     the quantizers write with MXGG_POW2_SCALES; given to a
 *                     quantizer, these formats imply that flag). The GEMMs
 *                     then apply the scales inside the MFMA (the fp32
 *                     exponent field is a UE8M0 code) instead of scaling a
 *                     per-128 partial: exact for powers of two, while a scale
 *                     that is not one loses its mantissa. In the forward,
 *                     mixing a _P2 format with a general one selects the
 *                     general path; the input and weight gradients take one
 *                     format for both operands, where _P2 asserts both.
 *
 * MX quantization rule (what mxgg_quantize_* produce): amax = max |x| over the
 * block; e = clamp(floor(log2 amax) - emax, -127, 127) with emax = 2 (E2M1) or
 * 8 (E4M3), e = -127 for an all-zero block; codes = round-to-nearest-even of
 * x * 2^-e, saturating at +-6 / +-448, sign kept (so -0 stays -0); scale byte
 * = e + 127. Blockwise FP8 with MXGG_POW2_SCALES: amax floored at fp32(1e-4),
 * s = 2^-t with t the largest integer such that amax * 2^t <= 448, codes =
 * RNE-saturating E4M3 of x * 2^t; without the flag: q = fp32(448/amax),
 * codes from fp32(x*q), s = fp32(1/q).
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument except m_splits is a DEVICE pointer on the device
 *     that owns `stream` (NULL stream = the current device). m_splits is a
 *     HOST array of G int64 values, read only during the call.
 *   - bf16 tensors are row-major with a leading dimension (elements) and unit
 *     inner stride; quantized tensors are dense row-major (row stride = the
 *     row's byte count).
 *   - The caller owns every buffer, outputs included; the library allocates
 *     nothing per call and keeps no state beyond a cached per-device
 *     architecture check.
 *   - All work is enqueued on `stream` and is asynchronous: no host
 *     synchronization and no device-to-host copy happen inside a call.
 *   - Every argument check runs before anything is enqueued: an error return
 *     means nothing was launched or written. A batch with no rows is checked
 *     first and then returns MXGG_OK without a launch (except wgrad with
 *     accumulate == 0, which zero-fills its output).
 *   - Device pointers with a nonzero extent must be 16-byte aligned
 *     (MXGG_ERR_ALIGN), bf16 leading dimensions multiples of 8 elements.
 *   - Errors never abort and never throw; mxgg_last_error() returns a
 *     thread-local text for the last failing call on the calling thread.
 */
#ifndef MXGG_H
#define MXGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (the same declaration as the HIP runtime's). */
typedef struct ihipStream_t* hipStream_t;

typedef enum mxgg_status {
  MXGG_OK = 0,
  MXGG_ERR_NULL = 1,      /* a required pointer is NULL                        */
  MXGG_ERR_SHAPE = 2,     /* bad G, dimension, multiple or leading dimension   */
  MXGG_ERR_SPLITS = 3,    /* negative split or splits not summing to the rows  */
  MXGG_ERR_FORMAT = 4,    /* unsupported format or format pair for this pass   */
  MXGG_ERR_ALIGN = 5,     /* a device pointer / leading dimension misaligned   */
  MXGG_ERR_WORKSPACE = 6, /* workspace smaller than mxgg_workspace_size()      */
  MXGG_ERR_DEVICE = 7,    /* a pointer is not device memory of the stream's GPU */
  MXGG_ERR_ARCH = 8,      /* the stream's GPU is not gfx950                     */
  MXGG_ERR_HIP = 9        /* a HIP runtime call or kernel launch failed        */
} mxgg_status;

typedef enum mxgg_format {
  MXGG_MXFP4 = 0,
  MXGG_MXFP8 = 1,
  MXGG_FP8_1x128 = 2,
  MXGG_FP8_128x128 = 3,
  MXGG_FP8_1x128_P2 = 4,
  MXGG_FP8_128x128_P2 = 5
} mxgg_format;

/*
 * MX scale layouts. An MX format argument may carry the layout of the scales
 * it describes in its high bits: fmt = MXGG_MXFP4 | MXGG_LAYOUT_MFMA.
 * The layout is never inferred from shapes.
 *   MXGG_LAYOUT_BLOCK_MAJOR (0, what a plain format means): u8 [blocks, R4]
 *     (see "MX scale layout" above) -- what the quantizers write by default
 *     and every GEMM reads for every operand: a GEMM stage loads four rows of
 *     a block with one aligned 4-byte DMA.
 *   MXGG_LAYOUT_ROW_MAJOR: plain per-row scales, u8 [rows, blocks] (the
 *     un-arranged scale layout of the page "Integrate MXFP4 hipblaslt GEMM
 *     support"). The quantizers and GEMMs refuse it with MXGG_ERR_FORMAT; it
 *     is never read as another layout. mxgg_mx_scales_relayout converts it.
 *   MXGG_LAYOUT_MFMA: the pre-arranged layout of the scaled 32x32x64 MFMA
 *     (the page above compares plain scales with pre-swizzled ones packed in
 *     units of 32 rows by a run of blocks; this is such a packing, defined
 *     here). With R32 = rows rounded up to a multiple of 32 and blocks a
 *     multiple of 4, it is u8 [blocks/4, R32/32, 64, 2]: unit (g, u) holds
 *     rows 32u..32u+31 and blocks 4g..4g+3, and byte (g, u, L, j) is the
 *     scale of row 32u + L%32, block 4g + 2j + L/32 -- the two scale operands
 *     lane L of one 32-row MFMA fragment takes for the two 64-deep K steps of
 *     a 128-element chunk, side by side (padding rows 0). Total bytes:
 *     blocks * R32. Written by the quantizers (rows of cols % 128 == 0;
 *     column-wise only when every split is a multiple of 128, so each
 *     expert's segment starts a unit) and read for the weights' scales: the
 *     forward's w_s (N % 32 == 0, K % 128 == 0) and the input gradient's
 *     wcol_s (N % 128 == 0). Activation and gradient scales stay block-major
 *     (a_s, dy_s and both weight-gradient operands refuse it with
 *     MXGG_ERR_FORMAT).
 * Blockwise formats take no layout bits (their fp32 scales have one layout,
 * block-major for 1x128); any layout bits on them are MXGG_ERR_FORMAT.
 */
typedef enum mxgg_scale_layout {
  MXGG_LAYOUT_BLOCK_MAJOR = 0x000,
  MXGG_LAYOUT_ROW_MAJOR = 0x100,
  MXGG_LAYOUT_MFMA = 0x200
} mxgg_scale_layout;
#define MXGG_LAYOUT_MASK 0xF00

/*
 * MX code layouts, further bits of an MX format argument (beside the scale
 * layout): fmt = MXGG_MXFP4 | MXGG_KBLOCK_ROWS | MXGG_KBLOCK_COLS. Without
 * them the codes are plain rows. With them an operand with L code bytes per
 * row is stored in 64-byte blocks along the row, u8 [L/64, rows, 64]: byte j
 * of row r at ((j/64)*rows + r)*64 + j%64 (how every blockwise code tensor is
 * stored). A GEMM stage needs 64 bytes of each of a 256-row tile's rows per
 * operand (128 E2M1 or 64 E4M3 elements), which are then one contiguous run.
 *   MXGG_KBLOCK_ROWS  row-wise codes: mxgg_quantize_rowwise's q and the dual
 *                     quantizer's q_row (cols % 128 == 0); the forward's a_q
 *                     and w_q, the input gradient's dy_q.
 *   MXGG_KBLOCK_COLS  column-wise codes along the padded length, u8
 *                     [mpad_bytes/64, cols, 64]: mxgg_quantize_colwise_segpad's
 *                     q and the dual quantizer's q_col (every split a multiple
 *                     of 128, so each expert's segment starts a block); the
 *                     input gradient's wcol_q.
 * The forward takes MXGG_KBLOCK_ROWS on a_fmt and w_fmt together or on
 * neither; the input gradient both bits on fmt or neither; the weight gradient
 * neither (its MX segments are padded to 32, so a 64-byte stage row would
 * straddle blocks). A GEMM with K-blocked operands needs rows < 2^25 per
 * operand. Any other use of the bits is MXGG_ERR_FORMAT.
 */
#define MXGG_KBLOCK_ROWS 0x1000
#define MXGG_KBLOCK_COLS 0x2000
#define MXGG_KBLOCK_MASK 0x3000

/* flags for the quantizers (blockwise formats only) */
#define MXGG_POW2_SCALES 1u

/* largest expert count a single launch handles */
#define MXGG_MAX_EXPERTS 512

/*
 * Block stride, in bytes, of the block-major MX scales of an operand with
 * `rows` rows: rows rounded up to a multiple of 4 (0 for rows <= 0).
 */
int64_t mxgg_mx_scale_stride(int64_t rows);

/*
 * MX scales from one layout into another, on `stream`: any two different
 * layouts among row-major u8 [rows, blocks], block-major u8 [blocks,
 * mxgg_mx_scale_stride(rows)] and the MFMA layout u8 [blocks/4, R32/32, 64,
 * 2] (padding rows written as 0). For callers that hold plain per-row UE8M0
 * scales (the un-arranged layout the page "Integrate MXFP4 hipblaslt GEMM
 * support" compares with pre-arranged ones) and want a GEMM's layout, or back.
 *   src, dst   device buffers in src_layout / dst_layout; must not overlap.
 *   rows       rows of the operand (>= 0, < 2^31); blocks (> 0, <= 4194240):
 *              scale blocks of 32 along the contraction (cols / 32), a
 *              multiple of 4 when either side is MXGG_LAYOUT_MFMA.
 * Equal or unknown layouts are MXGG_ERR_FORMAT. rows == 0 returns MXGG_OK (no
 * launch). Errors: NULL, SHAPE, FORMAT, DEVICE, ARCH, HIP (no alignment
 * requirement: byte data).
 */
mxgg_status mxgg_mx_scales_relayout(const void* src, mxgg_scale_layout src_layout, int64_t rows,
                                    int64_t blocks, void* dst, mxgg_scale_layout dst_layout,
                                    hipStream_t stream);

/*
 * Row-wise quantization ("Triton mxfp4 (and a8w4) grouped GEMM kernel", the
 * row operand; blockwise formats from "Add ROCm Triton blockwise FP8 grouped
 * GEMM").
 *   x       bf16 [rows, cols], leading dimension ldx (elements, >= cols,
 *           multiple of 8).
 *   fmt     MXGG_MXFP4 / MXGG_MXFP8: blocks of 32 along cols (cols % 32 == 0),
 *           optionally | MXGG_LAYOUT_MFMA (cols % 128 == 0).
 *           MXGG_FP8_1x128: blocks of 128 along cols (cols % 128 == 0).
 *           MXGG_FP8_128x128: 128x128 blocks (rows % 128 == 0, cols % 128 == 0).
 *   flags   MXGG_POW2_SCALES for the blockwise formats (ignored for MX).
 *   q       MXFP4: u8 [rows, cols/2]; MXFP8: u8 [rows, cols]; blockwise: E4M3
 *           codes u8 [cols/64, rows, 64] (64-byte blocks along cols).
 *   scales  MX: u8 [cols/32, R4] (block-major, R4 = mxgg_mx_scale_stride(rows)),
 *           or with MXGG_LAYOUT_MFMA u8 [cols/128, R32/32, 64, 2];
 *           FP8_1x128: f32 [cols/128, rows] (block-major);
 *           FP8_128x128: f32 [rows/128, cols/128].
 * rows == 0 returns MXGG_OK with no launch. Errors: NULL, SHAPE, FORMAT,
 * ALIGN, DEVICE, ARCH, HIP.
 */
mxgg_status mxgg_quantize_rowwise(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                  mxgg_format fmt, uint32_t flags, void* q, void* scales,
                                  hipStream_t stream);

/*
 * Column-wise, segment-padded quantization (the padded column operand of the
 * variable-K weight gradient, "Triton mxfp4 (and a8w4) grouped GEMM kernel";
 * the 1x128 blockwise form from "Add ROCm Triton blockwise FP8 grouped GEMM").
 * The rows of expert g (m_splits[g] of them, consecutive) become columns
 * [pad_offs[g], pad_offs[g] + m_splits[g]) of a transposed [cols, mpad]
 * operand; each segment is padded with zeros to a multiple of P (P = 32 for
 * MX formats, 128 for MXGG_FP8_1x128) and quantized along its padded length,
 * so no scale block straddles two experts. Also used on weights for dgrad:
 * W viewed as [G*N, K] with m_splits = {N, ..., N} gives W quantized along N.
 *   x        bf16 [rows, cols], leading dimension ldx; rows == sum(m_splits).
 *   m_splits host int64 [G], 1 <= G <= 512, each >= 0.
 *   fmt      MXGG_MXFP4, MXGG_MXFP8 or MXGG_FP8_1x128; cols % 32 == 0. MX
 *            formats | MXGG_LAYOUT_MFMA need every split to be a multiple of
 *            128 (else MXGG_ERR_SPLITS).
 *   q        MXFP4: u8 [cols, mpad/2]; MXFP8: u8 [cols, mpad]; FP8_1x128: u8
 *            [mpad/64, cols, 64], 64-byte blocks along the padded length
 *            (byte p of column c at ((p/64)*cols + c)*64 + p%64: a weight-
 *            gradient stage reads each tile row's 64 bytes of one block as
 *            one contiguous run).
 *   scales   MX: u8 [mpad/32, cols] (block-major; cols % 32 == 0, so R4 == cols),
 *            or with MXGG_LAYOUT_MFMA u8 [mpad/128, cols/32, 64, 2];
 *            FP8_1x128: f32 [mpad/128, cols] (block-major).
 *   mpad     must equal mxgg_segpad_rows(m_splits, G, fmt).
 * Padding positions hold zero codes. rows == 0 returns MXGG_OK (no launch).
 * Errors: NULL, SHAPE, SPLITS, FORMAT, ALIGN, DEVICE, ARCH, HIP.
 */
mxgg_status mxgg_quantize_colwise_segpad(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                         const int64_t* m_splits, int32_t G, mxgg_format fmt,
                                         uint32_t flags, void* q, void* scales, int64_t mpad,
                                         hipStream_t stream);

/*
 * Dual-output quantization: the row-wise and the column-wise segment-padded
 * quantizations of one bf16 tensor from a single read of it (the "Changes"
 * list of "Add ROCm Triton blockwise FP8 grouped GEMM" describes one grouped
 * kernel emitting both training operands in one pass). Bit-identical to
 * mxgg_quantize_rowwise followed by mxgg_quantize_colwise_segpad on the same
 * arguments.
 *   x, rows, cols, ldx, m_splits, G, mpad  as for mxgg_quantize_colwise_segpad.
 *   fmt     MXGG_MXFP4, MXGG_MXFP8, or MXGG_FP8_1x128 / MXGG_FP8_1x128_P2
 *           (1x128 blocks along cols row-wise, along each expert's padded
 *           segment column-wise; cols % 128 == 0). An MX format may carry
 *           MXGG_LAYOUT_MFMA, which then applies to both scale outputs (the
 *           rules of the two quantizers above apply).
 *   flags   MXGG_POW2_SCALES for MXGG_FP8_1x128 (implied by the _P2 format);
 *           ignored for MX formats.
 *   q_row, s_row  the row-wise outputs, as mxgg_quantize_rowwise.
 *   q_col, s_col  the column-wise outputs, as mxgg_quantize_colwise_segpad.
 * Weights for dgrad (MX): W as [G*N, K] with m_splits = {N, ..., N} gives the
 * forward's W_q/W_s and dgrad's wcol_q/wcol_s together (in MXGG_LAYOUT_MFMA
 * too when N % 128 == 0 and K % 128 == 0).
 * rows == 0 returns MXGG_OK (no launch). Errors: NULL, SHAPE, SPLITS, FORMAT,
 * ALIGN, DEVICE, ARCH, HIP.
 */
mxgg_status mxgg_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                               const int64_t* m_splits, int32_t G, mxgg_format fmt,
                               uint32_t flags, void* q_row, void* s_row, void* q_col,
                               void* s_col, int64_t mpad, hipStream_t stream);

/*
 * 128x128-block FP8 weights transposed for the input gradient: the blocks are
 * square, so the transpose's 128x128 quantization is the same codes and the
 * same scale per block ("Add ROCm Triton blockwise FP8 grouped GEMM", weight
 * blocks used in both passes).
 *   w_q, w_s    from mxgg_quantize_rowwise(W as [G*N, K], MXGG_FP8_128x128):
 *               E4M3 u8 [K/64, G*N, 64] + f32 [G*N/128, K/128].
 *   wt_q, wt_s  written: E4M3 u8 [N/64, G*K, 64] (the [G*K, N] transpose in
 *               64-byte blocks along N; expert g's rows [g*K, (g+1)*K)) +
 *               f32 [G*K/128, N/128]. Caller-owned; must not overlap w.
 * N % 128 == 0, K % 128 == 0, N, K < 2^23, G in [1, 512].
 * Errors: NULL, SHAPE, ALIGN, DEVICE, ARCH, HIP.
 */
mxgg_status mxgg_transpose_128x128(const void* w_q, const void* w_s, int32_t G, int64_t N,
                                   int64_t K, void* wt_q, void* wt_s, hipStream_t stream);

/*
 * Grouped forward, TN: out[r, n] = sum_k A[r, k] * W_g[n, k] for every row r
 * of expert g (rows of expert g are consecutive, in expert order). One launch
 * covers every expert ("Triton mxfp4 (and a8w4) grouped GEMM kernel": the
 * persistent grouped MXFP4 forward over the row operand and the packed expert
 * weights; "route te.GroupedLinear through #723; a8w4 fwd-only": the a8w4
 * pair; "Add ROCm Triton blockwise FP8 grouped GEMM": the blockwise pair).
 *   a_q, a_s  A quantized row-wise along K: (MXFP4: u8 [M, K/2] | MXFP8: u8 [M, K])
 *             + u8 [K/32, mxgg_mx_scale_stride(M)]; or MXGG_FP8_1x128: u8
 *             [K/64, M, 64] + f32 [K/128, M] (M < 2^25).
 *   w_q, w_s  packed expert weights [G*N, K] quantized row-wise along K:
 *             MXFP4 u8 [G*N, K/2] + u8 [K/32, G*N], or with w_fmt =
 *             MXGG_MXFP4 | MXGG_LAYOUT_MFMA the scales u8 [K/128, G*N/32,
 *             64, 2] (K % 128 == 0); or MXGG_FP8_128x128: u8 [K/64, G*N, 64]
 *             + f32 [G*N/128, K/128] (G*N < 2^25).
 *   format pairs (a_fmt, w_fmt): (MXFP4, MXFP4) a4w4, (MXFP8, MXFP4) a8w4,
 *             (FP8_1x128, FP8_128x128) blockwise FP8. a_fmt takes no layout
 *             bits other than block-major.
 *   m_splits  host int64 [G]; sum == M.
 *   M, N, K   K % 32 == 0 and N % 32 == 0 (MX); K % 128 == 0 and N % 128 == 0
 *             (blockwise); M < 2^31; N, K < 2^23.
 *   out       bf16 [M, N] (dense), written with round-to-nearest-even.
 *   ws        workspace of at least mxgg_workspace_size(G) bytes (may be NULL
 *             when that is 0).
 * Errors: NULL, SHAPE, SPLITS, FORMAT, ALIGN, WORKSPACE, DEVICE, ARCH, HIP.
 */
mxgg_status mxgg_grouped_fwd(const void* a_q, const void* a_s, mxgg_format a_fmt,
                             const void* w_q, const void* w_s, mxgg_format w_fmt,
                             const int64_t* m_splits, int32_t G, int64_t M, int64_t N,
                             int64_t K, void* out, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * Grouped input gradient, NN: dx[r, k] = sum_n dY[r, n] * W_g[n, k]
 * (the backward of the expert layers on "Triton mxfp4 (and a8w4) grouped GEMM
 * kernel" and, for the blockwise formats, "Add ROCm Triton blockwise FP8
 * grouped GEMM", whose 128x128 weight blocks serve both orientations).
 *   fmt            dY's format, which fixes the weights':
 *                  MXGG_MXFP4 (a4w4) and MXGG_MXFP8 (a8w4): W in MXFP4;
 *                  MXGG_FP8_1x128 / _P2: W as transposed 128x128 blocks.
 *                  MXGG_LAYOUT_MFMA on an MX fmt says that wcol_s is in the
 *                  MFMA layout, u8 [G*N/128, K/32, 64, 2] (N % 128 == 0);
 *                  dy_s stays block-major.
 *   dy_q, dy_s     dY quantized row-wise along N: MX, u8 [M, N/2] (E2M1) or
 *                  [M, N] (E4M3) + u8 [N/32, mxgg_mx_scale_stride(M)];
 *                  blockwise, E4M3 u8 [N/64, M, 64] + f32 [N/128, M] (M < 2^25).
 *   wcol_q, wcol_s MX: W quantized along N with mxgg_quantize_colwise_segpad
 *                  on W as [G*N, K] with splits {N, ..., N}: u8 [K, G*N/2] +
 *                  u8 [G*N/32, K] (expert g owns columns [g*N, (g+1)*N) and
 *                  scale blocks [g*N/32, (g+1)*N/32)).
 *                  Blockwise: W^T from mxgg_transpose_128x128, E4M3 u8
 *                  [N/64, G*K, 64] + f32 [G*K/128, N/128] (G*K < 2^25).
 *                  MXGG_FP8_1x128_P2
 *                  asserts that the scales of BOTH operands (dY's and the
 *                  transposed weights') are powers of two, and the MFMA then
 *                  applies them (a non-power-of-two scale would lose its
 *                  mantissa); pass MXGG_FP8_1x128 when either is general.
 *   dx             bf16 [M, K].
 * Shape rules as for the forward, and (MX) G*N/2 < 2^23. Errors as for the
 * forward.
 */
mxgg_status mxgg_grouped_dgrad(const void* dy_q, const void* dy_s, const void* wcol_q,
                               const void* wcol_s, mxgg_format fmt, const int64_t* m_splits,
                               int32_t G, int64_t M, int64_t N, int64_t K, void* dx,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped variable-K weight gradient, NT: dW_g[n, k] = sum over the tokens t of
 * expert g of dY[t, n] * X[t, k], contracted over the expert's padded segment
 * (pad positions are zero codes, so they add nothing). One launch covers every
 * expert, each with its own contraction length ("Triton mxfp4 (and a8w4)
 * grouped GEMM kernel": the variable-K wgrad over the segment-padded column
 * operands; "Add ROCm Triton blockwise FP8 grouped GEMM": its blockwise form
 * and the in-place accumulation into the weight's main_grad).
 *   dycol_q/_s  dY from mxgg_quantize_colwise_segpad: [N, mpad] operand
 *               (MX scales u8 [mpad/32, N]; 1x128 codes u8 [mpad/64, N, 64]
 *               and scales f32 [mpad/128, N]).
 *   xcol_q/_s   X from mxgg_quantize_colwise_segpad: [K, mpad] operand
 *               (MX scales u8 [mpad/32, K]; 1x128 codes u8 [mpad/64, K, 64]
 *               and scales f32 [mpad/128, K]).
 *   fmt         MXGG_MXFP4 or MXGG_MXFP8 (both operands in that format: the
 *               a4w4 and a8w4 weight gradients; pad 32; block-major scales
 *               only), or MXGG_FP8_1x128
 *               (pad 128). MXGG_FP8_1x128_P2 asserts that the scales of BOTH
 *               operands are powers of two (the MFMA then applies them and a
 *               non-power-of-two scale would lose its mantissa); pass
 *               MXGG_FP8_1x128 when either operand's scales are general.
 *   mpad        mxgg_segpad_rows(m_splits, G, fmt).
 *   main_grad   [G, N, K]: fp32 when out_is_bf16 == 0, else bf16 (blockwise
 *               formats only; an MX format with out_is_bf16 = 1 is
 *               MXGG_ERR_FORMAT).
 *   accumulate  1: main_grad[g] += dW_g in place (experts with no tokens are
 *               left untouched); 0: main_grad[g] = dW_g (experts with no
 *               tokens are zero-filled). Every element is read/written by
 *               exactly one thread, so in-place accumulation is race-free.
 * Shape rules: N % 32 == 0 and K % 32 == 0 (MX), % 128 (blockwise); N, K and
 * mpad < 2^23.
 * Errors: NULL, SHAPE, SPLITS, FORMAT, ALIGN, WORKSPACE, DEVICE, ARCH, HIP.
 */
mxgg_status mxgg_grouped_wgrad(const void* dycol_q, const void* dycol_s, const void* xcol_q,
                               const void* xcol_s, mxgg_format fmt, const int64_t* m_splits,
                               int32_t G, int64_t N, int64_t K, int64_t mpad, void* main_grad,
                               int32_t out_is_bf16, int32_t accumulate, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* Workspace bytes the GEMM entry points need for G experts (0 today: the
 * per-expert tables travel as kernel arguments and are rebuilt in LDS). */
size_t mxgg_workspace_size(int32_t G);

/* Padded row count of the segment-padded operand: sum_g ceil(m_g/P)*P with
 * P = 32 (MX formats, any scale layout bits) or 128 (MXGG_FP8_1x128). Returns
 * -1 for invalid input (NULL, G outside [1, 512], a negative split or one of
 * 2^31 or more, other formats). */
int64_t mxgg_segpad_rows(const int64_t* m_splits, int32_t G, mxgg_format fmt);

/* Static text for a status code. */
const char* mxgg_status_string(mxgg_status status);

/* Thread-local description of the last error returned on this thread
 * ("" when the last call succeeded). Valid until the next call on the thread. */
const char* mxgg_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXGG_H */
