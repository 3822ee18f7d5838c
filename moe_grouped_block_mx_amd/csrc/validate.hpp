// Host-side argument validation of the C ABI. Pure C++ (no HIP calls), so
// every rule can be exercised on a machine without a GPU.
//
// Split rules follow the review of "Triton mxfp4 (and a8w4) grouped GEMM
// kernel": splits are non-negative, there is one per expert, and they sum to
// the row count of every row-split operand (unchecked offsets read or write out
// of bounds, or leave part of a gradient unwritten). Empty experts are allowed.
// The expert limit (512) and the rejection of unsupported shapes with a
// status the caller can fall back on follow "Grouped MXFP8 GEMMs with
// HipKittens"; validating before the empty-batch early return follows
// "route te.GroupedLinear through #723; a8w4 fwd-only".
#pragma once
#include <stdint.h>

#include <cstdio>
#include <string>

#include "../../include/mxgg.h"

namespace mxgg {

struct Check {
  mxgg_status st = MXGG_OK;
  std::string msg;
  bool ok() const { return st == MXGG_OK; }
};

inline Check fail(mxgg_status st, const char* fmt, long long a = 0, long long b = 0, long long c = 0) {
  Check r;
  r.st = st;
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, a, b, c);
  r.msg = buf;
  return r;
}

inline bool is_mx(mxgg_format f) { return f == MXGG_MXFP4 || f == MXGG_MXFP8; }
inline bool valid_format(int f) { return f >= MXGG_MXFP4 && f <= MXGG_FP8_128x128_P2; }

// A format argument with layout bits: the scales it describes are not
// block-major. Each entry point accepts the MFMA layout where it reads or
// writes it and refuses every other layout by name, so a caller's scales are
// never read in a layout they are not in.
inline bool has_layout_bits(int f) { return (f & ~0xFF) != 0; }
inline int layout_bits(int f) { return f & MXGG_LAYOUT_MASK; }   // the scales' layout
inline int kblock_bits(int f) { return f & MXGG_KBLOCK_MASK; }   // the codes' layout
inline int format_bits(int f) { return f & 0xFF; }
inline bool is_mfma_layout(int f) { return layout_bits(f) == MXGG_LAYOUT_MFMA; }
// The power-of-two blockwise formats share their base format's layout.
inline bool is_p2(int f) { return f == MXGG_FP8_1x128_P2 || f == MXGG_FP8_128x128_P2; }
inline int base_format(int f) {
  return f == MXGG_FP8_1x128_P2 ? MXGG_FP8_1x128 : f == MXGG_FP8_128x128_P2 ? MXGG_FP8_128x128 : f;
}

// Segment pad multiple of the column-wise operand of a format.
inline int segpad_multiple(mxgg_format f) { return base_format(f) == MXGG_FP8_1x128 ? 128 : 32; }

// Splits: pointer, count, non-negativity and sum.
inline Check check_splits(const int64_t* m, int32_t G, int64_t rows, const char* what) {
  if (G < 1 || G > MXGG_MAX_EXPERTS) return fail(MXGG_ERR_SHAPE, "G=%lld outside [1, 512]", G);
  if (!m) return fail(MXGG_ERR_NULL, "m_splits is NULL");
  // Each split is bounded before it is added (a split above the row count
  // can never be part of a valid sum), so the int64 running sum cannot wrap:
  // huge splits must not add up, modulo 2^64, to the right total.
  for (int32_t g = 0; g < G; ++g)
    if (m[g] < 0) return fail(MXGG_ERR_SPLITS, "m_splits[%lld] = %lld is negative", g, m[g]);
  int64_t sum = 0;
  for (int32_t g = 0; g < G; ++g) {
    if (m[g] > rows) return fail(MXGG_ERR_SPLITS, "m_splits[%lld] = %lld exceeds the %lld rows", g, m[g], rows);
    if (__builtin_add_overflow(sum, m[g], &sum)) return fail(MXGG_ERR_SPLITS, "m_splits sum overflows");
  }
  if (sum != rows) {
    Check r = fail(MXGG_ERR_SPLITS, "sum(m_splits) = %lld but %s has %lld rows", sum, 0, rows);
    r.msg = "sum(m_splits) = " + std::to_string(sum) + " but " + what + " has " + std::to_string(rows) + " rows";
    return r;
  }
  return Check{};
}

// Largest split any entry point accepts: row counts stay below 2^31.
constexpr int64_t kMaxSplit = ((int64_t)1 << 31) - 1;

// Padded row count; callers have checked 0 <= m[g] <= kMaxSplit, so neither
// the rounding nor the sum (at most 512 terms) can overflow.
// mfma_ok: the operand's MX scales may be in the MFMA layout; kblock_ok: the
// code-layout bits the entry point takes for this argument.
inline Check check_layout(int f, const char* what, bool mfma_ok = false, int kblock_ok = 0) {
  if (!has_layout_bits(f)) return Check{};
  const bool mx = is_mx((mxgg_format)format_bits(f));
  if ((f & ~(0xFF | MXGG_LAYOUT_MASK | MXGG_KBLOCK_MASK)) != 0)
    return fail(MXGG_ERR_FORMAT, "format 0x%llx: unknown bits", f);
  if (kblock_bits(f)) {
    if (!mx || (kblock_bits(f) & ~kblock_ok)) {
      Check r;
      r.st = MXGG_ERR_FORMAT;
      r.msg = std::string(what) + ": these 64-byte K-block code bits are not taken here (MX formats only: "
              "MXGG_KBLOCK_ROWS for row-wise codes, MXGG_KBLOCK_COLS for column-wise codes)";
      return r;
    }
  }
  const int lay = layout_bits(f);
  if (lay == MXGG_LAYOUT_BLOCK_MAJOR) return Check{};
  if (mx && lay == MXGG_LAYOUT_MFMA) {
    if (mfma_ok) return Check{};
    Check r;
    r.st = MXGG_ERR_FORMAT;
    r.msg = std::string(what) + ": MFMA-layout scales are read only for the weights (the forward's w_s and "
            "the input gradient's wcol_s); this operand's scales must be block-major";
    return r;
  }
  if (mx && lay == MXGG_LAYOUT_ROW_MAJOR) {
    Check r;
    r.st = MXGG_ERR_FORMAT;
    r.msg = std::string(what) + ": row-major MX scales are not accepted (the kernels read block-major or "
            "MFMA-layout scales); convert them with mxgg_mx_scales_relayout";
    return r;
  }
  return fail(MXGG_ERR_FORMAT, "format 0x%llx: unknown layout bits or a layout on a blockwise format", f);
}

// MFMA-layout column scales and K-blocked column codes: every expert segment
// starts a 128-element unit.
inline Check check_mfma_splits(const int64_t* m, int32_t G, const char* what,
                               const char* why = "MFMA-layout column scales") {
  for (int32_t g = 0; g < G; ++g)
    if (m[g] % 128) {
      Check r = fail(MXGG_ERR_SPLITS, "m_splits[%lld] = %lld is not a multiple of 128", g, m[g]);
      r.msg = std::string(what) + ": " + why + " need every split a multiple of 128; " + r.msg;
      return r;
    }
  return Check{};
}

inline int64_t segpad_rows(const int64_t* m, int32_t G, int pad) {
  int64_t s = 0;
  for (int32_t g = 0; g < G; ++g) s += (m[g] + pad - 1) / pad * pad;
  return s;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A pointer that must be non-NULL and 16-byte aligned when the extent is
// nonzero.
inline Check check_ptr(const void* p, bool nonzero, const char* name) {
  if (!nonzero) return Check{};
  if (!p) {
    Check r; r.st = MXGG_ERR_NULL; r.msg = std::string(name) + " is NULL"; return r;
  }
  if (!aligned16(p)) {
    Check r; r.st = MXGG_ERR_ALIGN; r.msg = std::string(name) + " is not 16-byte aligned"; return r;
  }
  return Check{};
}

#define MXGG_TRY(expr)          \
  do {                          \
    ::mxgg::Check c_ = (expr);  \
    if (!c_.ok()) return c_;    \
  } while (0)

// --- per entry point -------------------------------------------------------

inline Check validate_quantize_rowwise(const void* x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                       const void* q, const void* scales) {
  MXGG_TRY(check_layout(fmt, "quantize_rowwise", true, MXGG_KBLOCK_ROWS));
  const bool mfma = is_mfma_layout(fmt), kb = kblock_bits(fmt) != 0;
  fmt = format_bits(fmt);
  if (!valid_format(fmt)) return fail(MXGG_ERR_FORMAT, "unknown format %lld", fmt);
  if (mfma && cols % 128) return fail(MXGG_ERR_SHAPE, "cols=%lld: MFMA-layout scales need cols %% 128 == 0", cols);
  if (kb && cols % 128) return fail(MXGG_ERR_SHAPE, "cols=%lld: K-blocked codes need cols %% 128 == 0", cols);
  if (rows < 0 || cols <= 0) return fail(MXGG_ERR_SHAPE, "rows=%lld cols=%lld", rows, cols);
  const mxgg_format f = (mxgg_format)fmt;
  const int blk = is_mx(f) ? 32 : 128;
  if (cols % blk) return fail(MXGG_ERR_SHAPE, "cols=%lld is not a multiple of %lld", cols, blk);
  if (f == MXGG_FP8_128x128 && rows % 128) return fail(MXGG_ERR_SHAPE, "rows=%lld not a multiple of 128", rows);
  if (ldx < cols) return fail(MXGG_ERR_SHAPE, "ldx=%lld < cols=%lld", ldx, cols);
  if (ldx % 8) return fail(MXGG_ERR_ALIGN, "ldx=%lld not a multiple of 8 elements", ldx);
  if (rows >= ((int64_t)1 << 31)) return fail(MXGG_ERR_SHAPE, "rows=%lld >= 2^31", rows);
  // one 128x128 block per workgroup, block rows on the grid's y axis
  if (f == MXGG_FP8_128x128 && rows / 128 > 65535)
    return fail(MXGG_ERR_SHAPE, "rows=%lld too large for 128x128 blocks (<= 65535 block rows)", rows);
  const bool nz = rows > 0;
  MXGG_TRY(check_ptr(x, nz, "x"));
  MXGG_TRY(check_ptr(q, nz, "q"));
  MXGG_TRY(check_ptr(scales, nz, "scales"));
  return Check{};
}

inline Check validate_quantize_colwise(const void* x, int64_t rows, int64_t cols, int64_t ldx, const int64_t* m,
                                       int32_t G, int fmt, const void* q, const void* scales, int64_t mpad) {
  MXGG_TRY(check_layout(fmt, "quantize_colwise", true, MXGG_KBLOCK_COLS));
  const bool mfma = is_mfma_layout(fmt), kb = kblock_bits(fmt) != 0;
  fmt = format_bits(fmt);
  if (!valid_format(fmt)) return fail(MXGG_ERR_FORMAT, "unknown format %lld", fmt);
  const mxgg_format f = (mxgg_format)fmt;
  if (f == MXGG_FP8_128x128) return fail(MXGG_ERR_FORMAT, "128x128 blocks have no column-wise form");
  if (rows < 0 || cols <= 0) return fail(MXGG_ERR_SHAPE, "rows=%lld cols=%lld", rows, cols);
  const int blk = is_mx(f) ? 32 : 128;
  if (cols % 32) return fail(MXGG_ERR_SHAPE, "cols=%lld is not a multiple of 32", cols);
  (void)blk;
  // 64 columns per workgroup on the grid's y axis
  if ((cols + 63) / 64 > 65535) return fail(MXGG_ERR_SHAPE, "cols=%lld too large (<= 4194240)", cols);
  if (ldx < cols) return fail(MXGG_ERR_SHAPE, "ldx=%lld < cols=%lld", ldx, cols);
  if (ldx % 8) return fail(MXGG_ERR_ALIGN, "ldx=%lld not a multiple of 8 elements", ldx);
  if (rows >= ((int64_t)1 << 31)) return fail(MXGG_ERR_SHAPE, "rows=%lld >= 2^31", rows);
  MXGG_TRY(check_splits(m, G, rows, "x"));
  if (mfma) MXGG_TRY(check_mfma_splits(m, G, "quantize_colwise"));
  if (kb) MXGG_TRY(check_mfma_splits(m, G, "quantize_colwise", "K-blocked column codes"));
  const int64_t need = segpad_rows(m, G, segpad_multiple(f));
  if (mpad != need) return fail(MXGG_ERR_SHAPE, "mpad=%lld but the padded row count is %lld", mpad, need);
  if (mpad >= ((int64_t)1 << 31)) return fail(MXGG_ERR_SHAPE, "mpad=%lld >= 2^31", mpad);
  const bool nz = rows > 0;
  MXGG_TRY(check_ptr(x, nz, "x"));
  MXGG_TRY(check_ptr(q, nz, "q"));
  MXGG_TRY(check_ptr(scales, nz, "scales"));
  return Check{};
}

inline Check validate_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, const int64_t* m,
                                    int32_t G, int fmt, const void* q_row, const void* s_row, const void* q_col,
                                    const void* s_col, int64_t mpad) {
  MXGG_TRY(check_layout(fmt, "quantize_dual", true, MXGG_KBLOCK_MASK));
  const int f0 = format_bits(fmt);
  if (!valid_format(f0)) return fail(MXGG_ERR_FORMAT, "unknown format %lld", fmt);
  if (!is_mx((mxgg_format)f0) && f0 != MXGG_FP8_1x128)
    return fail(MXGG_ERR_FORMAT, "the dual quantizer takes MX formats and MXGG_FP8_1x128 (got %lld)", fmt);
  // each output takes its own code-layout bit
  MXGG_TRY(validate_quantize_rowwise(x, rows, cols, ldx, fmt & ~MXGG_KBLOCK_COLS, q_row, s_row));
  MXGG_TRY(validate_quantize_colwise(x, rows, cols, ldx, m, G, fmt & ~MXGG_KBLOCK_ROWS, q_col, s_col, mpad));
  return Check{};
}

// The GEMM kernels address a 256-row tile with 32-bit byte offsets, so every
// operand row stride is kept below 2^23 bytes (tile span < 2^31).
constexpr int64_t kMaxRowStride = (int64_t)1 << 23;

// Blockwise codes sit in 64-byte K blocks of rows*64 bytes, and a GEMM
// lane's 32-bit DMA offset spans up to two blocks: rows < 2^25.
constexpr int64_t kMaxKBlockRows = (int64_t)1 << 25;

inline Check validate_gemm_dims(int64_t M, int64_t N, int64_t K, int blk) {
  if (M < 0 || N <= 0 || K <= 0) return fail(MXGG_ERR_SHAPE, "M=%lld N=%lld K=%lld", M, N, K);
  if (N % blk || K % blk) return fail(MXGG_ERR_SHAPE, "N=%lld and K=%lld must be multiples of %lld", N, K, blk);
  if (M >= ((int64_t)1 << 31) || N >= kMaxRowStride || K >= kMaxRowStride)
    return fail(MXGG_ERR_SHAPE, "M=%lld N=%lld K=%lld too large (N, K < 2^23)", M, N, K);
  return Check{};
}

inline Check validate_fwd(const void* a_q, const void* a_s, int a_fmt, const void* w_q, const void* w_s, int w_fmt,
                          const int64_t* m, int32_t G, int64_t M, int64_t N, int64_t K, const void* out,
                          const void* ws, size_t ws_bytes, size_t ws_need) {
  MXGG_TRY(check_layout(a_fmt, "fwd A", false, MXGG_KBLOCK_ROWS));
  MXGG_TRY(check_layout(w_fmt, "fwd W", true, MXGG_KBLOCK_ROWS));
  const bool w_mfma = is_mfma_layout(w_fmt);
  const bool kb = kblock_bits(a_fmt) != 0;
  if (kb != (kblock_bits(w_fmt) != 0))
    return fail(MXGG_ERR_FORMAT, "fwd: a_fmt and w_fmt carry MXGG_KBLOCK_ROWS together or not at all");
  a_fmt = format_bits(a_fmt);
  w_fmt = format_bits(w_fmt);
  if (!valid_format(a_fmt) || !valid_format(w_fmt)) return fail(MXGG_ERR_FORMAT, "unknown format");
  if (w_mfma && K % 128) return fail(MXGG_ERR_SHAPE, "K=%lld: MFMA-layout weight scales need K %% 128 == 0", K);
  if (kb && K % 128) return fail(MXGG_ERR_SHAPE, "K=%lld: K-blocked codes need K %% 128 == 0", K);
  if (kb && (M >= kMaxKBlockRows || (int64_t)G * N >= kMaxKBlockRows))
    return fail(MXGG_ERR_SHAPE, "K-blocked codes: M=%lld and G*N=%lld must stay below 2^25", M, (int64_t)G * N);
  const bool a4w4 = a_fmt == MXGG_MXFP4 && w_fmt == MXGG_MXFP4;
  const bool a8w4 = a_fmt == MXGG_MXFP8 && w_fmt == MXGG_MXFP4;
  const bool blk = a_fmt == MXGG_FP8_1x128 && w_fmt == MXGG_FP8_128x128;
  if (!(a4w4 || a8w4 || blk))
    return fail(MXGG_ERR_FORMAT, "format pair (%lld, %lld) is not supported by the forward", a_fmt, w_fmt);
  MXGG_TRY(validate_gemm_dims(M, N, K, blk ? 128 : 32));
  if (blk && (M >= kMaxKBlockRows || (int64_t)G * N >= kMaxKBlockRows))
    return fail(MXGG_ERR_SHAPE, "blockwise: M=%lld and G*N=%lld must stay below 2^25", M, (int64_t)G * N);
  MXGG_TRY(check_splits(m, G, M, "A"));
  if (ws_bytes < ws_need) return fail(MXGG_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes,
                                      (long long)ws_need);
  if (ws_need) MXGG_TRY(check_ptr(ws, true, "ws"));
  const bool nz = M > 0;
  MXGG_TRY(check_ptr(a_q, nz, "a_q"));
  MXGG_TRY(check_ptr(a_s, nz, "a_s"));
  MXGG_TRY(check_ptr(w_q, nz, "w_q"));
  MXGG_TRY(check_ptr(w_s, nz, "w_s"));
  MXGG_TRY(check_ptr(out, nz, "out"));
  return Check{};
}

inline Check validate_dgrad(const void* dy_q, const void* dy_s, const void* wc_q, const void* wc_s, int fmt,
                            const int64_t* m, int32_t G, int64_t M, int64_t N, int64_t K, const void* dx,
                            const void* ws, size_t ws_bytes, size_t ws_need) {
  MXGG_TRY(check_layout(fmt, "dgrad", true, MXGG_KBLOCK_MASK));
  const bool w_mfma = is_mfma_layout(fmt);
  const int kbits = kblock_bits(fmt);
  if (kbits != 0 && kbits != MXGG_KBLOCK_MASK)
    return fail(MXGG_ERR_FORMAT, "dgrad: fmt carries MXGG_KBLOCK_ROWS and MXGG_KBLOCK_COLS together or neither");
  fmt = format_bits(fmt);
  if (!valid_format(fmt)) return fail(MXGG_ERR_FORMAT, "unknown format %lld", fmt);
  if (w_mfma && N % 128) return fail(MXGG_ERR_SHAPE, "N=%lld: MFMA-layout weight scales need N %% 128 == 0", N);
  if (kbits && N % 128) return fail(MXGG_ERR_SHAPE, "N=%lld: K-blocked codes need N %% 128 == 0", N);
  if (kbits && (M >= kMaxKBlockRows || K >= kMaxKBlockRows))
    return fail(MXGG_ERR_SHAPE, "K-blocked codes: M=%lld and K=%lld must stay below 2^25", M, K);
  // fmt is dY's format: MXFP4 (a4w4) or MXFP8 (a8w4) with W column-wise in
  // MXFP4; FP8_1x128 with the transposed 128x128 weight blocks
  if (fmt != MXGG_MXFP4 && fmt != MXGG_MXFP8 && fmt != MXGG_FP8_1x128)
    return fail(MXGG_ERR_FORMAT, "dgrad supports MXGG_MXFP4, MXGG_MXFP8 and MXGG_FP8_1x128 (got %lld)", fmt);
  const bool blk = fmt == MXGG_FP8_1x128;
  MXGG_TRY(validate_gemm_dims(M, N, K, blk ? 128 : 32));
  if (blk && (M >= kMaxKBlockRows || (int64_t)G * K >= kMaxKBlockRows))
    return fail(MXGG_ERR_SHAPE, "blockwise: M=%lld and G*K=%lld must stay below 2^25", M, (int64_t)G * K);
  MXGG_TRY(check_splits(m, G, M, "dY"));
  if (!blk && (int64_t)G * N / 2 >= kMaxRowStride)
    return fail(MXGG_ERR_SHAPE, "G*N=%lld too large (G*N/2 < 2^23)", (int64_t)G * N);
  if (ws_bytes < ws_need) return fail(MXGG_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes,
                                      (long long)ws_need);
  if (ws_need) MXGG_TRY(check_ptr(ws, true, "ws"));
  const bool nz = M > 0;
  MXGG_TRY(check_ptr(dy_q, nz, "dy_q"));
  MXGG_TRY(check_ptr(dy_s, nz, "dy_s"));
  MXGG_TRY(check_ptr(wc_q, nz, "wcol_q"));
  MXGG_TRY(check_ptr(wc_s, nz, "wcol_s"));
  MXGG_TRY(check_ptr(dx, nz, "dx"));
  return Check{};
}

// 128x128-block weight transpose: w [G*N, K] codes + f32 [G*N/128, K/128]
// scales -> [G*K, N] + [G*K/128, N/128].
inline Check validate_transpose_128x128(const void* w_q, const void* w_s, int32_t G, int64_t N, int64_t K,
                                        const void* wt_q, const void* wt_s) {
  if (G < 1 || G > MXGG_MAX_EXPERTS) return fail(MXGG_ERR_SHAPE, "G=%lld outside [1, 512]", G);
  if (N <= 0 || K <= 0 || N % 128 || K % 128)
    return fail(MXGG_ERR_SHAPE, "N=%lld and K=%lld must be positive multiples of 128", N, K);
  if (N >= kMaxRowStride || K >= kMaxRowStride) return fail(MXGG_ERR_SHAPE, "N or K too large (< 2^23)");
  MXGG_TRY(check_ptr(w_q, true, "w_q"));
  MXGG_TRY(check_ptr(w_s, true, "w_s"));
  MXGG_TRY(check_ptr(wt_q, true, "wt_q"));
  MXGG_TRY(check_ptr(wt_s, true, "wt_s"));
  return Check{};
}

inline Check validate_wgrad(const void* dy_q, const void* dy_s, const void* x_q, const void* x_s, int fmt,
                            const int64_t* m, int32_t G, int64_t N, int64_t K, int64_t mpad, const void* main_grad,
                            int32_t out_is_bf16, int32_t accumulate, const void* ws, size_t ws_bytes,
                            size_t ws_need) {
  MXGG_TRY(check_layout(fmt, "wgrad"));
  if (!valid_format(fmt)) return fail(MXGG_ERR_FORMAT, "unknown format %lld", fmt);
  if (fmt != MXGG_MXFP4 && fmt != MXGG_MXFP8 && fmt != MXGG_FP8_1x128)
    return fail(MXGG_ERR_FORMAT, "wgrad supports MXGG_MXFP4, MXGG_MXFP8 and MXGG_FP8_1x128 (got %lld)", fmt);
  if (out_is_bf16 != 0 && out_is_bf16 != 1) return fail(MXGG_ERR_SHAPE, "out_is_bf16=%lld", out_is_bf16);
  // bf16 output is the blockwise workload's; the MX weight gradient writes
  // the fp32 main_grad it accumulates into (its 256x256 bf16 epilogue is not
  // covered by the GPU tests)
  if (fmt != MXGG_FP8_1x128 && out_is_bf16) return fail(MXGG_ERR_FORMAT, "MX wgrad writes fp32 main_grad only");
  if (accumulate != 0 && accumulate != 1) return fail(MXGG_ERR_SHAPE, "accumulate=%lld", accumulate);
  const mxgg_format f = (mxgg_format)fmt;
  const int blk = f == MXGG_FP8_1x128 ? 128 : 32;
  if (N <= 0 || K <= 0 || N % blk || K % blk)
    return fail(MXGG_ERR_SHAPE, "N=%lld and K=%lld must be positive multiples of %lld", N, K, blk);
  if (N >= kMaxRowStride || K >= kMaxRowStride) return fail(MXGG_ERR_SHAPE, "N or K too large (< 2^23)");
  if (G < 1 || G > MXGG_MAX_EXPERTS) return fail(MXGG_ERR_SHAPE, "G=%lld outside [1, 512]", G);
  if (!m) return fail(MXGG_ERR_NULL, "m_splits is NULL");
  int64_t rows = 0;  // at most 512 splits below 2^31 each: no overflow
  for (int32_t g = 0; g < G; ++g) {
    if (m[g] < 0) return fail(MXGG_ERR_SPLITS, "m_splits[%lld] = %lld is negative", g, m[g]);
    if (m[g] > kMaxSplit) return fail(MXGG_ERR_SPLITS, "m_splits[%lld] = %lld >= 2^31", g, m[g]);
    rows += m[g];
  }
  if (rows >= ((int64_t)1 << 31)) return fail(MXGG_ERR_SPLITS, "sum(m_splits)=%lld >= 2^31", rows);
  const int64_t need = segpad_rows(m, G, segpad_multiple(f));
  if (mpad != need) return fail(MXGG_ERR_SHAPE, "mpad=%lld but the padded row count is %lld", mpad, need);
  if (mpad >= kMaxRowStride) return fail(MXGG_ERR_SHAPE, "mpad=%lld too large (< 2^23)", mpad);
  if (ws_bytes < ws_need) return fail(MXGG_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes,
                                      (long long)ws_need);
  if (ws_need) MXGG_TRY(check_ptr(ws, true, "ws"));
  const bool nz = mpad > 0;
  MXGG_TRY(check_ptr(dy_q, nz, "dycol_q"));
  MXGG_TRY(check_ptr(dy_s, nz, "dycol_s"));
  MXGG_TRY(check_ptr(x_q, nz, "xcol_q"));
  MXGG_TRY(check_ptr(x_s, nz, "xcol_s"));
  MXGG_TRY(check_ptr(main_grad, true, "main_grad"));
  return Check{};
}

// Scale relayout between any two of the MX scale layouts.
inline bool known_layout(int l) {
  return l == MXGG_LAYOUT_ROW_MAJOR || l == MXGG_LAYOUT_BLOCK_MAJOR || l == MXGG_LAYOUT_MFMA;
}
inline Check validate_relayout(const void* src, int src_layout, int64_t rows, int64_t blocks, const void* dst,
                               int dst_layout) {
  if (!known_layout(src_layout) || !known_layout(dst_layout) || src_layout == dst_layout)
    return fail(MXGG_ERR_FORMAT, "relayout from 0x%llx to 0x%llx: need two different known layouts", src_layout,
                dst_layout);
  if ((src_layout == MXGG_LAYOUT_MFMA || dst_layout == MXGG_LAYOUT_MFMA) && blocks % 4)
    return fail(MXGG_ERR_SHAPE, "blocks=%lld: the MFMA layout needs a multiple of 4 blocks", blocks);
  // 64 blocks per workgroup on the grid's y axis
  if (rows < 0 || rows >= ((int64_t)1 << 31) || blocks <= 0 || blocks > (int64_t)65535 * 64)
    return fail(MXGG_ERR_SHAPE, "rows=%lld blocks=%lld (0 <= rows < 2^31, 0 < blocks <= 4194240)", rows, blocks);
  if (rows > 0 && (!src || !dst)) return fail(MXGG_ERR_NULL, "src or dst is NULL");
  return Check{};
}

}  // namespace mxgg
