// Internal host-side launch interface between the C ABI (api.cpp) and the
// kernels (*.hip). Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <utility>

#include "device_common.hpp"

namespace mxgg {

// Raise a kernel's dynamic LDS limit on the stream's device before its first
// launch there. The limit is an attribute of one kernel on one device, so it
// is set once per (kernel, device) pair, with that device current; host
// threads may launch concurrently, hence the lock.
inline hipError_t ensure_dynamic_lds(const void* kernel, int bytes, hipStream_t st) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  int cur = 0;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (cur != dev) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

// Row-split grouped GEMM (forward and input gradient): out[r, :] for every row
// r of expert g is A[r, :] . B_g^T, where B_g is the [n_out, kc] operand of
// expert g starting at b + g * b_gstride with row stride ldb.
// Block stride of block-major MX scales: rows rounded up to a multiple of 4.
__host__ __device__ inline int64_t mx_scale_stride(int64_t rows) { return rows > 0 ? (rows + 3) & ~(int64_t)3 : 0; }

// MFMA layout of MX scales: rows padded to a multiple of 32 (r32), blocks in
// groups of 4; unit (b/4, r/32) holds 128 bytes, and lane L = r%32 + 32*(b%2)
// of a 32x32x64 scaled MFMA fragment finds the scales of its two 64-deep K
// steps at bytes 2L and 2L+1 (j = (b%4)/2). Byte offset of row r, block b.
__host__ __device__ inline int64_t mx_rows32(int64_t rows) { return rows > 0 ? (rows + 31) & ~(int64_t)31 : 0; }
__host__ __device__ inline int64_t mfma_scale_offset(int64_t r, int64_t b, int64_t r32) {
  return (b >> 2) * (r32 * 4) + (r >> 5) * 128 + ((r & 31) + 32 * (b & 1)) * 2 + ((b >> 1) & 1);
}

struct RowsGemmParams {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  uint16_t* c;            // bf16 output
  int64_t lda, ldb;       // A / B data row strides (bytes)
  int64_t ldas, ldbs;     // scale strides (bytes): MX scales are block-major
                          // [blocks, R4] (ld = the block stride R4, a
                          // multiple of 4); 1x128 fp32 scales block-major
                          // [blocks, rows] (ld = rows * 4); 128x128 weight
                          // scales row-major over blocks (ld = the row stride)
  int64_t b_gstride;      // bytes between consecutive experts' B data
  int64_t bs_gstride;     // bytes between consecutive experts' B scales
  int64_t ldc;            // output row stride (elements)
  int32_t n_out;          // output columns
  int32_t kc;             // contraction length (elements), multiple of 32
  SplitArgs sp;
};

// Variable-K grouped weight gradient: out[g] (rows n_rows, cols n_cols) =
// A_g . B_g^T contracted over expert g's padded segment.
struct WgradParams {
  const uint8_t* a;       // [n_rows, mpad] operand (dY column-wise)
  const uint8_t* as;
  const uint8_t* b;       // [n_cols, mpad] operand (X column-wise)
  const uint8_t* bs;
  void* c;                // [G, n_rows, n_cols] fp32 (or bf16)
  int64_t lda, ldas, ldb, ldbs;  // as in RowsGemmParams
  int32_t n_rows, n_cols;
  int32_t accumulate;
  int32_t out_bf16;
  SplitArgs sp;
  int16_t order[kMaxExperts];  // experts by decreasing split (longest first)
};

struct DeviceInfo {
  int num_cus;
};

// MX quantizers; mfma: scales in the MFMA layout (column-wise: every split a
// multiple of 128), else block-major
// kb / kbr / kbc: the row-wise / column-wise codes in 64-byte K blocks
// (u8 [bytes per row / 64, rows, 64]), else rows
hipError_t launch_quant_rowwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool fp8, bool mfma,
                                   bool kb, uint8_t* q, uint8_t* s, int num_cus, hipStream_t st);
hipError_t launch_quant_dual_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                bool fp8, bool mfma, bool kbr, bool kbc, uint8_t* qr, uint8_t* sr, uint8_t* qc,
                                uint8_t* sc, int64_t mpad, int num_cus, hipStream_t st);
hipError_t launch_quant_colwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                   bool fp8, bool mfma, bool kbc, uint8_t* q, uint8_t* s, int64_t mpad, int num_cus,
                                   hipStream_t st);

// MX scales from one layout (mxgg_scale_layout value) into another
hipError_t launch_relayout_scales(const uint8_t* src, int src_layout, int64_t rows, int64_t blocks, int dst_layout,
                                  uint8_t* dst, hipStream_t st);

// dgrad selects the input-gradient kernel symbol (same code as the forward's);
// mfma_b: B's scales in the MFMA layout (bs_gstride then in bytes of it)
// kblk: both operands' codes in 64-byte K blocks (lda / ldb = bytes per block)
hipError_t launch_grouped_rows_mx(const RowsGemmParams& p, bool a_fp8, bool dgrad, bool mfma_b, bool kblk,
                                  int num_cus, hipStream_t st);
// fp8: E4M3 operands on both sides (MXFP8), else E2M1 (MXFP4)
hipError_t launch_grouped_wgrad_mx(const WgradParams& p, bool fp8, int num_cus, hipStream_t st);

// Blockwise FP8 (E4M3 codes, fp32 scales per 128 along the contraction;
// 1x128 scales block-major: [blocks, rows] row-wise, [mpad/128, cols]
// column-wise).
hipError_t launch_quant_rowwise_blk(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool blk128x128,
                                    bool pow2, uint8_t* q, float* s, hipStream_t st);
// both of the above (1x128 row-wise and column-wise segment-padded) from one
// read; cols a multiple of 128
hipError_t launch_quant_dual_blk(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                 bool pow2, uint8_t* qr, float* sr, uint8_t* qc, float* sc, int64_t mpad,
                                 hipStream_t st);
hipError_t launch_quant_colwise_blk(const uint16_t* x, int64_t cols, int64_t ldx, const SplitArgs& sp, bool pow2,
                                    uint8_t* q, float* s, int64_t mpad, hipStream_t st);
// 128x128-block weights [G*N, K] (+ f32 [G*N/128, K/128]) -> [G*K, N] (+ f32
// [G*K/128, N/128]); N, K multiples of 128
hipError_t launch_transpose_128x128(const uint8_t* wq, const float* ws, int32_t G, int64_t N, int64_t K, uint8_t* tq,
                                    float* ts, hipStream_t st);
// pow2: every scale is a power of two (the MFMA applies it; no per-128 partial)
hipError_t launch_grouped_rows_blk(const RowsGemmParams& p, bool pow2, bool dgrad, int num_cus, hipStream_t st);
hipError_t launch_grouped_wgrad_blk(const WgradParams& p, bool pow2, int num_cus, hipStream_t st);

}  // namespace mxgg
