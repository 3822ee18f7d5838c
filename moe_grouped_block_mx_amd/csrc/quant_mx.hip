// MX quantizers (E2M1 / E4M3 elements, UE8M0 scale per 32 elements) for gfx950.
//
// Row-wise: the row operand of "Triton mxfp4 (and a8w4) grouped GEMM kernel"
// (data [rows, cols/2] or [rows, cols]; scales block-major [cols/32, R4],
// R4 = rows rounded up to a multiple of 4, so a GEMM stage reads the scales of
// consecutive rows contiguously, four rows per aligned word).
// Column-wise, segment-padded: the padded column operand of the variable-K
// weight gradient on the same page (each expert's rows transposed, blocks of 32
// starting at the segment start, zeros past the segment end).
//
// Both kernels are HBM-bound (2 B read, 0.53 B (E2M1) or 1.03 B (E4M3) written
// per element): they read with 16-byte fully coalesced loads, keep several
// loads in flight per thread, reduce amax inside the wavefront (row-wise) or
// per thread after an LDS transpose (column-wise), and encode with gfx950's
// scaled conversions (mx_round.hpp states why they match the MX rule).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launch.hpp"
#include "mx_round.hpp"

namespace mxgg {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v2bf16 as_bf16x2(uint32_t w) { return __builtin_bit_cast(v2bf16, w); }

// ---------------------------------------------------------------------------
// Row-wise. A wave owns 64 consecutive 16-byte chunks (8 elements each) of one
// row, so every load instruction reads 1 KiB contiguous; 4 consecutive lanes
// hold one 32-element block and reduce amax with two xor-shuffles. Each thread
// keeps U = 4 consecutive rows' loads in flight before encoding (memory-level
// parallelism), so the four scale bytes of a block's rows are adjacent in the
// block-major scale layout and go out as one 4-byte store.
// Grid: x over 64-chunk column groups, y over 4*U-row groups (grid-strided).
// ---------------------------------------------------------------------------
template <class F, int U>
__global__ __launch_bounds__(256) void quant_rowwise_kernel(const uint16_t* __restrict__ x, int64_t ldx, int rows,
                                                            int cpr, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ s, int64_t sld) {
  constexpr bool FP4 = F::MB == 1;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;  // chunk inside the row
  const bool cvalid = c < cpr;
  const int64_t qrow_bytes = FP4 ? (int64_t)cpr * 4 : (int64_t)cpr * 8;
  static_assert(U == 4, "four rows per thread: one 4-byte scale store");
  for (int rb = blockIdx.y * (4 * U); rb < rows; rb += gridDim.y * (4 * U)) {
    uint4 v[U];
    uint32_t sbytes = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + w * U + u;
      v[u] = (cvalid && r < rows) ? *reinterpret_cast<const uint4*>(x + (int64_t)r * ldx + (int64_t)c * 8)
                                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + w * U + u;
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = max(amax, max(wd[i] & 0x7fffu, (wd[i] >> 16) & 0x7fffu));
      amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
      amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 64));
      const int e = mx_shared_exp<F>(amax);
      if (!(cvalid && r < rows)) continue;
      const float sc = __uint_as_float(mx_scale_operand_bits(e));
      if constexpr (FP4) {
        uint32_t packed = 0;
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[0]), sc, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[1]), sc, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[2]), sc, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[3]), sc, 3);
        *reinterpret_cast<uint32_t*>(q + (int64_t)r * qrow_bytes + (int64_t)c * 4) = packed;
      } else {
        const uint32_t lim = e4m3_sat_limit_bits(e);
        v2s p0 = {0, 0}, p1 = {0, 0};
        p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p0, as_bf16x2(clamp_bf16x2_mag(wd[0], lim)), sc, false);
        p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p0, as_bf16x2(clamp_bf16x2_mag(wd[1], lim)), sc, true);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p1, as_bf16x2(clamp_bf16x2_mag(wd[2], lim)), sc, false);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p1, as_bf16x2(clamp_bf16x2_mag(wd[3], lim)), sc, true);
        *reinterpret_cast<uint2*>(q + (int64_t)r * qrow_bytes + (int64_t)c * 8) =
            make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
      }
      sbytes |= (uint32_t)(e + 127) << (8 * u);
    }
    // block-major scales [cols/32, sld], sld = rows rounded up to a multiple
    // of 4: the thread's four rows are one aligned word (padding rows get 0)
    const int r0 = rb + w * U;
    if (cvalid && (c & 3) == 0 && r0 < rows) *reinterpret_cast<uint32_t*>(s + (int64_t)(c >> 2) * sld + r0) = sbytes;
  }
}

// ---------------------------------------------------------------------------
// Column-wise, segment-padded. A workgroup transposes a tile of 128 padded
// rows (four 32-row blocks, each mapped to its own expert segment) by 64
// columns through LDS: the tile is read with 16-byte loads (8 lanes per
// 128-byte row segment), then thread (column c, block b) encodes the 32 values
// of its block. The four blocks of one column are consecutive in the output, so
// a column's 64 (E2M1) or 128 (E4M3) bytes are written by the four waves
// together.
// ---------------------------------------------------------------------------
template <class F>
__global__ __launch_bounds__(256) void quant_colwise_segpad_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                   int64_t cols, const SplitArgs sp, int64_t mpad,
                                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  constexpr bool FP4 = F::MB == 1;
  constexpr int PITCH = 64 + 2;  // bf16 elements per LDS row (padding spreads column reads over banks)
  __shared__ int64_t pref[kMaxExperts + 1];   // low: padded offsets, high: row offsets
  __shared__ int64_t wtot[4];
  __shared__ int32_t pad_offs[kMaxExperts + 1];
  __shared__ uint16_t tile[128 * PITCH];
  __shared__ int64_t blk_row0[4];             // first source row of each 32-row block (-1: outside mpad)
  __shared__ int32_t blk_valid[4];            // real rows in the block

  const int G = sp.G;
  block_prefix64<256>(G, [&](int g) {
    const int64_t m = sp.m[g];
    return (m << 32) | ((m + 31) & ~31ll);
  }, pref, wtot);
  for (int g = threadIdx.x; g <= G; g += 256) pad_offs[g] = (int32_t)(pref[g] & 0xffffffffll);
  __syncthreads();

  const int64_t pt0 = (int64_t)blockIdx.x * 128;  // first padded row of the tile
  if (threadIdx.x < 4) {
    const int64_t p0 = pt0 + threadIdx.x * 32;
    if (p0 < mpad) {
      const int g = upper_bound_i32(pad_offs, G + 1, (int32_t)p0) - 1;
      const int64_t local = p0 - pad_offs[g];
      const int64_t nv = (int64_t)sp.m[g] - local;
      blk_row0[threadIdx.x] = (pref[g] >> 32) + local;
      blk_valid[threadIdx.x] = nv > 32 ? 32 : (int)nv;
    } else {
      blk_row0[threadIdx.x] = -1;
      blk_valid[threadIdx.x] = 0;
    }
  }
  __syncthreads();

  const int64_t c0 = (int64_t)blockIdx.y * 64;
  const int ncol = cols - c0 < 64 ? (int)(cols - c0) : 64;  // multiple of 32 (cols % 32 == 0)
  // load: 128 rows x 8 chunks of 16 bytes; thread -> (row, chunk), 4 passes
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = pass * 256 + threadIdx.x;
    const int row = idx >> 3, ch = idx & 7;
    const int b = row >> 5, rin = row & 31;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rin < blk_valid[b] && ch * 8 < ncol)
      v = *reinterpret_cast<const uint4*>(x + (blk_row0[b] + rin) * ldx + c0 + ch * 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * PITCH + ch * 8);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
  __syncthreads();

  const int c = threadIdx.x & 63, b = threadIdx.x >> 6;
  const int64_t p0 = pt0 + b * 32;
  if (c >= ncol || p0 >= mpad) return;
  uint32_t vals[32];
  uint32_t amax = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    vals[r] = tile[(b * 32 + r) * PITCH + c];
    amax = max(amax, vals[r] & 0x7fffu);
  }
  const int e = mx_shared_exp<F>(amax);
  const float sc = __uint_as_float(mx_scale_operand_bits(e));
  const int64_t qld = FP4 ? mpad / 2 : mpad;
  uint8_t* qp = q + (c0 + c) * qld + (FP4 ? p0 / 2 : p0);
  if constexpr (FP4) {
    uint32_t a[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t wv = 0;
      wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(wv, as_bf16x2(vals[8 * d + 0] | (vals[8 * d + 1] << 16)), sc, 0);
      wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(wv, as_bf16x2(vals[8 * d + 2] | (vals[8 * d + 3] << 16)), sc, 1);
      wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(wv, as_bf16x2(vals[8 * d + 4] | (vals[8 * d + 5] << 16)), sc, 2);
      wv = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(wv, as_bf16x2(vals[8 * d + 6] | (vals[8 * d + 7] << 16)), sc, 3);
      a[d] = wv;
    }
    *reinterpret_cast<uint4*>(qp) = make_uint4(a[0], a[1], a[2], a[3]);
  } else {
    const uint32_t lim = e4m3_sat_limit_bits(e);
    uint32_t a[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      v2s wv = {0, 0};
      wv = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
          wv, as_bf16x2(clamp_bf16x2_mag(vals[4 * d + 0] | (vals[4 * d + 1] << 16), lim)), sc, false);
      wv = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(
          wv, as_bf16x2(clamp_bf16x2_mag(vals[4 * d + 2] | (vals[4 * d + 3] << 16), lim)), sc, true);
      a[d] = __builtin_bit_cast(uint32_t, wv);
    }
    reinterpret_cast<uint4*>(qp)[0] = make_uint4(a[0], a[1], a[2], a[3]);
    reinterpret_cast<uint4*>(qp)[1] = make_uint4(a[4], a[5], a[6], a[7]);
  }
  s[(p0 / 32) * cols + c0 + c] = (uint8_t)(e + 127);  // block-major: [mpad/32, cols]
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quant_rowwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool fp8,
                                   uint8_t* q, uint8_t* s, int num_cus, hipStream_t st) {
  (void)num_cus;
  constexpr int U = 4;
  const int cpr = (int)(cols / 8);
  const int64_t gy_need = (rows + 4 * U - 1) / (4 * U);
  const dim3 grid((unsigned)((cpr + 63) / 64), (unsigned)(gy_need < 65535 ? gy_need : 65535));
  if (fp8)
    hipLaunchKernelGGL((quant_rowwise_kernel<E4M3Fmt, U>), grid, dim3(256), 0, st, x, ldx, (int)rows, cpr, q, s,
                       mx_scale_stride(rows));
  else
    hipLaunchKernelGGL((quant_rowwise_kernel<E2M1Fmt, U>), grid, dim3(256), 0, st, x, ldx, (int)rows, cpr, q, s,
                       mx_scale_stride(rows));
  return hipGetLastError();
}

hipError_t launch_quant_colwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                   bool fp8, uint8_t* q, uint8_t* s, int64_t mpad, hipStream_t st) {
  (void)rows;
  const dim3 grid((unsigned)((mpad + 127) / 128), (unsigned)((cols + 63) / 64));
  if (fp8)
    hipLaunchKernelGGL(quant_colwise_segpad_kernel<E4M3Fmt>, grid, dim3(256), 0, st, x, ldx, cols, sp, mpad, q, s);
  else
    hipLaunchKernelGGL(quant_colwise_segpad_kernel<E2M1Fmt>, grid, dim3(256), 0, st, x, ldx, cols, sp, mpad, q, s);
  return hipGetLastError();
}

}  // namespace mxgg
