// MX quantizers (E2M1 / E4M3 elements, UE8M0 scale per 32 elements) for gfx950.
//
// Row-wise: the row operand of "Triton mxfp4 (and a8w4) grouped GEMM kernel"
// (data [rows, cols/2] or [rows, cols], scales [rows, cols/32]).
// Column-wise, segment-padded: the padded column operand of the variable-K
// weight gradient on the same page (each expert's rows transposed, blocks of 32
// starting at the segment start, zeros past the segment end).
//
// Both kernels are HBM-bound (2 B read, 0.53 B (E2M1) or 1.03 B (E4M3) written
// per element): they read with 16-byte (row-wise) or 4-byte-per-lane fully
// coalesced loads, reduce amax inside the wavefront, and encode in integer
// arithmetic (mx_round.hpp).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launch.hpp"
#include "mx_round.hpp"

namespace mxgg {

// ---------------------------------------------------------------------------
// Row-wise. A lane owns one 16-byte chunk (8 elements); 4 consecutive lanes
// own one 32-element block, so amax takes two xor-shuffles. Chunks are
// numbered row-major over the whole matrix; cols % 32 == 0 keeps every group
// of 4 consecutive chunks inside one block.
// ---------------------------------------------------------------------------
template <class F>
__global__ __launch_bounds__(256) void quant_rowwise_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                            int64_t chunks_per_row, int64_t total_chunks,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  constexpr bool FP4 = F::MB == 1;
  const int64_t qrow_bytes = FP4 ? chunks_per_row * 4 : chunks_per_row * 8;
  const int64_t srow_bytes = chunks_per_row / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // every lane of a wave runs the same number of iterations (the grid size and
  // the chunk count are multiples of 64 or the tail is masked), keeping the
  // shuffles below convergent
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < total_chunks; base += stride) {
    const int64_t c = base + threadIdx.x;
    const bool valid = c < total_chunks;
    const int64_t row = valid ? c / chunks_per_row : 0;
    const int64_t col = valid ? c - row * chunks_per_row : 0;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (valid) v = *reinterpret_cast<const uint4*>(x + row * ldx + col * 8);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
      amax = max(amax, max(lo, hi));
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 64));
    const int e = mx_shared_exp<F>(amax);
    if (!valid) continue;
    if constexpr (FP4) {
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        packed |= mx_encode<F>(w[i] & 0xffffu, e) << (8 * i);
        packed |= mx_encode<F>(w[i] >> 16, e) << (8 * i + 4);
      }
      *reinterpret_cast<uint32_t*>(q + row * qrow_bytes + col * 4) = packed;
    } else {
      uint32_t p0 = 0, p1 = 0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        p0 |= mx_encode<F>(w[i] & 0xffffu, e) << (16 * i);
        p0 |= mx_encode<F>(w[i] >> 16, e) << (16 * i + 8);
        p1 |= mx_encode<F>(w[i + 2] & 0xffffu, e) << (16 * i);
        p1 |= mx_encode<F>(w[i + 2] >> 16, e) << (16 * i + 8);
      }
      *reinterpret_cast<uint2*>(q + row * qrow_bytes + col * 8) = make_uint2(p0, p1);
    }
    if ((col & 3) == 0) s[row * srow_bytes + (col >> 2)] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------
// Column-wise, segment-padded. One workgroup handles one 32-row block of the
// padded row space and 512 columns; a lane owns 2 adjacent columns and loads
// 4 bytes per row (a wave reads 256 contiguous bytes per row). Rows past the
// expert's segment end are zeros. Output per column: 16 (E2M1) or 32 (E4M3)
// contiguous bytes plus one scale byte.
// ---------------------------------------------------------------------------
template <class F>
__global__ __launch_bounds__(256) void quant_colwise_segpad_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                   int64_t cols, const SplitArgs sp, int64_t mpad,
                                                                   uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  constexpr bool FP4 = F::MB == 1;
  __shared__ int64_t pref[kMaxExperts + 1];   // low: padded offsets, high: row offsets
  __shared__ int64_t wtot[4];
  __shared__ int32_t pad_offs[kMaxExperts + 1];
  const int G = sp.G;
  block_prefix64<256>(G, [&](int g) {
    const int64_t m = sp.m[g];
    return (m << 32) | ((m + 31) & ~31ll);
  }, pref, wtot);
  for (int g = threadIdx.x; g <= G; g += 256) pad_offs[g] = (int32_t)(pref[g] & 0xffffffffll);
  __syncthreads();

  const int64_t p0 = (int64_t)blockIdx.x * 32;             // first padded row of this block
  const int g = upper_bound_i32(pad_offs, G + 1, (int32_t)p0) - 1;
  const int64_t seg_row0 = pref[g] >> 32;                  // first real row of expert g
  const int64_t local = p0 - pad_offs[g];                  // block start inside the segment
  const int64_t nvalid_ll = (int64_t)sp.m[g] - local;
  const int nvalid = nvalid_ll > 32 ? 32 : (int)nvalid_ll;  // >= 1 by construction

  const int64_t c0 = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 2;  // first of 2 columns
  if (c0 >= cols) return;
  const uint16_t* xp = x + (seg_row0 + local) * ldx + c0;
  uint32_t v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = (r < nvalid) ? *reinterpret_cast<const uint32_t*>(xp + r * ldx) : 0u;
  uint32_t amax0 = 0, amax1 = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    amax0 = max(amax0, v[r] & 0x7fffu);
    amax1 = max(amax1, (v[r] >> 16) & 0x7fffu);
  }
  const int e0 = mx_shared_exp<F>(amax0), e1 = mx_shared_exp<F>(amax1);
  const int64_t qld = FP4 ? mpad / 2 : mpad;
  uint8_t* q0 = q + c0 * qld + (FP4 ? p0 / 2 : p0);
  uint8_t* q1 = q0 + qld;
  if constexpr (FP4) {
    uint32_t a[4] = {0, 0, 0, 0}, b[4] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      a[r >> 3] |= mx_encode<F>(v[r] & 0xffffu, e0) << (4 * (r & 7));
      b[r >> 3] |= mx_encode<F>(v[r] >> 16, e1) << (4 * (r & 7));
    }
    *reinterpret_cast<uint4*>(q0) = make_uint4(a[0], a[1], a[2], a[3]);
    *reinterpret_cast<uint4*>(q1) = make_uint4(b[0], b[1], b[2], b[3]);
  } else {
    uint32_t a[8] = {0, 0, 0, 0, 0, 0, 0, 0}, b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      a[r >> 2] |= mx_encode<F>(v[r] & 0xffffu, e0) << (8 * (r & 3));
      b[r >> 2] |= mx_encode<F>(v[r] >> 16, e1) << (8 * (r & 3));
    }
    reinterpret_cast<uint4*>(q0)[0] = make_uint4(a[0], a[1], a[2], a[3]);
    reinterpret_cast<uint4*>(q0)[1] = make_uint4(a[4], a[5], a[6], a[7]);
    reinterpret_cast<uint4*>(q1)[0] = make_uint4(b[0], b[1], b[2], b[3]);
    reinterpret_cast<uint4*>(q1)[1] = make_uint4(b[4], b[5], b[6], b[7]);
  }
  const int64_t sld = mpad / 32;
  s[c0 * sld + p0 / 32] = (uint8_t)(e0 + 127);
  s[(c0 + 1) * sld + p0 / 32] = (uint8_t)(e1 + 127);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quant_rowwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool fp8,
                                   uint8_t* q, uint8_t* s, int num_cus, hipStream_t st) {
  const int64_t cpr = cols / 8;
  const int64_t total = rows * cpr;
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = (int64_t)num_cus * 16;
  if (blocks > cap) blocks = cap;
  if (fp8)
    hipLaunchKernelGGL(quant_rowwise_kernel<E4M3Fmt>, dim3((unsigned)blocks), dim3(256), 0, st, x, ldx, cpr, total,
                       q, s);
  else
    hipLaunchKernelGGL(quant_rowwise_kernel<E2M1Fmt>, dim3((unsigned)blocks), dim3(256), 0, st, x, ldx, cpr, total,
                       q, s);
  return hipGetLastError();
}

hipError_t launch_quant_colwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                   bool fp8, uint8_t* q, uint8_t* s, int64_t mpad, hipStream_t st) {
  (void)rows;
  const dim3 grid((unsigned)(mpad / 32), (unsigned)((cols / 2 + 255) / 256));
  if (fp8)
    hipLaunchKernelGGL(quant_colwise_segpad_kernel<E4M3Fmt>, grid, dim3(256), 0, st, x, ldx, cols, sp, mpad, q, s);
  else
    hipLaunchKernelGGL(quant_colwise_segpad_kernel<E2M1Fmt>, grid, dim3(256), 0, st, x, ldx, cols, sp, mpad, q, s);
  return hipGetLastError();
}

}  // namespace mxgg
