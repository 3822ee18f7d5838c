// Device-side helpers shared by the quantizer and GEMM kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxgg {

constexpr int kMaxExperts = 512;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Expert split counts travel as kernel arguments (int32, at most 512), so a
// launch needs no device-side copy of the host array.
struct SplitArgs {
  int32_t G;
  int32_t m[kMaxExperts];
};

// Block-wide exclusive prefix sum of 64-bit values v(g), g < G, into
// out[0..G] (out[G] = total). Every thread of the block must call it.
// Used on packed pairs (low and high 32-bit halves summed independently:
// neither half's total may exceed 2^32 - 1).
template <int THREADS, class F>
__device__ inline void block_prefix64(int G, F v, int64_t* out, int64_t* wave_tot) {
  static_assert(THREADS % 64 == 0 && THREADS >= 64, "threads");
  constexpr int NW = THREADS / 64;
  constexpr int PER = (kMaxExperts + THREADS - 1) / THREADS;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int64_t local[PER];
  int64_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = t * PER + i;
    local[i] = (g < G) ? v(g) : 0;
    sum += local[i];
  }
  // inclusive scan of per-thread sums inside the wave
  int64_t inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int64_t o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int64_t base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wave) base += wave_tot[w];
  int64_t run = base + inc - sum;  // exclusive prefix of this thread's first item
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = t * PER + i;
    if (g < G) out[g] = run;
    run += local[i];
  }
  if (t == THREADS - 1) out[G] = run;  // grand total (last thread's run covers all)
  __syncthreads();
}

// Number of entries of the non-decreasing arr[0..n) that are <= val
// (the upper_bound position). With arr = exclusive prefix offsets (arr[0] = 0)
// the owning segment of item `val` is upper_bound - 1.
__device__ inline int upper_bound_i32(const int32_t* arr, int n, int32_t val) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (arr[mid] <= val) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// The i-th 16-byte chunk position after an XOR swizzle of the chunk index by
// row bits, for the MFMA fragment reads (ds_read_b128: lane l reads row
// base + l%32, chunk k + l/32, base a multiple of 32). The masks were chosen by
// measuring that exact pattern on gfx950 (bank-conflict counter and read rate):
// 4 chunks per row, (row>>2)&3: conflict-free, 570 GB/s per CU, where
// ((row>>1)^(row>>3))&3 had half of its LDS cycles in bank conflicts (294 GB/s);
// 8 chunks, (row>>1)&7: 559 GB/s (row^(row>>3): 533); 2 chunks, (row>>3)&1:
// 562 GB/s ((row>>2)&1: 301). An XOR is its own inverse, so the DMA side
// (which global chunk lands in a given LDS slot) and the read side use the
// same function.
template <int CHUNKS_PER_ROW>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (CHUNKS_PER_ROW == 8) {
    return chunk ^ ((row >> 1) & 7);
  } else if constexpr (CHUNKS_PER_ROW == 4) {
    return chunk ^ ((row >> 2) & 3);
  } else if constexpr (CHUNKS_PER_ROW == 2) {
    return chunk ^ ((row >> 3) & 1);
  } else {
    return chunk;
  }
}

// Byte c (along the row) of row r of a code tensor with `rows` rows stored in
// 64-byte K blocks, u8 [bytes per row / 64, rows, 64].
__device__ __forceinline__ int64_t kblk_off(int64_t r, int64_t c, int64_t rows) {
  return (c >> 6) * rows * 64 + r * 64 + (c & 63);
}

}  // namespace mxgg
