// Blockwise FP8 quantizers for gfx950 ("Add ROCm Triton blockwise FP8 grouped
// GEMM"): E4M3 codes with one fp32 scale per block.
//
//   1x128 row-wise   activations: blocks of 128 along the row (the contraction
//                    axis of the forward pass); scales f32 [cols/128, rows]
//                    (block-major, as the GEMM's DMA reads them: a tile's rows
//                    of one block are contiguous).
//   128x128          weights: square blocks; scales f32 [rows/128, cols/128].
// Every blockwise code tensor is stored in 64-byte blocks along its rows,
// u8 [cols/64, rows, 64] (kblk_off): a GEMM stage's 64 bytes of each of a
// tile's rows are one contiguous run.
//   1x128 column-wise, segment-padded: the wgrad operands; each expert's rows
//                    transposed, padded with zeros to a multiple of 128, blocks
//                    of 128 along the padded length; codes in 64-byte K blocks,
//                    u8 [mpad/64, cols, 64] (the weight gradient's DMA reads a
//                    tile's 64-byte row pieces of one block as one run); scales
//                    f32 [mpad/128, cols] (block-major).
//
// Scale rule and encoder: blk_round.hpp. In power-of-two mode the codes come
// from gfx950's scaled conversion with the stored scale 2^-t as its operand
// (it divides by the scale: an exact multiplication by 2^t, and the rule keeps
// every product at or below 448, where the conversion rounds to nearest even);
// in fp32 mode the product x * q is rounded to fp32 first and encoded in
// software. All three kernels are HBM-bound (2 B read, 1 B + 4/128 B written
// per element) and read with 16-byte coalesced loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "blk_round.hpp"
#include "device_common.hpp"
#include "launch.hpp"

namespace mxgg {

namespace {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v2bf16 as_bf16x2(uint32_t w) { return __builtin_bit_cast(v2bf16, w); }

// Per-block encoding parameters from the block's bf16 amax magnitude.
struct BlkScale {
  float op;        // pow2: the conversion's scale operand 2^-t; fp32 mode: q
  float stored;    // the scale written out (2^-t or fp32(1/q))
};

template <bool POW2>
__device__ __forceinline__ BlkScale blk_scale(uint32_t amax_mag) {
  const uint32_t a = blk_amax_floored_bits(amax_mag);
  if constexpr (POW2) {
    const float s = __uint_as_float(blk_pow2_scale_bits(blk_pow2_t(a)));
    return BlkScale{s, s};
  } else {
    const float q = 448.0f / __uint_as_float(a);  // IEEE division (correctly rounded)
    return BlkScale{q, 1.0f / q};
  }
}

// 8 bf16 (4 packed words) -> 8 E4M3 codes (2 words, element 0 in byte 0).
template <bool POW2>
__device__ __forceinline__ uint2 encode8(const uint32_t (&wd)[4], const BlkScale& bs) {
  if constexpr (POW2) {
    v2s p0 = {0, 0}, p1 = {0, 0};
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p0, as_bf16x2(wd[0]), bs.op, false);
    p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p0, as_bf16x2(wd[1]), bs.op, true);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p1, as_bf16x2(wd[2]), bs.op, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p1, as_bf16x2(wd[3]), bs.op, true);
    return make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
  } else {
    uint32_t o[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(wd[i] << 16) * bs.op;
      const float hi = __uint_as_float(wd[i] & 0xffff0000u) * bs.op;
      const uint32_t pair = f32_to_e4m3_rne_sat(__float_as_uint(lo)) | (f32_to_e4m3_rne_sat(__float_as_uint(hi)) << 8);
      o[i >> 1] |= pair << (16 * (i & 1));
    }
    return make_uint2(o[0], o[1]);
  }
}

__device__ __forceinline__ uint32_t amax8(const uint32_t (&wd)[4]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(wd[i] & 0x7fffu, (wd[i] >> 16) & 0x7fffu));
  return m;
}

// 128x128-block weights transposed for the input gradient (which contracts
// over the weights' rows): the blocks are square, so W^T's 128x128
// quantization is W's, transposed: the same codes and the same scale per
// block. One workgroup per block: the 128 rows x 128 bytes are read with
// 16-byte loads into LDS (dword pitch 33), then written back transposed with
// 16-byte stores (both sides in 64-byte K blocks: W [K/64, G*N, 64], W^T
// [N/64, G*K, 64]). HBM-bound: 1 B read and 1 B written per element.
__global__ __launch_bounds__(256) void transpose_128x128_kernel(const uint8_t* __restrict__ wq,
                                                                const float* __restrict__ ws, int64_t G, int64_t N,
                                                                int64_t K, uint8_t* __restrict__ tq,
                                                                float* __restrict__ ts) {
  __shared__ uint32_t tile[128][33];
  const int64_t nbs = N / 128, kbs = K / 128;
  const int64_t b = blockIdx.x;
  const int64_t g = b / (nbs * kbs);
  const int64_t rem = b - g * nbs * kbs;
  const int64_t nb = rem / kbs, kb = rem - nb * kbs;
  const int64_t wrows = G * N, trows = G * K;
  // load chunk c: block half c/512, row (c/4)%128, 16-byte piece c%4 (a
  // wave's load is 16 consecutive rows of one block: one 1 KiB run)
  for (int c = threadIdx.x; c < 1024; c += 256) {
    const int r = (c >> 2) & 127, q = ((c >> 9) << 2) | (c & 3);
    const uint4 v = *reinterpret_cast<const uint4*>(wq + kblk_off(g * N + nb * 128 + r, kb * 128 + q * 16, wrows));
    tile[r][4 * q] = v.x;
    tile[r][4 * q + 1] = v.y;
    tile[r][4 * q + 2] = v.z;
    tile[r][4 * q + 3] = v.w;
  }
  __syncthreads();
  // The 128 output rows (k) by 128 bytes (n) are two 64-byte K blocks of
  // W^T, each one 8 KiB run. Chunk c: block half h = c/512, row k =
  // (c/4)%128, 16-byte piece qd = c%4, so the 64 chunks of a wave's store are
  // one contiguous 1 KiB (16 rows); a chunk gathers its 16 bytes from 16 LDS
  // rows.
  for (int c = threadIdx.x; c < 1024; c += 256) {
    const int h = c >> 9, k = (c >> 2) & 127, qd = c & 3;
    const int n0 = h * 64 + qd * 16, sh = 8 * (k & 3);
    uint32_t o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      o[m] = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[m] |= ((tile[n0 + 4 * m + t][k >> 2] >> sh) & 0xffu) << (8 * t);
    }
    *reinterpret_cast<uint4*>(tq + kblk_off(g * K + kb * 128 + k, nb * 128 + n0, trows)) =
        make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (threadIdx.x == 0) ts[(g * kbs + kb) * nbs + nb] = ws[(g * nbs + nb) * kbs + kb];
}

}  // namespace

// ---------------------------------------------------------------------------
// 1x128 row-wise. As the MX row-wise kernel: a wave owns 64 consecutive
// 16-byte chunks of one row (four 128-element blocks, 16 lanes each, amax
// reduced with four xor-shuffles); each thread keeps U rows' loads in flight.
// The workgroup's 4*U rows x 512 code bytes (eight 64-byte K blocks) are
// staged in LDS as [K block][row][64 bytes], so that after a barrier every
// store instruction writes 1 KiB of contiguous K-blocked codes.
// ---------------------------------------------------------------------------
template <bool POW2, int U>
__global__ __launch_bounds__(256) void quant_rowwise_1x128_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                  int rows, int cpr, uint8_t* __restrict__ q,
                                                                  float* __restrict__ s) {
  static_assert(U == 4, "16 rows per workgroup and iteration: 64 threads per staged K block");
  __shared__ uint4 stage[8 * 16 * 4];  // [K block][row][4 x 16 bytes]
  uint2* const st = reinterpret_cast<uint2*>(stage);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;  // 8-element chunk inside the row
  const bool cvalid = c < cpr;
  const int64_t nkb = cpr / 8;           // K blocks per row (cpr % 16 == 0)
  for (int rb = blockIdx.y * (4 * U); rb < rows; rb += gridDim.y * (4 * U)) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * 4 + w;
      v[u] = (cvalid && r < rows) ? *reinterpret_cast<const uint4*>(x + (int64_t)r * ldx + (int64_t)c * 8)
                                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * 4 + w;
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t amax = amax8(wd);
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, m, 64));
      const BlkScale bs = blk_scale<POW2>(amax);
      // code bytes 8*lane .. of the tile's row u*4 + w: K block lane/8
      st[((lane >> 3) * 16 + u * 4 + w) * 8 + (lane & 7)] = encode8<POW2>(wd, bs);
      if (cvalid && r < rows && (c & 15) == 0) s[(int64_t)(c >> 4) * rows + r] = bs.stored;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = threadIdx.x + 256 * j;
      const int r = rb + ((p >> 2) & 15);
      const int64_t kbg = (int64_t)blockIdx.x * 8 + (p >> 6);
      if (kbg < nkb && r < rows) *reinterpret_cast<uint4*>(q + (kbg * rows + r) * 64 + (p & 3) * 16) = stage[p];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 128x128 blocks. One workgroup per block: thread t reads rows t/16 + 16 i
// (i < 8), chunk t%16 (8 elements), i.e. every load instruction covers 16
// full 256-byte row segments; amax is reduced in the wave, then across the
// four waves through LDS. (Staging the block's codes in LDS so that every
// store writes 1 KiB of a K block measured equal: the 256-byte row loads set
// the pace.)
// ---------------------------------------------------------------------------
template <bool POW2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t rows,
                                                            int64_t cols, uint8_t* __restrict__ q,
                                                            float* __restrict__ s) {
  __shared__ uint32_t wmax[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.y * 128, c0 = (int64_t)blockIdx.x * 128;
  const int rr = t >> 4, ch = t & 15;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const uint4*>(x + (r0 + rr + 16 * i) * ldx + c0 + ch * 8);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    amax = max(amax, amax8(wd));
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, m, 64));
  if (lane == 0) wmax[w] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const BlkScale bs = blk_scale<POW2>(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    *reinterpret_cast<uint2*>(q + kblk_off(r0 + rr + 16 * i, c0 + ch * 8, rows)) = encode8<POW2>(wd, bs);
  }
  if (t == 0) s[(int64_t)blockIdx.y * (cols / 128) + blockIdx.x] = bs.stored;
}

// ---------------------------------------------------------------------------
// 1x128 column-wise, segment-padded. A workgroup transposes one 128-row block
// of the padded row space (all of it inside one expert segment, zeros past the
// segment end) by 64 columns through LDS; thread (column c, quarter b) holds
// rows 32b .. 32b+31 of column c, the four quarters combine their amax through
// LDS, and each thread writes its 32 codes (two 16-byte stores).
// ---------------------------------------------------------------------------
template <bool POW2>
__global__ __launch_bounds__(256) void quant_colwise_1x128_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                                  int64_t cols, const SplitArgs sp, int64_t mpad,
                                                                  uint8_t* __restrict__ q, float* __restrict__ s) {
  constexpr int PITCH = 64 + 2;
  __shared__ int64_t pref[kMaxExperts + 1];  // low: padded offsets, high: row offsets
  __shared__ int64_t wtot[4];
  __shared__ int32_t pad_offs[kMaxExperts + 1];
  __shared__ uint16_t tile[128 * PITCH];
  __shared__ uint32_t qmax[4][64];
  __shared__ int64_t blk_row0;
  __shared__ int32_t blk_valid;

  const int G = sp.G;
  block_prefix64<256>(G, [&](int g) {
    const int64_t m = sp.m[g];
    return (m << 32) | ((m + 127) & ~127ll);
  }, pref, wtot);
  for (int g = threadIdx.x; g <= G; g += 256) pad_offs[g] = (int32_t)(pref[g] & 0xffffffffll);
  __syncthreads();

  const int64_t p0 = (int64_t)blockIdx.x * 128;  // first padded row (< mpad by the grid)
  if (threadIdx.x == 0) {
    const int g = upper_bound_i32(pad_offs, G + 1, (int32_t)p0) - 1;
    const int64_t local = p0 - pad_offs[g];
    const int64_t nv = (int64_t)sp.m[g] - local;
    blk_row0 = (pref[g] >> 32) + local;
    blk_valid = nv > 128 ? 128 : (int)nv;
  }
  __syncthreads();

  const int64_t c0 = (int64_t)blockIdx.y * 64;
  const int ncol = cols - c0 < 64 ? (int)(cols - c0) : 64;  // multiple of 32
  const int nvalid = blk_valid;
  const int64_t row0 = blk_row0;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = pass * 256 + threadIdx.x;
    const int row = idx >> 3, ch = idx & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < nvalid && ch * 8 < ncol) v = *reinterpret_cast<const uint4*>(x + (row0 + row) * ldx + c0 + ch * 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * PITCH + ch * 8);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
  __syncthreads();

  const int c = threadIdx.x & 63, b = threadIdx.x >> 6;
  uint32_t vals[32];
  uint32_t amax = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    vals[r] = tile[(b * 32 + r) * PITCH + c];
    amax = max(amax, vals[r] & 0x7fffu);
  }
  qmax[b][c] = amax;
  __syncthreads();
  amax = max(max(qmax[0][c], qmax[1][c]), max(qmax[2][c], qmax[3][c]));
  if (c >= ncol) return;
  const BlkScale bs = blk_scale<POW2>(amax);
  uint8_t* qp = q + kblk_off(c0 + c, p0 + b * 32, cols);
  uint32_t o[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t wd[4] = {vals[8 * d] | (vals[8 * d + 1] << 16), vals[8 * d + 2] | (vals[8 * d + 3] << 16),
                            vals[8 * d + 4] | (vals[8 * d + 5] << 16), vals[8 * d + 6] | (vals[8 * d + 7] << 16)};
    const uint2 e = encode8<POW2>(wd, bs);
    o[2 * d] = e.x;
    o[2 * d + 1] = e.y;
  }
  reinterpret_cast<uint4*>(qp)[0] = make_uint4(o[0], o[1], o[2], o[3]);
  reinterpret_cast<uint4*>(qp)[1] = make_uint4(o[4], o[5], o[6], o[7]);
  if (b == 0) s[p0 / 128 * cols + c0 + c] = bs.stored;
}

// ---------------------------------------------------------------------------
// Dual output: the 1x128 row-wise and the 1x128 column-wise segment-padded
// quantizations of one bf16 tensor from a single read of it (the page's
// unified grouped kernel that emits both the row-wise activation operand and
// the segment-padded column-wise wgrad operand in one pass). A workgroup takes
// one 128-row block of the padded row space (inside one expert segment, zeros
// past its end) by 128 columns:
//   rows  thread t loads chunk t%16 (8 elements) of rows t/16 + 16 i, so the
//         16 lanes of a row hold its whole 128-element block: amax by four
//         xor-shuffles, encode from registers, one 8-byte store per lane;
//   tile  the bf16 values go to LDS;
//   cols  four threads per column (32 rows each) combine their amax through
//         LDS and write 32 codes each (two 16-byte stores).
// Identical output to the two single-output kernels (same scale rule and
// encoder on the same values).
// ---------------------------------------------------------------------------
template <bool POW2, bool ROWS = true>
__global__ __launch_bounds__(256) void quant_dual_1x128_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                               int64_t rows, int64_t cols, const SplitArgs sp,
                                                               int64_t mpad,
                                                               uint8_t* __restrict__ qr, float* __restrict__ sr,
                                                               uint8_t* __restrict__ qc, float* __restrict__ sc) {
  constexpr int PITCH = 128 + 8;  // bf16 per LDS row: 16-byte aligned rows
  __shared__ int64_t pref[kMaxExperts + 1];  // low: padded offsets, high: row offsets
  __shared__ int64_t wtot[4];
  __shared__ int32_t pad_offs[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * PITCH];
  __shared__ uint32_t qmax[4][128];
  __shared__ int64_t blk_row0;
  __shared__ int32_t blk_valid;

  const int G = sp.G;
  block_prefix64<256>(G, [&](int g) {
    const int64_t m = sp.m[g];
    return (m << 32) | ((m + 127) & ~127ll);
  }, pref, wtot);
  for (int g = threadIdx.x; g <= G; g += 256) pad_offs[g] = (int32_t)(pref[g] & 0xffffffffll);
  __syncthreads();

  const int64_t p0 = (int64_t)blockIdx.x * 128;  // first padded row (< mpad by the grid)
  if (threadIdx.x == 0) {
    const int g = upper_bound_i32(pad_offs, G + 1, (int32_t)p0) - 1;
    const int64_t local = p0 - pad_offs[g];
    const int64_t nv = (int64_t)sp.m[g] - local;
    blk_row0 = (pref[g] >> 32) + local;
    blk_valid = nv > 128 ? 128 : (int)nv;
  }
  __syncthreads();
  const int nvalid = blk_valid;
  const int64_t row0 = blk_row0;
  const int64_t c0 = (int64_t)blockIdx.y * 128;  // cols is a multiple of 128
  const int ch = threadIdx.x & 15, rg = threadIdx.x >> 4;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rg + 16 * i;
    v[i] = row < nvalid ? *reinterpret_cast<const uint4*>(x + (row0 + row) * ldx + c0 + ch * 8)
                        : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rg + 16 * i;
    const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    *reinterpret_cast<uint4*>(tile + row * PITCH + ch * 8) = v[i];
    if constexpr (!ROWS) continue;
    uint32_t amax = amax8(wd);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, m, 64));
    if (row >= nvalid) continue;
    const BlkScale bs = blk_scale<POW2>(amax);
    const int64_t r = row0 + row;
    *reinterpret_cast<uint2*>(qr + kblk_off(r, c0 + ch * 8, rows)) = encode8<POW2>(wd, bs);
    if (ch == 0) sr[c0 / 128 * rows + r] = bs.stored;
  }
  __syncthreads();

  // column-wise: item (column c, quarter b), two per thread; the quarters'
  // amax meet in LDS, then each item re-reads its 32 values and encodes them
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int item = threadIdx.x + 256 * j, c = item & 127, b = item >> 7;
    uint32_t amax = 0;
#pragma unroll
    for (int r = 0; r < 32; ++r) amax = max(amax, (uint32_t)tile[(b * 32 + r) * PITCH + c] & 0x7fffu);
    qmax[b][c] = amax;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int item = threadIdx.x + 256 * j, c = item & 127, b = item >> 7;
    const uint32_t amax = max(max(qmax[0][c], qmax[1][c]), max(qmax[2][c], qmax[3][c]));
    const BlkScale bs = blk_scale<POW2>(amax);
    uint32_t o[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t vv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) vv[k] = tile[(b * 32 + 8 * d + k) * PITCH + c];
      const uint32_t wd[4] = {vv[0] | (vv[1] << 16), vv[2] | (vv[3] << 16), vv[4] | (vv[5] << 16),
                              vv[6] | (vv[7] << 16)};
      const uint2 e = encode8<POW2>(wd, bs);
      o[2 * d] = e.x;
      o[2 * d + 1] = e.y;
    }
    uint8_t* qp = qc + kblk_off(c0 + c, p0 + b * 32, cols);
    reinterpret_cast<uint4*>(qp)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4*>(qp)[1] = make_uint4(o[4], o[5], o[6], o[7]);
    if (b == 0) sc[p0 / 128 * cols + c0 + c] = bs.stored;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quant_dual_blk(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                 bool pow2, uint8_t* qr, float* sr, uint8_t* qc, float* sc, int64_t mpad,
                                 hipStream_t st) {
  const dim3 grid((unsigned)(mpad / 128), (unsigned)(cols / 128));
  if (pow2)
    hipLaunchKernelGGL(quant_dual_1x128_kernel<true>, grid, dim3(256), 0, st, x, ldx, rows, cols, sp, mpad, qr, sr,
                       qc, sc);
  else
    hipLaunchKernelGGL(quant_dual_1x128_kernel<false>, grid, dim3(256), 0, st, x, ldx, rows, cols, sp, mpad, qr, sr,
                       qc, sc);
  return hipGetLastError();
}

hipError_t launch_quant_rowwise_blk(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool blk128x128,
                                    bool pow2, uint8_t* q, float* s, hipStream_t st) {
  if (blk128x128) {
    const dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128));
    if (pow2)
      hipLaunchKernelGGL(quant_128x128_kernel<true>, grid, dim3(256), 0, st, x, ldx, rows, cols, q, s);
    else
      hipLaunchKernelGGL(quant_128x128_kernel<false>, grid, dim3(256), 0, st, x, ldx, rows, cols, q, s);
    return hipGetLastError();
  }
  constexpr int U = 4;
  const int cpr = (int)(cols / 8);
  const int64_t gy_need = (rows + 4 * U - 1) / (4 * U);
  const dim3 grid((unsigned)((cpr + 63) / 64), (unsigned)(gy_need < 65535 ? gy_need : 65535));
  if (pow2)
    hipLaunchKernelGGL((quant_rowwise_1x128_kernel<true, U>), grid, dim3(256), 0, st, x, ldx, (int)rows, cpr, q, s);
  else
    hipLaunchKernelGGL((quant_rowwise_1x128_kernel<false, U>), grid, dim3(256), 0, st, x, ldx, (int)rows, cpr, q, s);
  return hipGetLastError();
}

hipError_t launch_quant_colwise_blk(const uint16_t* x, int64_t cols, int64_t ldx, const SplitArgs& sp, bool pow2,
                                    uint8_t* q, float* s, int64_t mpad, hipStream_t st) {
  if (cols % 128 == 0) {  // the dual kernel without its row-wise output: 128 columns per workgroup
    const dim3 grid((unsigned)(mpad / 128), (unsigned)(cols / 128));
    if (pow2)
      hipLaunchKernelGGL((quant_dual_1x128_kernel<true, false>), grid, dim3(256), 0, st, x, ldx, (int64_t)0, cols,
                         sp, mpad, nullptr, nullptr, q, s);
    else
      hipLaunchKernelGGL((quant_dual_1x128_kernel<false, false>), grid, dim3(256), 0, st, x, ldx, (int64_t)0, cols,
                         sp, mpad, nullptr, nullptr, q, s);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(mpad / 128), (unsigned)((cols + 63) / 64));
  if (pow2)
    hipLaunchKernelGGL(quant_colwise_1x128_kernel<true>, grid, dim3(256), 0, st, x, ldx, cols, sp, mpad, q, s);
  else
    hipLaunchKernelGGL(quant_colwise_1x128_kernel<false>, grid, dim3(256), 0, st, x, ldx, cols, sp, mpad, q, s);
  return hipGetLastError();
}

hipError_t launch_transpose_128x128(const uint8_t* wq, const float* ws, int32_t G, int64_t N, int64_t K, uint8_t* tq,
                                    float* ts, hipStream_t st) {
  const int64_t blocks = (int64_t)G * (N / 128) * (K / 128);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_128x128_kernel, dim3((unsigned)blocks), dim3(256), 0, st, wq, ws, (int64_t)G, N, K, tq,
                     ts);
  return hipGetLastError();
}

}  // namespace mxgg
