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

// Eight bf16 values (four words, low half first) of one block with shared
// exponent e (scale operand sc = 2^e as fp32) -> E2M1 codes, 4 bytes, element
// order kept (low nibble first).
__device__ __forceinline__ uint32_t encode8_fp4(const uint32_t (&wd)[4], float sc) {
  uint32_t packed = 0;
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[0]), sc, 0);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[1]), sc, 1);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[2]), sc, 2);
  packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, as_bf16x2(wd[3]), sc, 3);
  return packed;
}

// ... -> E4M3 codes, 8 bytes (magnitudes clamped to 448 * 2^e first: the
// scaled conversion turns scaled magnitudes >= 464 into NaN)
__device__ __forceinline__ uint2 encode8_fp8(const uint32_t (&wd)[4], int e, float sc) {
  const uint32_t lim = e4m3_sat_limit_bits(e);
  v2s p0 = {0, 0}, p1 = {0, 0};
  p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p0, as_bf16x2(clamp_bf16x2_mag(wd[0], lim)), sc, false);
  p0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p0, as_bf16x2(clamp_bf16x2_mag(wd[1], lim)), sc, true);
  p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p1, as_bf16x2(clamp_bf16x2_mag(wd[2], lim)), sc, false);
  p1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p1, as_bf16x2(clamp_bf16x2_mag(wd[3], lim)), sc, true);
  return make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
}

// A 32-element column block (pairs[i] = elements 2i (low) and 2i+1 (high))
// encoded and stored at qp: 16 bytes (E2M1) or 32 bytes (E4M3).
template <bool FP4>
__device__ __forceinline__ void encode32_store(const uint32_t (&pairs)[16], int e, float sc, uint8_t* qp) {
  if constexpr (FP4) {
    uint32_t a[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t wd[4] = {pairs[4 * d], pairs[4 * d + 1], pairs[4 * d + 2], pairs[4 * d + 3]};
      a[d] = encode8_fp4(wd, sc);
    }
    *reinterpret_cast<uint4*>(qp) = make_uint4(a[0], a[1], a[2], a[3]);
  } else {
    uint2 a[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t wd[4] = {pairs[4 * d], pairs[4 * d + 1], pairs[4 * d + 2], pairs[4 * d + 3]};
      a[d] = encode8_fp8(wd, e, sc);
    }
    reinterpret_cast<uint4*>(qp)[0] = make_uint4(a[0].x, a[0].y, a[1].x, a[1].y);
    reinterpret_cast<uint4*>(qp)[1] = make_uint4(a[2].x, a[2].y, a[3].x, a[3].y);
  }
}

// ---------------------------------------------------------------------------
// Row-wise. A wave owns 64 consecutive 16-byte chunks (8 elements each) of one
// row, so every load instruction reads 1 KiB contiguous; 4 consecutive lanes
// hold one 32-element block and reduce amax with two xor-shuffles. Each thread
// keeps U = 4 consecutive rows' loads in flight before encoding (memory-level
// parallelism), so the four scale bytes of a block's rows are adjacent in the
// block-major scale layout and go out as one 4-byte store. In the MFMA layout
// the lane of a 128-element group's first block collects the other three
// blocks' words (lanes +4, +8, +12) and writes the group's 16 bytes of its
// four rows as two 8-byte runs (K step pairs of fragment lanes r%32 and
// r%32 + 32); the row groups then run to the 32-row padding, whose scales
// are 0.
// K-blocked codes (KB) go through LDS: the workgroup's 16 rows x 64 chunks
// are staged as [K block][row][64 bytes], so that after one barrier every
// store instruction writes 1 KiB that is contiguous in the K-blocked layout
// (the 16 rows of one K block), not 64-byte pieces of rows*64 apart.
// Grid: x over 64-chunk column groups, y over 4*U-row groups (grid-strided).
// ---------------------------------------------------------------------------
// bytes (a0 b0 a1 b1 | a2 b2 a3 b3) of two words
__device__ __forceinline__ uint2 interleave_bytes(uint32_t a, uint32_t b) {
  const uint32_t lo = (a & 0xffu) | (b & 0xffu) << 8 | (a & 0xff00u) << 8 | (b & 0xff00u) << 16;
  const uint32_t hi = (a >> 16 & 0xffu) | (b >> 16 & 0xffu) << 8 | (a >> 24) << 16 | (b >> 24) << 24;
  return make_uint2(lo, hi);
}

template <class F, int U, bool MFMA, bool KB>
__global__ __launch_bounds__(256) void quant_rowwise_kernel(const uint16_t* __restrict__ x, int64_t ldx, int rows,
                                                            int cpr, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ s, int64_t sld) {
  constexpr bool FP4 = F::MB == 1;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;  // chunk inside the row
  const bool cvalid = c < cpr;
  const int64_t qrow_bytes = FP4 ? (int64_t)cpr * 4 : (int64_t)cpr * 8;
  static_assert(U == 4, "four rows per thread: one 4-byte scale store");
  constexpr int BPC = FP4 ? 4 : 8;  // code bytes per 8-element chunk
  constexpr int CPB = 64 / BPC;     // chunks per 64-byte K block
  // K-blocked staging: 16 rows x 64 chunks x BPC bytes (64 * BPC uint4)
  __shared__ uint4 stage[KB ? 64 * BPC : 1];
  // MFMA: sld is the 128-element group stride (padded rows x 4 bytes)
  const int row_end = MFMA ? (int)(sld / 4) : rows;
  for (int rb = blockIdx.y * (4 * U); rb < row_end; rb += gridDim.y * (4 * U)) {
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
      const float sc = __uint_as_float(mx_scale_operand_bits(e));
      if constexpr (KB) {
        // every lane stages its codes (rows past the end and chunks past the
        // row are zeros and never stored); the stores follow the barrier
        uint8_t* sp = reinterpret_cast<uint8_t*>(stage) + ((lane / CPB) * 16 + w * U + u) * 64 + (lane % CPB) * BPC;
        if constexpr (FP4)
          *reinterpret_cast<uint32_t*>(sp) = encode8_fp4(wd, sc);
        else
          *reinterpret_cast<uint2*>(sp) = encode8_fp8(wd, e, sc);
        if (!(cvalid && r < rows)) continue;
      } else {
        if (!(cvalid && r < rows)) continue;
        uint8_t* qp = q + (int64_t)r * qrow_bytes + (int64_t)c * BPC;
        if constexpr (FP4)
          *reinterpret_cast<uint32_t*>(qp) = encode8_fp4(wd, sc);
        else
          *reinterpret_cast<uint2*>(qp) = encode8_fp8(wd, e, sc);
      }
      sbytes |= (uint32_t)(e + 127) << (8 * u);
    }
    const int r0 = rb + w * U;
    if constexpr (MFMA) {
      const uint32_t s1 = (uint32_t)__shfl_down((int)sbytes, 4, 64);
      const uint32_t s2 = (uint32_t)__shfl_down((int)sbytes, 8, 64);
      const uint32_t s3 = (uint32_t)__shfl_down((int)sbytes, 12, 64);
      if (cvalid && (c & 15) == 0 && r0 < row_end) {
        uint8_t* u = s + (int64_t)(c >> 4) * sld + (r0 >> 5) * 128 + (r0 & 31) * 2;
        *reinterpret_cast<uint2*>(u) = interleave_bytes(sbytes, s2);    // blocks 0, 2 (lane r%32)
        *reinterpret_cast<uint2*>(u + 64) = interleave_bytes(s1, s3);   // blocks 1, 3 (lane r%32 + 32)
      }
    } else {
      // block-major scales [cols/32, sld], sld = rows rounded up to a multiple
      // of 4: the thread's four rows are one aligned word (padding rows get 0)
      if (cvalid && (c & 3) == 0 && r0 < rows) *reinterpret_cast<uint32_t*>(s + (int64_t)(c >> 2) * sld + r0) = sbytes;
    }
    if constexpr (KB) {
      __syncthreads();
      // the tile's BPC K blocks of 16 rows: 16 bytes per thread and store,
      // 64 threads (one wave) per K block
      const int64_t nkb = (int64_t)cpr * BPC / 64;  // K blocks per row
#pragma unroll
      for (int i = 0; i < BPC / 4; ++i) {
        const int p = threadIdx.x + i * 256;
        const int rl = (p >> 2) & 15, r = rb + rl;
        const int64_t kbg = (int64_t)blockIdx.x * BPC + (p >> 6);
        if (kbg < nkb && r < rows)
          *reinterpret_cast<uint4*>(q + (kbg * rows + r) * 64 + (p & 3) * 16) = stage[p];
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Dual output: the row-wise and the column-wise segment-padded quantization of
// the same tensor from one read of it (activations and output gradients are
// quantized both ways in training; so are the weights, with segments of N
// rows). A workgroup of NT threads takes TR padded rows (TR/32 blocks of 32,
// each inside one expert segment) by TC columns:
//   load   lane groups of TC/8 lanes read one row's TC columns (16 bytes
//          each), PH phases of loads in flight;
//   rows   four consecutive lanes hold one 32-element row block: amax by two
//          xor-shuffles, encode, store, one scale byte per block;
//   tile   the bf16 values go to LDS (zeros for padding rows);
//   cols   a wave encodes one block of 64 column pairs (one 4-byte LDS read
//          per row: conflict-free), 16 or 32 bytes per column and block.
// Scale padding rows of the row-wise output (the last rows' word) are zeroed
// by the workgroup holding the tensor's last row.
// ---------------------------------------------------------------------------
template <int TR_, int TC_, int NT_, int PH_, int OCC_, int CMAP_ = 0>
struct DualCfg {
  static constexpr int TR = TR_, TC = TC_, NT = NT_, PH = PH_;
  static constexpr int OCC = OCC_;                          // workgroups per CU
  // column-wise lane map: 0, a wave takes one 32-row block of 128 columns
  // (a store instruction writes 16 bytes into each of 64 output rows);
  // 1, a lane takes one column pair of one block, four lanes the four
  // blocks of a pair (a store instruction writes 64 contiguous bytes into
  // each of 16 output rows); the LDS tile's 16-byte chunks are then XOR
  // swizzled by 4 x block so the four blocks' reads fall on distinct banks
  static constexpr int CMAP = CMAP_;
  static constexpr int CIPT = TC / 2 * (TR / 32) / NT;  // column map 1: (pair, block) items per thread
  static_assert(CMAP == 0 || (TR % 128 == 0 && TC / 2 == NT / 4 && CIPT * NT == TC / 2 * (TR / 32)),
                "column map 1 shape");
  static constexpr int PITCH = TC + 8;                      // bf16 per LDS row
  static constexpr int LDS_BYTES = TR * PITCH * 2;
  static constexpr int CPR = TC / 8;                        // 16-byte chunks per row
  static constexpr int RPP = NT / CPR;                      // rows per load pass
  static constexpr int PASSES = TR / RPP, PER_PHASE = PASSES / PH;
  static constexpr int NB = TR / 32, NW = NT / 64;
  static constexpr int WITEMS = NB * (TC / 128);            // (block, 64 column pairs) items
  static constexpr int WAVES_PER_SIMD = OCC * NW / 4;        // the register budget that allows OCC
  static_assert(OCC * (LDS_BYTES + 8 * 1024) <= 160 * 1024, "LDS per CU");
  static_assert(CPR % 4 == 0 && 64 % CPR == 0 && TR % RPP == 0 && PASSES % PH == 0, "dual tile");
  static_assert(TC % 128 == 0 && WITEMS % NW == 0, "column items per wave");
};

// The grid holds OCC workgroups per CU and each walks tiles t = blockIdx.x,
// + gridDim.x, ... in the order ORDER picks (XCD: consecutive logical ids on
// one XCD). The expert scan runs once per workgroup, and the loads of the next
// tile are issued before the column-wise pass of the current one, so they
// overlap it. ROWS = false: the column-wise output alone (qr, sr unused).
template <class F, class D, bool XCD, int ORDER, bool MFMA, bool ROWS = true, bool KBR = false, bool KBC = false>
__global__ __launch_bounds__(D::NT, D::WAVES_PER_SIMD) void quant_dual_mx_persistent(const uint16_t* __restrict__ x, int64_t ldx,
                                                                    int rows, int64_t cols, const SplitArgs sp,
                                                                    int64_t mpad, uint8_t* __restrict__ qr,
                                                                    uint8_t* __restrict__ sr,
                                                                    uint8_t* __restrict__ qc,
                                                                    uint8_t* __restrict__ sc_) {
  static_assert(D::PH == 1, "one load phase per tile");
  constexpr bool FP4 = F::MB == 1;
  constexpr int NL = D::PER_PHASE;  // loads per thread per tile
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
  uint16_t* tile = reinterpret_cast<uint16_t*>(dsm);
  __shared__ int64_t pref[kMaxExperts + 1];   // low: padded offsets, high: row offsets
  __shared__ int64_t wtot[D::NW];
  __shared__ int32_t pad_offs[kMaxExperts + 1];
  __shared__ int64_t blk_row0[2][D::NB];      // per tile parity: first source row of each 32-row block
  __shared__ int32_t blk_valid[2][D::NB];     // real rows in the block (0: outside mpad)

  const int G = sp.G;
  block_prefix64<D::NT>(G, [&](int g) {
    const int64_t m = sp.m[g];
    return (m << 32) | ((m + 31) & ~31ll);
  }, pref, wtot);
  for (int g = threadIdx.x; g <= G; g += D::NT) pad_offs[g] = (int32_t)(pref[g] & 0xffffffffll);
  __syncthreads();

  const int n_tx = (int)((mpad + D::TR - 1) / D::TR);
  const int n_ty = (int)((cols + D::TC - 1) / D::TC);
  const int total = n_tx * n_ty;
  // tile order: 0 row tiles fastest; 1 column tiles fastest; 2 groups of RB
  // row tiles x every column tile (RB * n_ty ~ the grid, so each round of
  // co-running workgroups reads whole input rows and writes RB*TR/2-byte runs
  // of every column-wise output row)
  const int RB = (int)gridDim.x / n_ty > 0 ? (int)gridDim.x / n_ty : 1;
  auto tx_of = [&](int tt) {
    if (ORDER == 0) return tt % n_tx;
    if (ORDER == 1) return tt / n_ty;
    const int blk = tt / (RB * n_ty), in = tt - blk * RB * n_ty;
    const int rbg = n_tx - blk * RB < RB ? n_tx - blk * RB : RB;
    return blk * RB + in % rbg;
  };
  auto ty_of = [&](int tt) {
    if (ORDER == 0) return tt / n_tx;
    if (ORDER == 1) return tt % n_ty;
    const int blk = tt / (RB * n_ty), in = tt - blk * RB * n_ty;
    const int rbg = n_tx - blk * RB < RB ? n_tx - blk * RB : RB;
    return in / rbg;
  };
  auto map_blocks = [&](int t, int par) {  // threads < NB
    const int64_t p0 = (int64_t)tx_of(t) * D::TR + threadIdx.x * 32;
    if (p0 < mpad) {
      const int g = upper_bound_i32(pad_offs, G + 1, (int32_t)p0) - 1;
      const int64_t local = p0 - pad_offs[g];
      const int64_t nv = (int64_t)sp.m[g] - local;
      blk_row0[par][threadIdx.x] = (pref[g] >> 32) + local;
      blk_valid[par][threadIdx.x] = nv > 32 ? 32 : (int)nv;
    } else {
      blk_row0[par][threadIdx.x] = 0;
      blk_valid[par][threadIdx.x] = 0;
    }
  };
  // XCD: the hardware deals block ids round-robin over the 8 XCDs; consecutive
  // logical ids on one XCD put adjacent row tiles (the two halves of a
  // column-wise output line) into the same L2
  const int nb = gridDim.x, bid = blockIdx.x;
  int t = (XCD && nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  if (t >= total) return;
  if (threadIdx.x < D::NB) map_blocks(t, 0);
  __syncthreads();

  const int64_t srow_ld = MFMA ? mx_rows32(rows) : mx_scale_stride(rows);
  const int ch = threadIdx.x % D::CPR, rg = threadIdx.x / D::CPR;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t qld = FP4 ? mpad / 2 : mpad;

  uint4 v[NL];
  auto issue_loads = [&](int tt, int par) {
    const int64_t c0 = (int64_t)ty_of(tt) * D::TC;
    const bool cvalid = c0 + ch * 8 < cols;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = rg + D::RPP * i;
      const int b = row >> 5, rin = row & 31;
      v[i] = make_uint4(0, 0, 0, 0);
      if (cvalid && rin < blk_valid[par][b])
        v[i] = *reinterpret_cast<const uint4*>(x + (blk_row0[par][b] + rin) * ldx + c0 + ch * 8);
    }
  };
  issue_loads(t, 0);

  for (int par = 0;; par ^= 1) {
    const int64_t pt0 = (int64_t)tx_of(t) * D::TR;
    const int64_t c0 = (int64_t)ty_of(t) * D::TC;
    const int ncol = cols - c0 < D::TC ? (int)(cols - c0) : D::TC;  // multiple of 32
    const bool cvalid = ch * 8 < ncol;
    const int tn = t + (int)gridDim.x;
    if (tn < total && threadIdx.x < D::NB) map_blocks(tn, par ^ 1);

    // row-wise from the loaded registers; the bf16 tile to LDS
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = rg + D::RPP * i;
      const int b = row >> 5, rin = row & 31;
      const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      const int pch = D::CMAP ? ch ^ (4 * ((row >> 5) & 3)) : ch;  // physical 16-byte chunk
      uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * D::PITCH + pch * 8);
      dst[0] = v[i].x; dst[1] = v[i].y; dst[2] = v[i].z; dst[3] = v[i].w;
      if constexpr (!ROWS) continue;
      uint32_t amax = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) amax = max(amax, max(wd[k] & 0x7fffu, (wd[k] >> 16) & 0x7fffu));
      amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, 64));
      amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, 64));
      if (!(cvalid && rin < blk_valid[par][b])) continue;
      const int64_t r = blk_row0[par][b] + rin;
      const int e = mx_shared_exp<F>(amax);
      const float sc = __uint_as_float(mx_scale_operand_bits(e));
      const int64_t qb = FP4 ? c0 / 2 + ch * 4 : c0 + ch * 8;  // first code byte in the row
      uint8_t* qp = qr + (KBR ? kblk_off(r, qb, rows) : r * (FP4 ? cols / 2 : cols) + qb);
      if constexpr (FP4)
        *reinterpret_cast<uint32_t*>(qp) = encode8_fp4(wd, sc);
      else
        *reinterpret_cast<uint2*>(qp) = encode8_fp8(wd, e, sc);
      if ((ch & 3) == 0) {
        const int64_t blk = (c0 + ch * 8) >> 5;
        if constexpr (MFMA) {
          sr[mfma_scale_offset(r, blk, srow_ld)] = (uint8_t)(e + 127);
          if (r == rows - 1)  // the 32-row padding
            for (int64_t k = r + 1; k < srow_ld; ++k) sr[mfma_scale_offset(k, blk, srow_ld)] = 0;
        } else {
          uint8_t* sp_ = sr + blk * srow_ld + r;
          sp_[0] = (uint8_t)(e + 127);
          if (r == rows - 1)  // the padding rows of the last word
            for (int64_t k = 1; r + k < srow_ld; ++k) sp_[k] = 0;
        }
      }
    }
    __syncthreads();  // tile in LDS; the next tile's block map visible
    if (tn < total) issue_loads(tn, par ^ 1);

    // column-wise from LDS while the next tile's loads are in flight
    if constexpr (D::CMAP == 1) {
#pragma unroll
      for (int it = 0; it < D::CIPT; ++it) {
      const int b = (lane & 3) + 4 * it, pr = wv * 16 + (lane >> 2);  // block, column pair
      const int64_t p0 = pt0 + b * 32;
      const int c = 2 * pr;
      if (p0 < mpad && c < ncol) {
        uint32_t w2[32];
        uint32_t a0 = 0, a1 = 0;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          const int row = b * 32 + r;
          w2[r] = *reinterpret_cast<const uint32_t*>(tile + row * D::PITCH + ((c >> 3) ^ (4 * (b & 3))) * 8 + (c & 7));
          a0 = max(a0, w2[r] & 0x7fffu);
          a1 = max(a1, (w2[r] >> 16) & 0x7fffu);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int e = mx_shared_exp<F>(j ? a1 : a0);
          const float sc = __uint_as_float(mx_scale_operand_bits(e));
          uint32_t pairs[16];
#pragma unroll
          for (int i = 0; i < 16; ++i)
            pairs[i] = j ? (w2[2 * i] >> 16) | (w2[2 * i + 1] & 0xffff0000u)
                         : (w2[2 * i] & 0xffffu) | (w2[2 * i + 1] << 16);
          encode32_store<FP4>(pairs, e, sc,
                              qc + (KBC ? kblk_off(c0 + c + j, FP4 ? p0 / 2 : p0, cols)
                                        : (c0 + c + j) * qld + (FP4 ? p0 / 2 : p0)));
          if constexpr (MFMA)
            sc_[mfma_scale_offset(c0 + c + j, p0 / 32, cols)] = (uint8_t)(e + 127);
          else
            sc_[(p0 / 32) * cols + c0 + c + j] = (uint8_t)(e + 127);
        }
      }
      }
    } else {
#pragma unroll
      for (int it = 0; it < D::WITEMS / D::NW; ++it) {
        const int item = wv + it * D::NW;
        const int b = item % D::NB, cq = item / D::NB;
        const int64_t p0 = pt0 + b * 32;
        const int c = cq * 128 + 2 * lane;
        if (p0 >= mpad || c >= ncol) continue;
        uint32_t w2[32];
        uint32_t a0 = 0, a1 = 0;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          w2[r] = *reinterpret_cast<const uint32_t*>(tile + (b * 32 + r) * D::PITCH + c);
          a0 = max(a0, w2[r] & 0x7fffu);
          a1 = max(a1, (w2[r] >> 16) & 0x7fffu);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int e = mx_shared_exp<F>(j ? a1 : a0);
          const float sc = __uint_as_float(mx_scale_operand_bits(e));
          uint32_t pairs[16];
#pragma unroll
          for (int i = 0; i < 16; ++i)  // rows 2i (low) and 2i+1 (high) of column c + j
            pairs[i] = j ? (w2[2 * i] >> 16) | (w2[2 * i + 1] & 0xffff0000u)
                         : (w2[2 * i] & 0xffffu) | (w2[2 * i + 1] << 16);
          encode32_store<FP4>(pairs, e, sc,
                              qc + (KBC ? kblk_off(c0 + c + j, FP4 ? p0 / 2 : p0, cols)
                                        : (c0 + c + j) * qld + (FP4 ? p0 / 2 : p0)));
          if constexpr (MFMA)
            sc_[mfma_scale_offset(c0 + c + j, p0 / 32, cols)] = (uint8_t)(e + 127);
          else
            sc_[(p0 / 32) * cols + c0 + c + j] = (uint8_t)(e + 127);
        }
      }
    }
    if (tn >= total) break;
    t = tn;
    __syncthreads();  // every wave done reading the LDS tile
  }
}

template <class D, bool XCD, int ORDER, bool MFMA, bool ROWS = true, bool KBR = false, bool KBC = false>
hipError_t launch_quant_dual_persistent(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                        const SplitArgs& sp, bool fp8, uint8_t* qr, uint8_t* sr, uint8_t* qc,
                                        uint8_t* sc, int64_t mpad, int num_cus, hipStream_t st) {
  auto kern = fp8 ? quant_dual_mx_persistent<E4M3Fmt, D, XCD, ORDER, MFMA, ROWS, KBR, KBC>
                  : quant_dual_mx_persistent<E2M1Fmt, D, XCD, ORDER, MFMA, ROWS, KBR, KBC>;
  const hipError_t e = ensure_dynamic_lds((const void*)kern, D::LDS_BYTES, st);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((mpad + D::TR - 1) / D::TR) * ((cols + D::TC - 1) / D::TC);
  int64_t grid = (int64_t)num_cus * D::OCC;
  if (tiles < grid) grid = tiles;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(D::NT), D::LDS_BYTES, st, x, ldx, (int)rows, cols, sp, mpad,
                     qr, sr, qc, sc);
  return hipGetLastError();
}

// 128 padded rows x 256 columns, 512 threads (one load per thread per 16
// rows), one workgroup per CU, column tiles fastest, the column-pair lane map
// of the column-wise pass: measured at the fc1 sizes X 99 us, dY 79 us, W
// 260 us (103 / 82 / 277 us with a wave per 32-row block of 128 columns),
// against 168 / 96 / 484 us for the two single-output kernels.
using DualCfgProduct = DualCfg<128, 256, 512, 1, 1, 1>;

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <bool MFMA, bool KB>
static void launch_rowwise_as(const uint16_t* x, int64_t rows, int64_t ldx, int cpr, bool fp8, uint8_t* q,
                              uint8_t* s, int64_t sld, hipStream_t st) {
  constexpr int U = 4;
  const int64_t row_end = MFMA ? sld / 4 : rows;
  const int64_t gy_need = (row_end + 4 * U - 1) / (4 * U);
  const dim3 grid((unsigned)((cpr + 63) / 64), (unsigned)(gy_need < 65535 ? gy_need : 65535));
  if (fp8)
    hipLaunchKernelGGL((quant_rowwise_kernel<E4M3Fmt, U, MFMA, KB>), grid, dim3(256), 0, st, x, ldx, (int)rows, cpr,
                       q, s, sld);
  else
    hipLaunchKernelGGL((quant_rowwise_kernel<E2M1Fmt, U, MFMA, KB>), grid, dim3(256), 0, st, x, ldx, (int)rows, cpr,
                       q, s, sld);
}

hipError_t launch_quant_rowwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, bool fp8, bool mfma,
                                   bool kb, uint8_t* q, uint8_t* s, int num_cus, hipStream_t st) {
  (void)num_cus;
  const int cpr = (int)(cols / 8);
  const int64_t m32 = mx_rows32(rows) * 4, r4 = mx_scale_stride(rows);
  if (mfma && kb) launch_rowwise_as<true, true>(x, rows, ldx, cpr, fp8, q, s, m32, st);
  else if (mfma) launch_rowwise_as<true, false>(x, rows, ldx, cpr, fp8, q, s, m32, st);
  else if (kb) launch_rowwise_as<false, true>(x, rows, ldx, cpr, fp8, q, s, r4, st);
  else launch_rowwise_as<false, false>(x, rows, ldx, cpr, fp8, q, s, r4, st);
  return hipGetLastError();
}

// The dual kernel for each scale layout and code layout of its two outputs.
template <bool MFMA>
static hipError_t launch_dual_as(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                 bool fp8, bool kbr, bool kbc, uint8_t* qr, uint8_t* sr, uint8_t* qc, uint8_t* sc,
                                 int64_t mpad, int num_cus, hipStream_t st) {
  using D = DualCfgProduct;
  if (kbr && kbc)
    return launch_quant_dual_persistent<D, false, 1, MFMA, true, true, true>(x, rows, cols, ldx, sp, fp8, qr, sr, qc,
                                                                             sc, mpad, num_cus, st);
  if (kbr)
    return launch_quant_dual_persistent<D, false, 1, MFMA, true, true, false>(x, rows, cols, ldx, sp, fp8, qr, sr,
                                                                              qc, sc, mpad, num_cus, st);
  if (kbc)
    return launch_quant_dual_persistent<D, false, 1, MFMA, true, false, true>(x, rows, cols, ldx, sp, fp8, qr, sr,
                                                                              qc, sc, mpad, num_cus, st);
  return launch_quant_dual_persistent<D, false, 1, MFMA, true, false, false>(x, rows, cols, ldx, sp, fp8, qr, sr, qc,
                                                                             sc, mpad, num_cus, st);
}

hipError_t launch_quant_dual_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                bool fp8, bool mfma, bool kbr, bool kbc, uint8_t* qr, uint8_t* sr, uint8_t* qc,
                                uint8_t* sc, int64_t mpad, int num_cus, hipStream_t st) {
  if (mfma) return launch_dual_as<true>(x, rows, cols, ldx, sp, fp8, kbr, kbc, qr, sr, qc, sc, mpad, num_cus, st);
  return launch_dual_as<false>(x, rows, cols, ldx, sp, fp8, kbr, kbc, qr, sr, qc, sc, mpad, num_cus, st);
}

// Column-wise alone: the dual kernel without its row-wise output (one read of
// the tile, the column-wise pass from LDS while the next tile's loads are in
// flight). Measured against a one-tile-per-workgroup transpose kernel: fc1 W
// 300 -> 204 us, X 122 -> 76 us, dY 85 -> 72 us; a8w4 W 1.34 -> 1.14 ms.
hipError_t launch_quant_colwise_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, const SplitArgs& sp,
                                   bool fp8, bool mfma, bool kbc, uint8_t* q, uint8_t* s, int64_t mpad, int num_cus,
                                   hipStream_t st) {
  using D = DualCfgProduct;
  if (mfma && kbc)
    return launch_quant_dual_persistent<D, false, 1, true, false, false, true>(x, rows, cols, ldx, sp, fp8, nullptr,
                                                                              nullptr, q, s, mpad, num_cus, st);
  if (mfma)
    return launch_quant_dual_persistent<D, false, 1, true, false>(x, rows, cols, ldx, sp, fp8, nullptr, nullptr, q,
                                                                  s, mpad, num_cus, st);
  if (kbc)
    return launch_quant_dual_persistent<D, false, 1, false, false, false, true>(x, rows, cols, ldx, sp, fp8, nullptr,
                                                                               nullptr, q, s, mpad, num_cus, st);
  return launch_quant_dual_persistent<D, false, 1, false, false>(x, rows, cols, ldx, sp, fp8, nullptr, nullptr, q, s,
                                                                 mpad, num_cus, st);
}

}  // namespace mxgg

namespace mxgg {

// ---------------------------------------------------------------------------
// MX scale relayout between the three layouts: row-major u8 [rows, blocks],
// block-major u8 [blocks, R4] and the MFMA layout u8 [blocks/4, R32/32, 64,
// 2] (padding rows 0). A 64 x 64 (row, block) byte tile per workgroup goes
// through LDS; the row-major side is read and written along blocks, the other
// two along rows.
// ---------------------------------------------------------------------------
enum { kLayBlock = 0, kLayRow = 1, kLayMfma = 2 };

template <int L>
__device__ __forceinline__ int64_t scale_offset(int64_t r, int64_t b, int64_t blocks, int64_t r4, int64_t r32) {
  if constexpr (L == kLayRow) return r * blocks + b;
  else if constexpr (L == kLayBlock) return b * r4 + r;
  else return mfma_scale_offset(r, b, r32);
}

template <int SRC, int DST>
__global__ __launch_bounds__(256) void relayout_scales_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                              int64_t blocks, int64_t r4, int64_t r32,
                                                              uint8_t* __restrict__ dst) {
  __shared__ uint8_t t[64][65];
  const int64_t r0 = (int64_t)blockIdx.x * 64, b0 = (int64_t)blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = SRC == kLayRow ? i >> 6 : i & 63, b = SRC == kLayRow ? i & 63 : i >> 6;
    const int64_t rr = r0 + r, bb = b0 + b;
    t[r][b] = (rr < rows && bb < blocks) ? src[scale_offset<SRC>(rr, bb, blocks, r4, r32)] : (uint8_t)0;
  }
  __syncthreads();
  // rows written: the destination's padded row count (padding rows get 0)
  const int64_t rend = DST == kLayRow ? rows : DST == kLayBlock ? r4 : r32;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = DST == kLayRow ? i >> 6 : i & 63, b = DST == kLayRow ? i & 63 : i >> 6;
    const int64_t rr = r0 + r, bb = b0 + b;
    if (rr < rend && bb < blocks) dst[scale_offset<DST>(rr, bb, blocks, r4, r32)] = t[r][b];
  }
}

static int layout_id(int mxgg_layout) {
  return mxgg_layout == 0x100 ? kLayRow : mxgg_layout == 0x200 ? kLayMfma : kLayBlock;
}

template <int SRC, int DST>
static void launch_relayout_as(const uint8_t* src, int64_t rows, int64_t blocks, uint8_t* dst, hipStream_t st) {
  const int64_t r4 = mx_scale_stride(rows), r32 = mx_rows32(rows);
  const dim3 grid((unsigned)((r32 + 63) / 64), (unsigned)((blocks + 63) / 64));
  hipLaunchKernelGGL((relayout_scales_kernel<SRC, DST>), grid, dim3(256), 0, st, src, rows, blocks, r4, r32, dst);
}

hipError_t launch_relayout_scales(const uint8_t* src, int src_layout, int64_t rows, int64_t blocks, int dst_layout,
                                  uint8_t* dst, hipStream_t st) {
  const int s = layout_id(src_layout), d = layout_id(dst_layout);
  if (s == kLayRow && d == kLayBlock) launch_relayout_as<kLayRow, kLayBlock>(src, rows, blocks, dst, st);
  else if (s == kLayRow && d == kLayMfma) launch_relayout_as<kLayRow, kLayMfma>(src, rows, blocks, dst, st);
  else if (s == kLayBlock && d == kLayRow) launch_relayout_as<kLayBlock, kLayRow>(src, rows, blocks, dst, st);
  else if (s == kLayBlock && d == kLayMfma) launch_relayout_as<kLayBlock, kLayMfma>(src, rows, blocks, dst, st);
  else if (s == kLayMfma && d == kLayRow) launch_relayout_as<kLayMfma, kLayRow>(src, rows, blocks, dst, st);
  else if (s == kLayMfma && d == kLayBlock) launch_relayout_as<kLayMfma, kLayBlock>(src, rows, blocks, dst, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mxgg
