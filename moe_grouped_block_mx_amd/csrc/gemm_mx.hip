// Grouped block-scaled (MX) GEMMs for gfx950: forward, input gradient and
// variable-K weight gradient in one launch each.
//
// Method (see the pages "Triton mxfp4 (and a8w4) grouped GEMM kernel" and
// "Grouped MXFP8 GEMMs with HipKittens"): a persistent grid walks all output
// tiles of all experts; a tile index maps to its expert with an upper_bound
// search over the prefix sum of per-expert tile counts, built in LDS by every
// workgroup from the split counts passed as kernel arguments. Every output
// element belongs to exactly one tile and is stored under masks on
// un-wrapped indices (the tail-tile rule of "Add ROCm Triton blockwise FP8
// grouped GEMM").
//
// All three passes are "TN" on quantized data (MX scales run along the
// contraction axis, so both operands are contraction-contiguous); only the
// tile scheduler and the epilogue differ between them.
//
// Tile: BM x BN outputs per workgroup, WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) block of 32x32 fragments computed with the CDNA4
// instruction v_mfma_scale_f32_32x32x64_f8f6f4. Measured operand layout of
// that instruction (32x32x64): lane l holds row l % 32 of its operand; for
// E2M1 the 16 bytes at byte offset 16*(l/32) of the row's 32-byte K chunk,
// for E4M3 the 16 bytes at 16*(l/32) and at 32 + 16*(l/32) of the 64-byte
// chunk; the scale byte (selected by op_sel) of lane l applies to row l % 32,
// K-block l/32; result register i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
// column l % 32.
//
// Per K stage (BK elements) the workgroup copies the A and B tiles from HBM
// into registers (16-byte coalesced loads), then into a double-buffered,
// XOR-swizzled LDS tile, while each lane fetches its own scale bytes
// (one per fragment per 32-element block) straight into registers and packs
// the K stage's bytes so op_sel picks the right one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace mxgg {

// Calls f(std::integral_constant<int, I>) for I = 0..N-1: the index is a
// compile-time constant, so arrays indexed by it stay in registers regardless
// of the loop-unrolling heuristics.
template <class F, int... Is>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BM_, int BN_, int WM_, int WN_, int BK_, bool AFP8_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_;
  static constexpr bool AFP8 = AFP8_;
  static constexpr int THREADS = 64 * WM * WN;
  static constexpr int RBA = AFP8 ? BK : BK / 2;  // A bytes per row per stage
  static constexpr int RBB = BK / 2;              // B (E2M1) bytes per row per stage
  static constexpr int CPA = RBA / 16, CPB = RBB / 16;
  static constexpr int KSTEPS = BK / 64;          // MFMA K steps per stage
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int NLA = BM * CPA / THREADS;  // 16-byte loads per thread per stage
  static constexpr int NLB = BN * CPB / THREADS;
  static constexpr int RSA = THREADS / CPA, RSB = THREADS / CPB;
  static constexpr int LDS_A = BM * RBA, LDS_B = BN * RBB;
  static_assert(BM * CPA % THREADS == 0 && BN * CPB % THREADS == 0, "load split");
  static_assert(THREADS % CPA == 0 && THREADS % CPB == 0, "load rows");
  static_assert(KSTEPS >= 1 && KSTEPS <= 4, "scale bytes per word");
  static_assert(FM >= 1 && FN >= 1, "fragments");
};

// Per-thread state of one tile's main loop.
template <class C>
struct LoopState {
  uint32_t pa[C::NLA], pb[C::NLB];     // byte offsets of this thread's copy rows
  uint32_t psa[C::FM], psb[C::FN];     // byte offsets of this lane's scale rows
  v4i ra[C::NLA], rb[C::NLB];          // staged 16-byte chunks of the next stage
  uint32_t sa_cur[C::FM], sb_cur[C::FN];           // packed scale words in use
  uint32_t sa_raw[C::FM][C::KSTEPS], sb_raw[C::FN][C::KSTEPS];  // next stage, unpacked
};

template <class C>
__device__ __forceinline__ void stage_gload(LoopState<C>& st, const uint8_t* __restrict__ A,
                                            const uint8_t* __restrict__ B, int s, int kca, int kcb) {
  const int tid = threadIdx.x;
  if ((s + 1) * C::RBA <= kca) {  // whole stage inside the contraction (uniform branch)
#pragma unroll
    for (int i = 0; i < C::NLA; ++i) st.ra[i] = *reinterpret_cast<const v4i*>(A + st.pa[i] + s * C::RBA);
#pragma unroll
    for (int i = 0; i < C::NLB; ++i) st.rb[i] = *reinterpret_cast<const v4i*>(B + st.pb[i] + s * C::RBB);
    return;
  }
  const int ka = s * C::RBA + (tid % C::CPA) * 16;
  const int kb = s * C::RBB + (tid % C::CPB) * 16;
#pragma unroll
  for (int i = 0; i < C::NLA; ++i)
    st.ra[i] = (ka < kca) ? *reinterpret_cast<const v4i*>(A + st.pa[i] + s * C::RBA) : v4i{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < C::NLB; ++i)
    st.rb[i] = (kb < kcb) ? *reinterpret_cast<const v4i*>(B + st.pb[i] + s * C::RBB) : v4i{0, 0, 0, 0};
}

// Scale bytes of stage s: for K step kk, lane half h uses block 2*kk + h of
// the stage. Loads are branch-free (the block index is clamped into the row)
// and stay unpacked until the stage is consumed, so waiting on them never
// waits on the data prefetch issued alongside.
template <class C, int NF>
__device__ __forceinline__ void stage_sload(const uint32_t (&ps)[NF], const uint8_t* __restrict__ S,
                                            uint32_t (&raw)[NF][C::KSTEPS], int s, int nblk) {
  const int h = (threadIdx.x & 63) >> 5;
  const int blk0 = s * (C::BK / 32) + h;
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    int blk = blk0 + 2 * kk;
    blk = blk < nblk ? blk : nblk - 1;
#pragma unroll
    for (int i = 0; i < NF; ++i) raw[i][kk] = S[ps[i] + blk];
  }
}

// Packs stage s's scale bytes (byte kk = K step kk); blocks past the
// contraction end get byte 127 (their data is zero).
template <class C, int NF>
__device__ __forceinline__ void stage_spack(const uint32_t (&raw)[NF][C::KSTEPS], uint32_t (&out)[NF], int s,
                                            int nblk) {
  const int h = (threadIdx.x & 63) >> 5;
  const int blk0 = s * (C::BK / 32) + h;
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) w |= (blk0 + 2 * kk < nblk ? raw[i][kk] : 127u) << (8 * kk);
    out[i] = w;
  }
}

template <class C>
__device__ __forceinline__ void stage_lstore(const LoopState<C>& st, uint8_t* la, uint8_t* lb) {
  const int tid = threadIdx.x;
  const int ca = tid % C::CPA, ra0 = tid / C::CPA;
  const int cb = tid % C::CPB, rb0 = tid / C::CPB;
#pragma unroll
  for (int i = 0; i < C::NLA; ++i) {
    const int r = ra0 + i * C::RSA;
    *reinterpret_cast<v4i*>(la + r * C::RBA + swz<C::CPA>(r, ca) * 16) = st.ra[i];
  }
#pragma unroll
  for (int i = 0; i < C::NLB; ++i) {
    const int r = rb0 + i * C::RSB;
    *reinterpret_cast<v4i*>(lb + r * C::RBB + swz<C::CPB>(r, cb) * 16) = st.rb[i];
  }
}

// One MFMA K step (64 contraction elements) of the wave's fragments.
template <class C, int KK>
__device__ __forceinline__ void kstep(const uint8_t* la, const uint8_t* lb, const uint32_t (&sa)[C::FM],
                                      const uint32_t (&sb)[C::FN], v16f (&acc)[C::FM][C::FN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int h = lane >> 5, l32 = lane & 31;
  v8i af[C::FM], bf[C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int r = wm * C::WTM + i * 32 + l32;
    if constexpr (C::AFP8) {
      const v4i lo = *reinterpret_cast<const v4i*>(la + r * C::RBA + swz<C::CPA>(r, 4 * KK + h) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(la + r * C::RBA + swz<C::CPA>(r, 4 * KK + 2 + h) * 16);
      af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const v4i lo = *reinterpret_cast<const v4i*>(la + r * C::RBA + swz<C::CPA>(r, 2 * KK + h) * 16);
      af[i] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int r = wn * C::WTN + j * 32 + l32;
    const v4i lo = *reinterpret_cast<const v4i*>(lb + r * C::RBB + swz<C::CPB>(r, 2 * KK + h) * 16);
    bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
  }
  unroll<C::FM>([&](auto ic) {
    unroll<C::FN>([&](auto jc) {
      constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], C::AFP8 ? 0 : 4, 4, KK,
                                                                  (int)sa[i], KK, (int)sb[j]);
    });
  });
}

template <class C>
__device__ __forceinline__ void stage_compute(const uint8_t* la, const uint8_t* lb, const uint32_t (&sa)[C::FM],
                                              const uint32_t (&sb)[C::FN], v16f (&acc)[C::FM][C::FN]) {
  kstep<C, 0>(la, lb, sa, sb, acc);
  if constexpr (C::KSTEPS > 1) kstep<C, 1>(la, lb, sa, sb, acc);
  if constexpr (C::KSTEPS > 2) kstep<C, 2>(la, lb, sa, sb, acc);
  if constexpr (C::KSTEPS > 3) kstep<C, 3>(la, lb, sa, sb, acc);
}

// One output tile: acc += A_tile . B_tile^T over kc contraction elements.
//   A rows [0, mrows) of A (row stride lda), scales AS (row stride ldas);
//   B rows [0, nrows) likewise. Rows beyond mrows / nrows read the last valid
//   row (their results are never stored). Contraction positions at or beyond
//   kc read zeros (scale byte 127), so the tail adds nothing.
//   Byte offsets inside a tile are 32-bit: the ABI bounds row strides so a
//   tile's rows span less than 4 GiB.
template <class C>
__device__ __forceinline__ void tile_mainloop(const uint8_t* __restrict__ A, int64_t lda,
                                              const uint8_t* __restrict__ AS, int64_t ldas, int mrows,
                                              const uint8_t* __restrict__ B, int64_t ldb,
                                              const uint8_t* __restrict__ BS, int64_t ldbs, int nrows, int kc,
                                              uint8_t* lds_a, uint8_t* lds_b, v16f (&acc)[C::FM][C::FN]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int l32 = lane & 31;
  const int nstages = (kc + C::BK - 1) / C::BK;
  if (nstages == 0) return;
  const int kca = C::AFP8 ? kc : kc / 2;  // valid A bytes per row
  const int kcb = kc / 2;                 // valid B bytes per row
  const int nblk = kc / 32;               // valid scale blocks

  LoopState<C> st;
  {
    const int ca = tid % C::CPA, ra0 = tid / C::CPA;
    const int cb = tid % C::CPB, rb0 = tid / C::CPB;
#pragma unroll
    for (int i = 0; i < C::NLA; ++i) {
      int r = ra0 + i * C::RSA;
      r = r < mrows ? r : mrows - 1;
      st.pa[i] = (uint32_t)(r * lda) + ca * 16;
    }
#pragma unroll
    for (int i = 0; i < C::NLB; ++i) {
      int r = rb0 + i * C::RSB;
      r = r < nrows ? r : nrows - 1;
      st.pb[i] = (uint32_t)(r * ldb) + cb * 16;
    }
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      int r = wm * C::WTM + i * 32 + l32;
      r = r < mrows ? r : mrows - 1;
      st.psa[i] = (uint32_t)(r * ldas);
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      int r = wn * C::WTN + j * 32 + l32;
      r = r < nrows ? r : nrows - 1;
      st.psb[j] = (uint32_t)(r * ldbs);
    }
  }

  stage_gload<C>(st, A, B, 0, kca, kcb);
  stage_sload<C>(st.psa, AS, st.sa_raw, 0, nblk);
  stage_sload<C>(st.psb, BS, st.sb_raw, 0, nblk);
  stage_lstore<C>(st, lds_a, lds_b);
  stage_spack<C>(st.sa_raw, st.sa_cur, 0, nblk);
  stage_spack<C>(st.sb_raw, st.sb_cur, 0, nblk);
  __syncthreads();
  if (nstages > 1) {
    stage_gload<C>(st, A, B, 1, kca, kcb);
    stage_sload<C>(st.psa, AS, st.sa_raw, 1, nblk);
    stage_sload<C>(st.psb, BS, st.sb_raw, 1, nblk);
  }
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    stage_compute<C>(lds_a + buf * C::LDS_A, lds_b + buf * C::LDS_B, st.sa_cur, st.sb_cur, acc);
    if (s + 1 < nstages) {
      stage_lstore<C>(st, lds_a + (buf ^ 1) * C::LDS_A, lds_b + (buf ^ 1) * C::LDS_B);
      stage_spack<C>(st.sa_raw, st.sa_cur, s + 1, nblk);
      stage_spack<C>(st.sb_raw, st.sb_cur, s + 1, nblk);
    }
    __syncthreads();
    if (s + 2 < nstages) {
      stage_gload<C>(st, A, B, s + 2, kca, kcb);
      stage_sload<C>(st.psa, AS, st.sa_raw, s + 2, nblk);
      stage_sload<C>(st.psb, BS, st.sb_raw, s + 2, nblk);
    }
  }
}

// Block index -> logical index so that the 32 workgroups resident on one XCD
// (the hardware deals consecutive ids round-robin over the 8 XCDs) take
// consecutive tile ids and share operands in that XCD's L2.
__device__ __forceinline__ int xcd_logical_block() {
  const int nb = gridDim.x, b = blockIdx.x;
  return (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
}

// ---------------------------------------------------------------------------
// forward / input gradient
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void grouped_rows_kernel(const RowsGemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * C::LDS_A];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * C::LDS_B];
  __shared__ int64_t pref[kMaxExperts + 1];
  __shared__ int64_t wtot[C::THREADS / 64];
  __shared__ int32_t tile_offs[kMaxExperts + 1];

  const int G = p.sp.G;
  const int n_tiles = (p.n_out + C::BN - 1) / C::BN;
  // packed prefix: high half = row offset, low half = M-tile offset
  block_prefix64<C::THREADS>(G, [&](int g) {
    const int64_t m = p.sp.m[g];
    return (m << 32) | ((m + C::BM - 1) / C::BM);
  }, pref, wtot);
  for (int g = threadIdx.x; g <= G; g += C::THREADS) tile_offs[g] = (int32_t)(pref[g] & 0xffffffffll) * n_tiles;
  __syncthreads();
  const int total = tile_offs[G];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int h = lane >> 5, l32 = lane & 31;

  for (int t = xcd_logical_block(); t < total; t += gridDim.x) {
    const int g = upper_bound_i32(tile_offs, G + 1, t) - 1;
    const int local = t - tile_offs[g];
    const int mt = local / n_tiles, nt = local - mt * n_tiles;
    const int64_t row0 = (pref[g] >> 32) + (int64_t)mt * C::BM;
    const int mleft = p.sp.m[g] - mt * C::BM;
    const int mrows = mleft < C::BM ? mleft : C::BM;
    const int col0 = nt * C::BN;
    const int nleft = p.n_out - col0;
    const int ncols = nleft < C::BN ? nleft : C::BN;

    v16f acc[C::FM][C::FN];
    unroll<C::FM>([&](auto ic) { unroll<C::FN>([&](auto jc) { acc[ic][jc] = v16f{}; }); });

    tile_mainloop<C>(p.a + row0 * p.lda, p.lda, p.as + row0 * p.ldas, p.ldas, mrows,
                     p.b + (int64_t)g * p.b_gstride + (int64_t)col0 * p.ldb, p.ldb,
                     p.bs + (int64_t)g * p.bs_gstride + (int64_t)col0 * p.ldbs, p.ldbs, ncols, p.kc, lds_a, lds_b,
                     acc);

    uint16_t* cbase = p.c + row0 * p.ldc + col0;
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      unroll<C::FN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int c = wn * C::WTN + j * 32 + l32;
        const v16f v = acc[i][j];
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const int row = wm * C::WTM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < mrows && c < ncols) cbase[(int64_t)row * p.ldc + c] = f32_to_bf16_rne(v[r]);
        });
      });
    });
  }
}

// ---------------------------------------------------------------------------
// variable-K weight gradient
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void grouped_wgrad_kernel(const WgradParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * C::LDS_A];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * C::LDS_B];
  __shared__ int64_t pad_pref[kMaxExperts + 1];   // natural expert order: padded offsets
  __shared__ int64_t tile_pref[kMaxExperts + 1];  // longest-first order: tile offsets
  __shared__ int64_t wtot[C::THREADS / 64];
  __shared__ int32_t tile_offs[kMaxExperts + 1];

  const int G = p.sp.G;
  const int tr = (p.n_rows + C::BM - 1) / C::BM, tc = (p.n_cols + C::BN - 1) / C::BN;
  block_prefix64<C::THREADS>(G, [&](int g) { return (int64_t)((p.sp.m[g] + 31) & ~31); }, pad_pref, wtot);
  block_prefix64<C::THREADS>(G, [&](int j) {
    const int g = p.order[j];
    return (int64_t)((p.sp.m[g] > 0 || !p.accumulate) ? tr * tc : 0);
  }, tile_pref, wtot);
  for (int j = threadIdx.x; j <= G; j += C::THREADS) tile_offs[j] = (int32_t)tile_pref[j];
  __syncthreads();
  const int total = tile_offs[G];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int h = lane >> 5, l32 = lane & 31;
  constexpr int ABYTE_NUM = C::AFP8 ? 1 : 1, ABYTE_DEN = C::AFP8 ? 1 : 2;

  for (int t = xcd_logical_block(); t < total; t += gridDim.x) {
    const int j = upper_bound_i32(tile_offs, G + 1, t) - 1;
    const int g = p.order[j];
    const int local = t - tile_offs[j];
    const int rt = local / tc, ct = local - rt * tc;
    const int row0 = rt * C::BM, col0 = ct * C::BN;
    const int rleft = p.n_rows - row0, cleft = p.n_cols - col0;
    const int mrows = rleft < C::BM ? rleft : C::BM;
    const int ncols = cleft < C::BN ? cleft : C::BN;
    const int64_t p0 = pad_pref[g];                 // segment start (padded)
    const int kc = (int)(pad_pref[g + 1] - p0);    // padded segment length

    v16f acc[C::FM][C::FN];
    unroll<C::FM>([&](auto ic) { unroll<C::FN>([&](auto jc) { acc[ic][jc] = v16f{}; }); });

    tile_mainloop<C>(p.a + (int64_t)row0 * p.lda + p0 * ABYTE_NUM / ABYTE_DEN, p.lda,
                     p.as + (int64_t)row0 * p.ldas + p0 / 32, p.ldas, mrows,
                     p.b + (int64_t)col0 * p.ldb + p0 / 2, p.ldb, p.bs + (int64_t)col0 * p.ldbs + p0 / 32, p.ldbs,
                     ncols, kc, lds_a, lds_b, acc);

    const int64_t obase = ((int64_t)g * p.n_rows + row0) * p.n_cols + col0;
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      unroll<C::FN>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        const int c = wn * C::WTN + jj * 32 + l32;
        const v16f v = acc[i][jj];
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const int row = wm * C::WTM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < mrows && c < ncols) {
            const int64_t idx = obase + (int64_t)row * p.n_cols + c;
            if (p.out_bf16) {
              uint16_t* o = reinterpret_cast<uint16_t*>(p.c) + idx;
              float x = v[r];
              if (p.accumulate) x += __uint_as_float((uint32_t)(*o) << 16);
              *o = f32_to_bf16_rne(x);
            } else {
              float* o = reinterpret_cast<float*>(p.c) + idx;
              *o = p.accumulate ? *o + v[r] : v[r];
            }
          }
        });
      });
    });
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
using CfgFwd4 = TileCfg<256, 256, 2, 2, 128, false>;   // a4w4
using CfgFwd8 = TileCfg<256, 256, 2, 2, 128, true>;    // a8w4

static int grid_for(int64_t tiles, int num_cus) {
  int64_t g = num_cus;
  if (tiles < g) g = tiles;
  if (g < 1) g = 1;
  return (int)g;
}

static int64_t rows_tiles(const RowsGemmParams& p, int BM, int BN) {
  int64_t mt = 0;
  for (int g = 0; g < p.sp.G; ++g) mt += (p.sp.m[g] + BM - 1) / BM;
  return mt * ((p.n_out + BN - 1) / BN);
}

hipError_t launch_grouped_rows_mx(const RowsGemmParams& p, bool a_fp8, int num_cus, hipStream_t st) {
  if (a_fp8) {
    const int grid = grid_for(rows_tiles(p, CfgFwd8::BM, CfgFwd8::BN), num_cus);
    hipLaunchKernelGGL(grouped_rows_kernel<CfgFwd8>, dim3(grid), dim3(CfgFwd8::THREADS), 0, st, p);
  } else {
    const int grid = grid_for(rows_tiles(p, CfgFwd4::BM, CfgFwd4::BN), num_cus);
    hipLaunchKernelGGL(grouped_rows_kernel<CfgFwd4>, dim3(grid), dim3(CfgFwd4::THREADS), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_wgrad_mx(const WgradParams& p, int num_cus, hipStream_t st) {
  using C = CfgFwd4;
  int64_t tiles = 0;
  const int64_t per = (int64_t)((p.n_rows + C::BM - 1) / C::BM) * ((p.n_cols + C::BN - 1) / C::BN);
  for (int g = 0; g < p.sp.G; ++g) tiles += (p.sp.m[g] > 0 || !p.accumulate) ? per : 0;
  if (tiles == 0) return hipSuccess;
  const int grid = grid_for(tiles, num_cus);
  hipLaunchKernelGGL(grouped_wgrad_kernel<C>, dim3(grid), dim3(C::THREADS), 0, st, p);
  return hipGetLastError();
}

}  // namespace mxgg
