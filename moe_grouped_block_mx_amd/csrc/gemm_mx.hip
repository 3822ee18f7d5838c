// Grouped block-scaled (MX) GEMMs for gfx950: forward, input gradient and
// variable-K weight gradient, one launch each.
//
// Method (pages "Triton mxfp4 (and a8w4) grouped GEMM kernel" and "Grouped
// MXFP8 GEMMs with HipKittens"): a persistent grid walks all output tiles of
// all experts; a tile index maps to its expert with an upper_bound search over
// the prefix sum of per-expert tile counts, built in LDS by every workgroup
// from the split counts passed as kernel arguments. Every output element
// belongs to exactly one tile and is stored under masks on un-wrapped indices
// (the tail-tile rule of "Add ROCm Triton blockwise FP8 grouped GEMM").
//
// All three passes are "TN" on quantized data (MX scales run along the
// contraction axis, so both operands are contraction-contiguous); only the tile
// source (which tile, which operand bases, how long the contraction) and the
// epilogue differ between them.
//
// MFMA: v_mfma_scale_f32_32x32x64_f8f6f4. Measured operand layout (32x32x64):
// lane l holds row l % 32 of its operand; for E2M1 the 16 bytes at byte offset
// 16*(l/32) of the row's 32-byte K chunk, for E4M3 the 16 bytes at 16*(l/32)
// and at 32 + 16*(l/32) of the 64-byte chunk; the op_sel-selected scale byte of
// lane l applies to row l % 32, K-block l/32; result register i of lane l is
// row 8*(i/4) + 4*(l/32) + i%4, column l % 32.
//
// Data movement: every load of the main loop is an LDS DMA
// (global_load_lds_dwordx4 for operand chunks, global_load_lds_ubyte for scale
// bytes, which land one per dword), so no VGPR is spent on staging and the
// waits are explicit: a STAGES-deep LDS ring is kept full, a stage is consumed
// after `s_waitcnt vmcnt` (counting only the DMAs issued after it) and a raw
// s_barrier (no fence: a workgroup fence would drain every DMA in flight). The
// ring runs across the tiles of a workgroup, so the next tile's first stages are
// in flight during the current tile's epilogue. Operand chunks are placed with
// an XOR swizzle of the 16-byte chunk index, chosen per lane on the global side
// (the DMA writes lane-contiguous LDS). The epilogue goes through a per-wave LDS
// scratch so global stores (and wgrad's fp32 read-modify-write) are 16-byte.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "launch.hpp"

#define MXGG_LDS __attribute__((address_space(3)))

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

// s_waitcnt encodings (gfx9): vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits
// 15:14, expcnt in 6:4, lgkmcnt in 11:8; a field at its maximum does not wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence; the compiler may not move memory
// operations across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Source of the zero chunks / zero scale bytes read past the contraction end.
static __device__ __attribute__((aligned(64))) uint32_t g_zero_page[16];

__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const void*)src, (MXGG_LDS void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const uint8_t* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const void*)src, (MXGG_LDS void*)lds, 4, 0, 0);
}

// Operand kinds: E2M1 x E2M1 and E4M3 x E2M1 with UE8M0 scales per 32 along
// the contraction (applied by the MFMA); E4M3 x E4M3 with one fp32 scale per
// 128 along the contraction ("blockwise": the MFMA runs unscaled into a
// per-128 partial that is then scaled and added, since fp32 scales are not
// powers of two in general); or blockwise E4M3 x E4M3 whose fp32 scales are
// powers of two, which the MFMA applies itself (the scale's exponent field is
// its UE8M0 code), so no partial is needed; or E4M3 x E4M3 with UE8M0 scales
// per 32 (the weight gradient of a8w4 training, whose operands are both
// activations or their gradients).
enum : int { kA4W4 = 0, kA8W4 = 1, kBlkFp8 = 2, kBlkP2 = 3, kA8A8 = 4 };

// OCC workgroups share a CU (the grid is OCC per CU): while one waits at a
// barrier or drains its epilogue, the other's MFMAs keep the SIMDs busy.
// SCHED picks the instruction order inside a stage (see compute_stage).
// BDIV: B rows sharing one scale row (128 for 128x128 weight blocks, else 1).
template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_, int KIND_, int OCC_ = 1, int SCHED_ = 0,
          int BDIV_ = 1>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_, OCC = OCC_;
  static constexpr int SCHED = SCHED_, BDIV = BDIV_;
  static constexpr bool MFB = false;  // B's MX scales in the MFMA layout (MfmaB)
  static constexpr bool KBLK_A = false, KBLK_B = false;  // A / B data in 64-byte K blocks (KBlocked)
  static constexpr bool AFP8 = KIND_ != kA4W4, BFP8 = KIND_ == kBlkFp8 || KIND_ == kBlkP2 || KIND_ == kA8A8;
  static constexpr bool BLK = KIND_ == kBlkFp8;                     // per-128 partial promotion
  // fp32 scales, one per 128 elements: A's (1x128) block-major [blocks][rows];
  // B's block-major too for 1x128 operands (BDIV 1), or one per 128x128
  // weight block ([row blocks][blocks], BDIV 128)
  static constexpr bool F32S = KIND_ == kBlkFp8 || KIND_ == kBlkP2;
  static constexpr int NW = WM * WN, THREADS = 64 * NW;
  static constexpr int RBA = AFP8 ? BK : BK / 2;  // A bytes per row per stage
  static constexpr int RBB = BFP8 ? BK : BK / 2;  // B bytes per row per stage
  static constexpr int CPA = RBA / 16, CPB = RBB / 16;
  static constexpr int KSTEPS = BK / 64;          // MFMA K steps per stage
  static constexpr int SB = F32S ? 1 : BK / 32;   // scale values per row per stage
  static constexpr int PROMO = BLK ? 128 / BK : 1;  // stages per 128-element scale block (blockwise)
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int round_up(int v, int m) { return (v + m - 1) / m * m; }
  // One ring stage: A chunks, B chunks, then the scales.
  //   MX: bytes, block-major like the global layout: A [SB][BM], then B
  //   [SB][BN]; one DMA lane moves four consecutive rows of one block, and the
  //   region is rounded up to whole DMA instructions over all waves (the extra
  //   lanes read the zero page into the padding).
  //   Blockwise: one fp32 per row (A region, then B region, each rounded up to
  //   whole instructions; the extra dwords hold repeats of the last row).
  static constexpr int A_OFF = 0, A_BYTES = BM * RBA;
  static constexpr int B_OFF = A_OFF + A_BYTES, B_BYTES = BN * RBB;
  static constexpr int MXS_BYTES = round_up((BM + BN) * SB, NW * 256);
  static constexpr int AS_OFF = B_OFF + B_BYTES, AS_BYTES = F32S ? round_up(BM * 4, NW * 256) : BM * SB;
  static constexpr int BS_OFF = AS_OFF + AS_BYTES, BS_BYTES = F32S ? round_up(BN * 4, NW * 256) : MXS_BYTES - AS_BYTES;
  static constexpr int STAGE_BYTES = BS_OFF + BS_BYTES;
  // LDS DMA instructions per wave per stage (1 KiB of chunks, or 256 bytes of
  // scales: MX, both operands' in DSA; blockwise, A's in DSA and B's in DSB)
  static constexpr int DA = A_BYTES / (NW * 1024), DB = B_BYTES / (NW * 1024);
  static constexpr int DSA = F32S ? AS_BYTES / (NW * 256) : MXS_BYTES / (NW * 256);
  static constexpr int DSB = F32S ? BS_BYTES / (NW * 256) : 0;
  static constexpr int DPS = DA + DB + DSA + DSB;
  // per-wave epilogue scratch: 16 rows of the wave's tile in fp32, padded
  // (the weight gradient stages whole rows; the rows kernels use a 16 x 32
  // corner of it)
  static constexpr int EPI_PITCH = WTN + 4;
  static constexpr int EPI_BYTES = 16 * EPI_PITCH * 4;
  // SCHED 7 and 8 keep the epilogue scratch in the ring slot of the tile's
  // last stage (free until the next tile's first DMA into it); the others
  // append it
  static constexpr bool EPI_IN_RING = SCHED == 7 || SCHED == 8;
  static constexpr int EPI_OFF = STAGES * STAGE_BYTES;
  static constexpr int SMEM_BYTES = EPI_OFF + (EPI_IN_RING ? 0 : NW * EPI_BYTES);
  static_assert(SMEM_BYTES <= 160 * 1024 - 12 * 1024, "LDS: ring, scratch and the kernels' static tables");
  static_assert(A_BYTES % (NW * 1024) == 0 && B_BYTES % (NW * 1024) == 0, "chunk DMA split");
  static_assert(KSTEPS == 1 || KSTEPS == 2, "K steps per stage");
  static_assert(!F32S || BK == 64 || BK == 128, "blockwise stages split a 128-element scale block");
  static_assert(FM >= 1 && FN >= 1 && STAGES >= 2 && STAGES <= 8, "shape");
  static_assert(DPS * (STAGES - 2) < 64, "vmcnt range");
  static_assert(F32S || (BM % 4 == 0 && BN % 4 == 0), "MX scale DMA moves four rows per lane");
  static_assert(STAGE_BYTES % 16 == 0, "stage alignment");
  static_assert(SCHED != 7 || (KSTEPS == 2 && !F32S && STAGES >= 4 && NW * EPI_BYTES <= STAGE_BYTES),
                "read-ahead schedule: two K steps per stage, MX scales, a 4+ stage ring");
  static_assert(SCHED != 8 || (KSTEPS == 1 && !BLK && STAGES >= 4 && NW * EPI_BYTES <= STAGE_BYTES),
                "stage read-ahead schedule: one K step per stage, scales applied by the MFMA, a 4+ stage ring");
};

// A configuration whose B operand (the weights) carries its MX scales in the
// MFMA layout: 128-byte units of 32 rows x 4 blocks in which lane L of a
// fragment finds its two K steps' scale bytes at 2L and 2L+1. A stage's B
// scales are then (BN/32) whole units, contiguous in memory and copied as one
// run (the block-major layout needs four runs of BN bytes), and a lane reads
// both K steps' bytes with one 2-byte LDS read.
template <class C>
struct MfmaB : C {
  static constexpr bool MFB = true;
  static_assert(!C::F32S && C::BK == 128 && C::BN % 32 == 0, "MFMA-layout scales: 128-deep MX stages");
};

// A configuration whose A and B data are stored in 64-byte blocks along the
// contraction, u8 [L/64, rows, 64] for rows of L bytes (the blockwise E4M3
// operands, and MX operands with the K-block code layout; contractions and
// segments are then multiples of 128 elements): byte
// j of row r sits at (j/64)*ld + r*64 + j%64 with ld = rows*64, so the 64
// bytes a stage needs from each of a tile's rows form one contiguous run per
// 64-byte block (one 1 KiB run per DMA instruction instead of 16 row pieces).
template <class C>
struct KBlocked : C {
  static constexpr bool KBLK_A = true, KBLK_B = true;
  static_assert(C::RBA % 64 == 0 && C::RBB % 64 == 0, "stages of whole 64-byte K blocks");
};

// Byte offset of data byte j (along the contraction) of row r: row-major
// rows of ld bytes, or 64-byte K blocks of ld bytes each (KBLK_A / KBLK_B
// for operand A / B).
template <class C, bool ON_B>
__host__ __device__ constexpr int64_t data_off(int64_t r, int64_t j, int64_t ld) {
  constexpr bool kb = ON_B ? C::KBLK_B : C::KBLK_A;
  return kb ? (j / 64) * ld + r * 64 + j % 64 : r * ld + j;
}

// The segment owning item t of a non-decreasing prefix offs[0..n] (offs[0] =
// 0), from a cursor: a workgroup visits its tiles in increasing order (or,
// reversed, in decreasing order; the issuing side and the computing side
// each with its own cursor), so the cursor's segment usually still owns t and
// one LDS read confirms it; else a binary search over the segments after it
// (before it, walking backwards).
__device__ __forceinline__ int seek_segment(const int32_t* offs, int n, int t, int& cursor) {
  int j = cursor;
  if (j >= 0 && t < offs[j]) {
    j = upper_bound_i32(offs, j + 1, t) - 1;  // a workgroup walking its tiles backwards
  } else if (j < 0 || offs[j + 1] <= t) {
    const int lo = j < 0 ? 0 : j + 1;
    j = lo + upper_bound_i32(offs + lo, n - lo, t) - 1;
  }
  cursor = j;
  return j;
}

// Operand bases and extents of one tile.
struct TileOps {
  const uint8_t* a;   // first row of the A tile (row stride lda)
  const uint8_t* as;  // its scales: MX, block-major (block stride ldas, row
                      // stride 1; the tile's first row a multiple of 4);
                      // blockwise 1x128, block-major fp32 (block stride ldas)
  const uint8_t* b;
  const uint8_t* bs;
  int mrows, nrows;   // valid rows of A and B (>= 1)
  int srows_a, srows_b;  // MX: scale rows readable from as / bs in every
                         // block (a multiple of 4, >= 4); MFMA-layout B:
                         // bytes readable in every 128-element group (a
                         // multiple of 128)
  int kc;             // contraction length (elements), multiple of 32
};

// Per-thread DMA offsets of the issuing tile (32-bit: a tile's rows span less
// than 4 GiB, which the ABI's shape limits guarantee).
template <class C>
struct DmaPlan {
  uint32_t offA[C::DA], offB[C::DB], offAS[C::DSA], offBS[C::DSB];
  int kA[C::DA], kB[C::DB];       // byte offset of the chunk inside a stage row
  // MX scales: per lane, the row offset of its four rows and its block inside
  // a stage (kNoBlock: padding); the operand of an instruction is
  // wave-uniform (A's and B's regions are whole instructions)
  uint32_t sOff[C::F32S ? 1 : C::DSA];
  int sBlk[C::F32S ? 1 : C::DSA];
  int64_t astep, bstep;  // data bytes from one stage to the next (K blocks: whole blocks)
};
constexpr int kNoBlock = 1 << 24;

// Blockwise fp32 scales: byte offset of 128-element block `blk` inside a
// tile's scale run. Block-major operands (A, and B with BDIV 1) step a whole
// block row of ld bytes; 128x128 weight scales are row-major over blocks.
template <class C, bool ON_B>
__device__ __forceinline__ int64_t blk_off(int blk, int64_t ld) {
  if constexpr (ON_B && C::BDIV != 1) return (int64_t)blk * 4;
  return (int64_t)blk * ld;
}

template <class C>
__device__ __forceinline__ void plan_dma(DmaPlan<C>& pl, const TileOps& t, int64_t lda, int64_t ldas, int64_t ldb,
                                         int64_t ldbs, int w, int lane) {
  unroll<C::DA>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int o = (i * C::NW + w) * 1024 + lane * 16;
    const int r = o / C::RBA;
    const int c = swz<C::CPA>(r, (o % C::RBA) / 16);
    const int rr = r < t.mrows ? r : t.mrows - 1;
    pl.offA[i] = (uint32_t)data_off<C, false>(rr, c * 16, lda);
    pl.kA[i] = c * 16;
  });
  unroll<C::DB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int o = (i * C::NW + w) * 1024 + lane * 16;
    const int r = o / C::RBB;
    const int c = swz<C::CPB>(r, (o % C::RBB) / 16);
    const int rr = r < t.nrows ? r : t.nrows - 1;
    pl.offB[i] = (uint32_t)data_off<C, true>(rr, c * 16, ldb);
    pl.kB[i] = c * 16;
  });
  pl.astep = data_off<C, false>(0, C::RBA, lda);
  pl.bstep = data_off<C, true>(0, C::RBB, ldb);
  // Scales. MX: lane word d of the stage's scale region holds four rows of
  // one block: A's [SB][BM] bytes, then B's [SB][BN], then padding. Rows past
  // the readable scale rows (which only invalid tile rows reach) read the last
  // readable group of four, so every read stays inside the buffer.
  // Blockwise: one fp32 per row of the stage's 128-element block (per-lane
  // row offsets here; the stage adds its block's offset, blk_off).
  if constexpr (C::F32S) {
    unroll<C::DSA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int d = (i * C::NW + w) * 64 + lane;
      const int rr = d < t.mrows ? d : t.mrows - 1;
      pl.offAS[i] = (uint32_t)(rr * 4);
    });
    unroll<C::DSB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int d = (i * C::NW + w) * 64 + lane;
      const int rr = d < t.nrows ? d : t.nrows - 1;
      pl.offBS[i] = C::BDIV == 1 ? (uint32_t)(rr * 4) : (uint32_t)((rr / C::BDIV) * ldbs);
    });
  } else {
    unroll<C::DSA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int byte = ((i * C::NW + w) * 64 + lane) * 4;
      if (byte < C::BM * C::SB) {
        const int r = byte % C::BM;
        pl.sOff[i] = (uint32_t)(r < t.srows_a - 4 ? r : t.srows_a - 4);
        pl.sBlk[i] = byte / C::BM;
      } else if (byte < (C::BM + C::BN) * C::SB) {
        const int bb = byte - C::BM * C::SB;
        if constexpr (C::MFB) {
          // byte bb of the tile's contiguous run in the stage's group (the
          // stage's first block, sBlk 0, addresses the group: ldbs is a
          // block's share of the group stride)
          pl.sOff[i] = (uint32_t)(bb < t.srows_b - 4 ? bb : t.srows_b - 4);
          pl.sBlk[i] = 0;
        } else {
          const int r = bb % C::BN;
          pl.sOff[i] = (uint32_t)(r < t.srows_b - 4 ? r : t.srows_b - 4);
          pl.sBlk[i] = bb / C::BN;
        }
      } else {
        pl.sOff[i] = 0;
        pl.sBlk[i] = kNoBlock;
      }
    });
  }
}

// Issue the DMAs of stage s of tile t into ring slot `st` (every wave issues
// exactly DPS instructions, the count the waits rely on).
// Pointer select without a branch (the scale-block conditions are uniform,
// and a uniform branch would split the stage's instruction block).
__device__ __forceinline__ const uint8_t* select_ptr(bool c, const uint8_t* a, const uint8_t* b) {
  const uint64_t m = 0 - (uint64_t)c;
  return reinterpret_cast<const uint8_t*>((reinterpret_cast<uint64_t>(a) & m) | (reinterpret_cast<uint64_t>(b) & ~m));
}

// A dummy stage (no work left) issues the same instructions from the zero
// page, so that every step issues exactly DPS DMAs.
// PART: -1 every DMA of the stage; 0 the A chunks and the scales; 1 the B chunks.
// `zero`: the zero page's address (g_zero_page), which a caller may hold in
// registers across its loop.
template <class C, int PART = -1>
__device__ __forceinline__ void issue_stage(const DmaPlan<C>& pl, const TileOps& t, int s, uint8_t* st, int w,
                                            int64_t ldas, int64_t ldbs, bool dummy = false,
                                            const uint8_t* zero = reinterpret_cast<const uint8_t*>(g_zero_page)) {
  constexpr bool DO_A = PART != 1, DO_B = PART != 0;
  const int kca = dummy ? 0 : (C::AFP8 ? t.kc : t.kc / 2);
  const int kcb = dummy ? 0 : (C::BFP8 ? t.kc : t.kc / 2);
  const int ka0 = s * C::RBA, kb0 = s * C::RBB;
  // scales of this stage: MX, blocks s*SB .. s*SB+SB-1 (blocks past the
  // contraction and padding lanes read zeros); blockwise, the fp32 of
  // 128-block s*BK/128
  const int nblk = dummy ? 0 : (C::F32S ? t.kc / 128 : t.kc / 32);
  const int bidx0 = C::F32S ? s * C::BK / 128 : s * C::SB;
  if constexpr (DO_A) {
    unroll<C::DA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint8_t* src = select_ptr(ka0 + pl.kA[i] < kca, t.a + s * pl.astep + pl.offA[i], zero);
      dma16(src, st + C::A_OFF + (i * C::NW + w) * 1024);
    });
  }
  if constexpr (DO_B) {
    unroll<C::DB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint8_t* src = select_ptr(kb0 + pl.kB[i] < kcb, t.b + s * pl.bstep + pl.offB[i], zero);
      dma16(src, st + C::B_OFF + (i * C::NW + w) * 1024);
    });
  }
  if constexpr (!DO_A) {
  } else if constexpr (C::F32S) {
    unroll<C::DSA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma4(select_ptr(bidx0 < nblk, t.as + blk_off<C, false>(bidx0, ldas) + pl.offAS[i], zero),
           st + C::AS_OFF + (i * C::NW + w) * 256);
    });
    unroll<C::DSB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma4(select_ptr(bidx0 < nblk, t.bs + blk_off<C, true>(bidx0, ldbs) + pl.offBS[i], zero),
           st + C::BS_OFF + (i * C::NW + w) * 256);
    });
  } else {
    static_assert((C::BM * C::SB) % 256 == 0 && (C::BN * C::SB) % 256 == 0, "operand regions: whole instructions");
    unroll<C::DSA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const bool on_b = (i * C::NW + w) * 256 >= C::BM * C::SB;  // wave-uniform
      const uint8_t* base = on_b ? t.bs : t.as;
      const int64_t ld = on_b ? ldbs : ldas;
      const int b = bidx0 + pl.sBlk[i];
      dma4(select_ptr(b < nblk, base + (int64_t)b * ld + pl.sOff[i], zero), st + C::AS_OFF + (i * C::NW + w) * 256);
    });
  }
}

// Sources of the B chunk DMAs of stage s (zero page past the contraction or
// for a dummy stage), and their issue into ring slot st.
template <class C>
__device__ __forceinline__ void stage_b_srcs(const DmaPlan<C>& pl, const TileOps& t, int s, bool dummy,
                                             const uint8_t* zero, const uint8_t* (&src)[C::DB]) {
  const int kcb = dummy ? 0 : (C::BFP8 ? t.kc : t.kc / 2);
  const int kb0 = s * C::RBB;
  unroll<C::DB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    src[i] = select_ptr(kb0 + pl.kB[i] < kcb, t.b + s * pl.bstep + pl.offB[i], zero);
  });
}
template <class C>
__device__ __forceinline__ void issue_b_srcs(const uint8_t* const (&src)[C::DB], uint8_t* st, int w) {
  unroll<C::DB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    dma16(src[i], st + C::B_OFF + (i * C::NW + w) * 1024);
  });
}

// ---------------------------------------------------------------------------
// DMA issue when every stage of a launch is full (the contraction a multiple
// of BK, so no stage needs zero-page chunks): an address is a wave-uniform
// base, advanced per stage with scalar adds, plus a per-lane 32-bit offset
// fixed for the tile, so a DMA costs no vector ALU work. The general path
// selects the zero page per lane and per stage with 64-bit vector address
// arithmetic; measured with per-wave cycle counters at the fc1 shapes, that
// work made the stage half issuing the A and scale DMAs take twice as long
// as the other half (which issues the same number of MFMAs).
// ---------------------------------------------------------------------------
template <class C>
struct FastPlan {
  // per lane: chunk offsets; scale offsets (MX: DSA words of either operand;
  // fp32 row scales: DSA of A's rows, then DSB of B's)
  uint32_t vA[C::DA], vB[C::DB], vS[C::DSA], vSB[C::DSB > 0 ? C::DSB : 1];
  // wave-uniform: the tile's operand bases; per scale DMA instruction, the
  // scale operand it reads and that operand's bytes per stage
  const uint8_t *a, *b, *s[C::DSA], *sb;
  int64_t sstep[C::DSA], sbstep;
  int64_t astep, bstep;  // data bytes per stage (as in DmaPlan)
};

// A wave-uniform pointer moved to scalar registers (the tile bases are
// uniform but computed through LDS reads; without this the compiler keeps
// them in vector registers and moves them back for every DMA).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// The offsets of plan_dma without the per-stage parts: chunks at row*ld +
// swizzled chunk; scale words at block*ld + first row (padding lanes: 0,
// which reads a valid word of the same operand into LDS padding). The
// caller guarantees (SB-1)*ld + rows < 2^32 for both scale operands.
template <class C>
__device__ __forceinline__ void plan_fast(FastPlan<C>& fp, const DmaPlan<C>& pl, const TileOps& t, int64_t ldas,
                                          int64_t ldbs, int w) {
  w = __builtin_amdgcn_readfirstlane(w);
  unroll<C::DA>([&](auto ic) { fp.vA[decltype(ic)::value] = pl.offA[decltype(ic)::value]; });
  unroll<C::DB>([&](auto ic) { fp.vB[decltype(ic)::value] = pl.offB[decltype(ic)::value]; });
  fp.a = uniform_ptr(t.a);
  fp.b = uniform_ptr(t.b);
  fp.astep = pl.astep;
  fp.bstep = pl.bstep;
  if constexpr (C::F32S) {
    // one fp32 per row and 128-element block: row offsets; the stage adds its
    // block's offset (sstep / sbstep bytes per block)
    unroll<C::DSA>([&](auto ic) {
      fp.vS[decltype(ic)::value] = pl.offAS[decltype(ic)::value];
      fp.s[decltype(ic)::value] = uniform_ptr(t.as);
      fp.sstep[decltype(ic)::value] = blk_off<C, false>(1, ldas);
    });
    unroll<C::DSB>([&](auto ic) { fp.vSB[decltype(ic)::value] = pl.offBS[decltype(ic)::value]; });
    fp.sb = uniform_ptr(t.bs);
    fp.sbstep = blk_off<C, true>(1, ldbs);
    return;
  }
  unroll<C::DSA>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const bool on_b = (i * C::NW + w) * 256 >= C::BM * C::SB;  // wave-uniform
    const int64_t ld = on_b ? ldbs : ldas;
    fp.vS[i] = pl.sBlk[i] < kNoBlock ? (uint32_t)pl.sBlk[i] * (uint32_t)ld + pl.sOff[i] : 0u;
    fp.s[i] = uniform_ptr(on_b ? t.bs : t.as);
    fp.sstep[i] = (int64_t)__builtin_amdgcn_readfirstlane((int)(C::SB * ld));
  });
}

// The same issue with no per-lane state kept across the loop: every stage
// recomputes the lane offsets from the lane index and the tile's uniform
// extents (a few vector ALU operations per DMA, beside 16 MFMAs of 64
// cycles), for the stage read-ahead loop, whose accumulators and operand
// sets leave no registers for ten offsets (fp32 row scales only).
template <class C>
struct LeanPlan {
  const uint8_t *a, *b, *as, *bs;  // the tile's bases (wave-uniform)
  int mlast, nlast;                // last valid row of the A / B tile
};

template <class C>
__device__ __forceinline__ void plan_lean(LeanPlan<C>& lp, const TileOps& t) {
  static_assert(C::F32S, "lean issue: fp32 row scales");
  lp.a = uniform_ptr(t.a);
  lp.b = uniform_ptr(t.b);
  lp.as = uniform_ptr(t.as);
  lp.bs = uniform_ptr(t.bs);
  lp.mlast = __builtin_amdgcn_readfirstlane(t.mrows - 1);
  lp.nlast = __builtin_amdgcn_readfirstlane(t.nrows - 1);
}

// DMAs [Q0, Q1) of stage s in the order: A chunks, A scales, B scales, B
// chunks (all of them for Q0 = 0, Q1 = DPS).
template <class C, int Q0 = 0, int Q1 = C::DPS>
__device__ __forceinline__ void issue_stage_lean(const LeanPlan<C>& lp, int s, uint8_t* st, int w, int lane, int lda,
                                                 int ldb, int ldas, int ldbs) {
  // rows per chunk DMA instruction over all waves: the swizzle of a lane's
  // chunk is the same in every instruction
  static_assert((C::NW * 1024 / C::RBA) % 16 == 0 && (C::NW * 1024 / C::RBB) % 16 == 0, "uniform swizzle");
  constexpr int QSA = C::DA, QSB = QSA + C::DSA, QB = QSB + C::DSB;
  uint32_t ln = (uint32_t)lane;
  asm volatile("" : "+v"(ln));  // recomputed here, not hoisted out of the loop
  const uint32_t wu = (uint32_t)w;
  const uint8_t* abase = lp.a + s * data_off<C, false>(0, C::RBA, lda);
  unroll<C::DA>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i >= Q0 && i < Q1) {
      const uint32_t o = (i * C::NW + wu) * 1024 + ln * 16;
      const int r = (int)(o / C::RBA);
      const int c = swz<C::CPA>(r, (int)(o % C::RBA) / 16);
      const int rr = r < lp.mlast ? r : lp.mlast;
      dma16(abase + (uint32_t)data_off<C, false>(rr, c * 16, lda), st + C::A_OFF + (i * C::NW + w) * 1024);
    }
  });
  const int blk = s * C::BK / 128;  // the stage's 128-element block
  const uint8_t* asb = lp.as + blk_off<C, false>(blk, ldas);
  const uint8_t* bsb = lp.bs + blk_off<C, true>(blk, ldbs);
  unroll<C::DSA>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (QSA + i >= Q0 && QSA + i < Q1) {
      const int d = (int)((i * C::NW + wu) * 64 + ln);
      const int rr = d < lp.mlast ? d : lp.mlast;
      dma4(asb + (uint32_t)(rr * 4), st + C::AS_OFF + (i * C::NW + w) * 256);
    }
  });
  unroll<C::DSB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (QSB + i >= Q0 && QSB + i < Q1) {
      const int d = (int)((i * C::NW + wu) * 64 + ln);
      const int rr = d < lp.nlast ? d : lp.nlast;
      const uint32_t ro = C::BDIV == 1 ? (uint32_t)(rr * 4) : (uint32_t)((rr / C::BDIV) * ldbs);
      dma4(bsb + ro, st + C::BS_OFF + (i * C::NW + w) * 256);
    }
  });
  const uint8_t* bbase = lp.b + s * data_off<C, true>(0, C::RBB, ldb);
  unroll<C::DB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (QB + i >= Q0 && QB + i < Q1) {
      const uint32_t o = (i * C::NW + wu) * 1024 + ln * 16;
      const int r = (int)(o / C::RBB);
      const int c = swz<C::CPB>(r, (int)(o % C::RBB) / 16);
      const int rr = r < lp.nlast ? r : lp.nlast;
      dma16(bbase + (uint32_t)data_off<C, true>(rr, c * 16, ldb), st + C::B_OFF + (i * C::NW + w) * 1024);
    }
  });
}

// Stage s of tile t into ring slot st (PART as for issue_stage). A dummy
// stage re-reads stage 0 of the last planned tile (or the zero page before
// any): its data is never consumed, the DMAs only keep the counts constant.
template <class C, int PART = -1>
__device__ __forceinline__ void issue_stage_fast(const FastPlan<C>& fp, int s, uint8_t* st, int w) {
  constexpr bool DO_A = PART != 1, DO_B = PART != 0;
  if constexpr (DO_A) {
    const uint8_t* base = fp.a + s * fp.astep;
    unroll<C::DA>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma16(base + fp.vA[i], st + C::A_OFF + (i * C::NW + w) * 1024);
    });
    if constexpr (C::F32S) {
      const int blk = s * C::BK / 128;  // the stage's 128-element block
      unroll<C::DSA>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        dma4(fp.s[i] + blk * fp.sstep[i] + fp.vS[i], st + C::AS_OFF + (i * C::NW + w) * 256);
      });
      unroll<C::DSB>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        dma4(fp.sb + blk * fp.sbstep + fp.vSB[i], st + C::BS_OFF + (i * C::NW + w) * 256);
      });
    } else {
      unroll<C::DSA>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        dma4(fp.s[i] + s * fp.sstep[i] + fp.vS[i], st + C::AS_OFF + (i * C::NW + w) * 256);
      });
    }
  }
  if constexpr (DO_B) {
    const uint8_t* base = fp.b + s * fp.bstep;
    unroll<C::DB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma16(base + fp.vB[i], st + C::B_OFF + (i * C::NW + w) * 1024);
    });
  }
}

// B fragments of K step KK (E2M1: 16 bytes per lane; E4M3: 2 x 16 bytes).
template <class C, int KK>
__device__ __forceinline__ void load_b_frags(const uint8_t* st, v8i (&bf)[C::FN], int wn, int h, int l32) {
  unroll<C::FN>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int r = wn * C::WTN + j * 32 + l32;
    const uint8_t* row = st + C::B_OFF + r * C::RBB;
    if constexpr (C::BFP8) {
      const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPB>(r, 4 * KK + h) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(row + swz<C::CPB>(r, 4 * KK + 2 + h) * 16);
      bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPB>(r, 2 * KK + h) * 16);
      bf[j] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
  });
}

// Blockwise FP8 stage: unscaled E4M3 x E4M3 MFMAs (scale bytes 127 = 2^0)
// into the partial P of the current 128-element block (FIRST: the block's
// first stage, P starts from zero); on its last stage (LAST) the partial is
// scaled by the rows' A scale and the columns' B scale (fp32, from the stage's
// scale region) and added to acc. Register r of a fragment holds row
// 8*(r/4) + 4*(lane/32) + r%4, column lane%32, so a lane's 16 row scales of a
// fragment are four runs of four consecutive dwords.
template <class C, bool FIRST, bool LAST>
__device__ __forceinline__ void compute_stage_blk(const uint8_t* st, v16f (&acc)[C::FM][C::FN],
                                                  v16f (&P)[C::FM][C::FN], int wm, int wn, int h, int l32) {
  constexpr int kUnit = 0x7F7F7F7F;
  unroll<C::KSTEPS>([&](auto kc_) {
    constexpr int kk = decltype(kc_)::value;
    v8i af[C::FM], bf[C::FN];
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int r = wm * C::WTM + i * 32 + l32;
      const uint8_t* row = st + C::A_OFF + r * C::RBA;
      const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 4 * kk + h) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 4 * kk + 2 + h) * 16);
      af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    });
    load_b_frags<C, kk>(st, bf, wn, h, l32);
    unroll<C::FM>([&](auto ic) {
      unroll<C::FN>([&](auto jc) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        const v16f c_in = (FIRST && kk == 0) ? v16f{} : P[i][j];
        P[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], c_in, 0, 0, 0, kUnit, 0, kUnit);
      });
    });
  });
  if constexpr (LAST) {
    const float* as = reinterpret_cast<const float*>(st + C::AS_OFF);
    const float* bs = reinterpret_cast<const float*>(st + C::BS_OFF);
    float sbv[C::FN];
    unroll<C::FN>([&](auto jc) { sbv[decltype(jc)::value] = bs[wn * C::WTN + decltype(jc)::value * 32 + l32]; });
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      v4f sa4[4];
      unroll<4>([&](auto qc) {
        sa4[decltype(qc)::value] =
            *reinterpret_cast<const v4f*>(as + wm * C::WTM + i * 32 + 8 * decltype(qc)::value + 4 * h);
      });
      unroll<C::FN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        unroll<16>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          acc[i][j][r] += P[i][j][r] * (sa4[r / 4][r % 4] * sbv[j]);
        });
      });
    });
  }
}

// MFMAs of one ring stage for this wave's fragments. `issue` issues the DMAs
// of a later stage; with SCHED 5 they are spread over the last K step's MFMAs.
struct NoIssue {
  __device__ __forceinline__ void operator()() const {}
};
template <class C, class Issue = NoIssue>
__device__ __forceinline__ void compute_stage(const uint8_t* st, v16f (&acc)[C::FM][C::FN], int wm, int wn, int h,
                                              int l32, Issue&& issue = Issue{}) {
  uint32_t sa[C::FM], sb[C::FN];
  if constexpr (C::F32S) {
    // power-of-two fp32 scales, one per row for the whole stage: the
    // exponent field is the UE8M0 code, the same for every K step
    constexpr uint32_t REP = C::KSTEPS == 2 ? 0x0101u : 0x01u;
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int r = wm * C::WTM + i * 32 + l32;
      sa[i] = ((reinterpret_cast<const uint32_t*>(st + C::AS_OFF)[r] >> 23) & 0xffu) * REP;
    });
    unroll<C::FN>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int r = wn * C::WTN + j * 32 + l32;
      sb[j] = ((reinterpret_cast<const uint32_t*>(st + C::BS_OFF)[r] >> 23) & 0xffu) * REP;
    });
  } else {
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int r = wm * C::WTM + i * 32 + l32;
      // lane half h takes block h of K step 0 (op_sel 0) and block 2+h of K step 1 (op_sel 1)
      const uint8_t* p = st + C::AS_OFF + h * C::BM + r;
      if constexpr (C::KSTEPS == 2) sa[i] = p[0] | ((uint32_t)p[2 * C::BM] << 8);
      else sa[i] = p[0];
    });
    unroll<C::FN>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (C::MFB) {
        sb[j] = *reinterpret_cast<const uint16_t*>(st + C::BS_OFF + (wn * C::FN + j) * 128 + (l32 + 32 * h) * 2);
      } else {
        const int r = wn * C::WTN + j * 32 + l32;
        const uint8_t* p = st + C::BS_OFF + h * C::BN + r;
        if constexpr (C::KSTEPS == 2) sb[j] = p[0] | ((uint32_t)p[2 * C::BN] << 8);
        else sb[j] = p[0];
      }
    });
  }
  unroll<C::KSTEPS>([&](auto kc_) {
    constexpr int kk = decltype(kc_)::value;
    v8i af[C::FM], bf[C::FN];
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int r = wm * C::WTM + i * 32 + l32;
      const uint8_t* row = st + C::A_OFF + r * C::RBA;
      if constexpr (C::AFP8) {
        const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 4 * kk + h) * 16);
        const v4i hi = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 4 * kk + 2 + h) * 16);
        af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 2 * kk + h) * 16);
        af[i] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      }
    });
    load_b_frags<C, kk>(st, bf, wn, h, l32);
    unroll<C::FM>([&](auto ic) {
      unroll<C::FN>([&](auto jc) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], C::AFP8 ? 0 : 4,
                                                                    C::BFP8 ? 0 : 4, kk, (int)sa[i], kk,
                                                                    (int)sb[j]);
      });
    });
  });
  // after every LDS read of the stage in program order: the DMAs write LDS
  // (another slot, which the compiler cannot prove), so reads may not pass them
  issue();
  // Instruction order of the stage (one basic block):
  //   0: the compiler's choice
  //   1: every LDS read first, then every MFMA
  //   2: the compiler's MFMA/LDS interleaving strategy 0
  //   3: reads of K step 0, then K step 0's MFMAs each followed by one read of
  //      K step 1, then the rest
  //   5: as 3, and the last K step's MFMAs each followed by one of the DMAs
  //      issued for a later stage (the address unit drains them while the
  //      MFMAs run instead of stalling the wave right after the barrier)
  constexpr int NR0 = C::FM * (C::AFP8 ? 2 : 1) + C::FN * (C::BFP8 ? 2 : 1);  // fragment reads per K step
  constexpr int NSR = (C::FM + C::FN) * C::KSTEPS;                                // scale reads per stage
  if constexpr (C::SCHED == 1) {
    __builtin_amdgcn_sched_group_barrier(0x100, 64, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 64, 0);
  } else if constexpr (C::SCHED == 2) {
    __builtin_amdgcn_iglp_opt(0);
  } else if constexpr (C::SCHED == 3) {
    __builtin_amdgcn_sched_group_barrier(0x100, NR0 + NSR, 0);
    unroll<NR0>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    });
    __builtin_amdgcn_sched_group_barrier(0x008, 64, 0);
  } else if constexpr (C::SCHED == 5) {
    constexpr int NMF = C::FM * C::FN;  // MFMAs per K step
    __builtin_amdgcn_sched_group_barrier(0x100, NR0 + NSR, 0);
    if constexpr (C::KSTEPS == 2) {
      unroll<NMF>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
    }
    constexpr int PER = (C::DPS + NMF - 1) / NMF;  // DMAs after each MFMA of the last K step
    unroll<NMF>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x060, PER, 0);
    });
    __builtin_amdgcn_sched_group_barrier(0x068, 64, 0);
  }
}


// ---------------------------------------------------------------------------
// SCHED 7 (read-ahead): a stage's two K steps are split by the workgroup
// barrier. Before it, the wave runs the MFMAs of K step 0 (operands read
// during the previous stage) and reads the operands of K step 1; after it,
// the MFMAs of K step 1 run while the wave reads the next stage's K step 0
// operands and issues the DMAs of a later stage. No LDS read sits between the
// barrier and the first MFMA after it. The barrier before K step 1 of stage s
// admits the reads of stage s+1 (its DMAs have landed) and the DMAs into the
// slot of stage s-1 (every wave's reads of it were consumed by MFMAs issued
// before the barrier). Each K step's operands (fragments and scale bytes) are
// written in one half and read in the other, so no register is copied.
// ---------------------------------------------------------------------------
template <class C>
struct KOps {
  v8i a[C::FM], b[C::FN];
  uint32_t sa[C::FM], sb[C::FN];  // scale byte in bits 0..7 (op_sel 0)
};

// lane half h takes block h of K step 0 and block 2+h of K step 1
template <class C, int KK>
__device__ __forceinline__ void read_kops(const uint8_t* st, KOps<C>& f, int wm, int wn, int h, int l32) {
  unroll<C::FM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int r = wm * C::WTM + i * 32 + l32;
    const uint8_t* row = st + C::A_OFF + r * C::RBA;
    if constexpr (C::AFP8) {
      const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 4 * KK + h) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 4 * KK + 2 + h) * 16);
      f.a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r, 2 * KK + h) * 16);
      f.a[i] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
    if constexpr (C::F32S)  // power-of-two fp32 row scale: its exponent field is the UE8M0 code
      f.sa[i] = (reinterpret_cast<const uint32_t*>(st + C::AS_OFF)[r] >> 23) & 0xffu;
    else
      f.sa[i] = st[C::AS_OFF + (2 * KK + h) * C::BM + r];
  });
  load_b_frags<C, KK>(st, f.b, wn, h, l32);
  unroll<C::FN>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (C::F32S)
      f.sb[j] = (reinterpret_cast<const uint32_t*>(st + C::BS_OFF)[wn * C::WTN + j * 32 + l32] >> 23) & 0xffu;
    else if constexpr (C::MFB)
      f.sb[j] = st[C::BS_OFF + (wn * C::FN + j) * 128 + (l32 + 32 * h) * 2 + KK];
    else
      f.sb[j] = st[C::BS_OFF + (2 * KK + h) * C::BN + wn * C::WTN + j * 32 + l32];
  });
}

template <class C>
__device__ __forceinline__ void mfma_kops(const KOps<C>& f, v16f (&acc)[C::FM][C::FN]) {
  unroll<C::FM>([&](auto ic) {
    unroll<C::FN>([&](auto jc) {
      constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], C::AFP8 ? 0 : 4,
                                                                  C::BFP8 ? 0 : 4, 0, (int)f.sa[i], 0,
                                                                  (int)f.sb[j]);
    });
  });
}

// One half: the MFMAs of `use`, each followed by a share of the reads into
// `fill` (from stage slot st) and of the DMAs issued by `issue`.
template <class C, int KK, int SYNC, int ND, class Issue>
__device__ __forceinline__ void ra_half(const uint8_t* st, const KOps<C>& use, KOps<C>& fill,
                                        v16f (&acc)[C::FM][C::FN], int wm, int wn, int h, int l32, Issue&& issue) {
  read_kops<C, KK>(st, fill, wm, wn, h, l32);
  mfma_kops<C>(use, acc);
  issue();
  constexpr int NMF = C::FM * C::FN;
  constexpr int NR = C::FM * (C::AFP8 ? 2 : 1) + C::FN * (C::BFP8 ? 2 : 1) + C::FM + C::FN;
  constexpr int PER = (NR + NMF - 1) / NMF;
  // ND DMAs spread evenly: one after MFMA m when (m+1)*ND/NMF steps up
  unroll<NMF>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);
    __builtin_amdgcn_sched_group_barrier(0x100, PER, SYNC);
    constexpr int nd = (m + 1) * ND / NMF - m * ND / NMF;
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x060, nd, SYNC);
  });
}

// ---------------------------------------------------------------------------
// SCHED 8 (stage read-ahead, one K step per stage): the operands of the next
// stage are read while the current stage's MFMAs run. The B fragments come in
// two sets (current, next); the A fragments of a row are replaced by the next
// stage's as soon as that row's MFMAs have issued, so one set suffices. The
// B scale bytes are packed in one register (byte j for column fragment j,
// picked by the MFMA's op_sel).
// ---------------------------------------------------------------------------
template <class C>
struct ROps {
  v8i a[C::FM];
  uint32_t sa[C::FM];
  v8i b[2][C::FN];
  uint32_t sb[2];
};

// Fragment rows 32 apart share their swizzle (it depends on row bits below
// 5), so every fragment's address is the first fragment's plus a constant:
// one lane offset serves them all (through the read's offset field).
template <class C>
__device__ __forceinline__ void read_a_frag(const uint8_t* st, int i, v8i& a, uint32_t& sa, int wm, int h,
                                            int l32) {
  const int r0 = wm * C::WTM + l32, r = r0 + i * 32;
  const uint8_t* row = st + C::A_OFF + r0 * C::RBA + i * 32 * C::RBA;
  if constexpr (C::AFP8) {
    const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r0, h) * 16);
    const v4i hi = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r0, 2 + h) * 16);
    a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPA>(r0, h) * 16);
    a = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
  }
  if constexpr (C::F32S)  // power-of-two fp32 row scale: its exponent field is the UE8M0 code
    sa = (reinterpret_cast<const uint32_t*>(st + C::AS_OFF)[r] >> 23) & 0xffu;
  else
    sa = st[C::AS_OFF + h * C::BM + r];
}

// B fragments [J0, J1) of a stage; with SCALES, every column fragment's scale
// byte packed into sb
template <class C, int J0, int J1, bool SCALES>
__device__ __forceinline__ void read_b_part(const uint8_t* st, v8i (&b)[C::FN], uint32_t& sb, int wn, int h, int l32) {
  unroll<C::FN>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j >= J0 && j < J1) {
      const int r0 = wn * C::WTN + l32;
      const uint8_t* row = st + C::B_OFF + r0 * C::RBB + j * 32 * C::RBB;
      if constexpr (C::BFP8) {
        const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPB>(r0, h) * 16);
        const v4i hi = *reinterpret_cast<const v4i*>(row + swz<C::CPB>(r0, 2 + h) * 16);
        b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const v4i lo = *reinterpret_cast<const v4i*>(row + swz<C::CPB>(r0, h) * 16);
        b[j] = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      }
    }
  });
  if constexpr (SCALES) {
    uint32_t packed = 0;
    unroll<C::FN>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int r = wn * C::WTN + j * 32 + l32;
      uint32_t byte;
      if constexpr (C::F32S) byte = (reinterpret_cast<const uint32_t*>(st + C::BS_OFF)[r] >> 23) & 0xffu;
      else byte = st[C::BS_OFF + h * C::BN + r];
      packed |= byte << (8 * j);
    });
    sb = packed;
  }
}

// One step: the MFMAs of the current stage (B set P), row by row. Each row's
// segment carries a share of the next stage's B reads and of the DMAs
// (issue_part<Q0, Q1>: DMAs [Q0, Q1) of the stage) and ends with the next
// stage's A fragment of that row, read into the registers the row's MFMAs
// have just consumed (the fences keep those reads behind the MFMAs, so one A
// set suffices).
template <class C, int P, class IssuePart>
__device__ __forceinline__ void ra_step(const uint8_t* nxt, ROps<C>& f, v16f (&acc)[C::FM][C::FN], int wm, int wn,
                                        int h, int l32, IssuePart&& issue_part) {
  static_assert(C::FN <= 4 && C::FM >= 2, "B scale bytes packed in one register; B reads over two rows");
  constexpr int Q = 1 - P;
  unroll<C::FM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    // the next stage's B fragments over the first two rows, their scales with the second half
    if constexpr (i == 0) read_b_part<C, 0, C::FN / 2, false>(nxt, f.b[Q], f.sb[Q], wn, h, l32);
    if constexpr (i == 1) read_b_part<C, C::FN / 2, C::FN, true>(nxt, f.b[Q], f.sb[Q], wn, h, l32);
    unroll<C::FN>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[P][j], acc[i][j], C::AFP8 ? 0 : 4,
                                                                  C::BFP8 ? 0 : 4, 0, (int)f.sa[i], j,
                                                                  (int)f.sb[P]);
    });
    constexpr int q0 = i * C::DPS / C::FM, q1 = (i + 1) * C::DPS / C::FM;
    issue_part(std::integral_constant<int, q0>{}, std::integral_constant<int, q1>{});
    constexpr int NRB = i < 2 ? (C::FN / 2) * (C::BFP8 ? 2 : 1) + (i == 1 ? C::FN : 0) : 0;  // B reads here
    constexpr int PER = (NRB + C::FN - 1) / C::FN;
    unroll<C::FN>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if constexpr (PER > 0) __builtin_amdgcn_sched_group_barrier(0x100, PER, 1);
      constexpr int nd = (m + 1) * (q1 - q0) / C::FN - m * (q1 - q0) / C::FN;
      if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x060, nd, 1);
    });
    __builtin_amdgcn_sched_barrier(0);
    read_a_frag<C>(nxt, i, f.a[i], f.sa[i], wm, h, l32);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Wait until this wave's DMAs of the stage about to be consumed have landed,
// given how many stages it issued after that one (DPS instructions each).
template <class C, int K>
__device__ __forceinline__ bool wait_if_after(int stages_after) {
  if (K > 0 && stages_after < K) return false;  // K = 0: wait for everything
  wait_vmcnt<K * C::DPS>();
  return true;
}
template <class C, int... Ks>
__device__ __forceinline__ void wait_stage_impl(int stages_after, std::integer_sequence<int, Ks...>) {
  // largest K first: at most STAGES-2 stages can follow the one awaited
  (void)(wait_if_after<C, C::STAGES - 2 - Ks>(stages_after) || ...);
}
template <class C>
__device__ __forceinline__ void wait_stage(int stages_after) {
  wait_stage_impl<C>(stages_after, std::make_integer_sequence<int, C::STAGES - 1>{});
}

// The pipelined persistent loop shared by all passes.
//   src.count()       number of tiles
//   src.ops(t, side)  TileOps of tile t; side 0 the issuing side, 1 the
//                     computing side (each keeps its own segment cursor)
//   src.epilogue(...) stores tile t (the last tile ops(t, 1) was asked for)
// Tiles are visited t = first, first + gridDim.x, ... (last to first on the
// odd XCDs when Src::kDesync).
// FAST (read-ahead loop only): every tile's contraction is a multiple of BK
// and the scale offsets fit 32 bits; the DMAs take the fast issue above.
template <class C, bool FAST = false, class Src>
__device__ __forceinline__ void persistent_loop(Src& src, uint8_t* smem, int64_t lda, int64_t ldas, int64_t ldb,
                                                int64_t ldbs) {
  static_assert(!FAST || C::SCHED == 7 || C::SCHED == 8 || C::SCHED == 5, "fast issue: read-ahead or 3-stage loop");
  static_assert(!FAST || !C::BLK, "fast issue: scales applied by the MFMA");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / C::WN, wn = w % C::WN;
  const int h = lane >> 5, l32 = lane & 31;
  uint8_t* scratch = smem + C::EPI_OFF + w * C::EPI_BYTES;
  const int total = src.count();
  const int stride = gridDim.x;
  const int nb = gridDim.x, b = blockIdx.x;
  // consecutive logical ids on one XCD (the hardware deals block ids
  // round-robin over the 8 XCDs), so co-resident tiles share operands in L2
  const int first = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  // Src::kDesync: the workgroups of odd XCDs take their tiles in reverse.
  // Each still computes the same tiles, but neighbouring XCDs no longer run
  // tiles of one expert (one contraction length) in lockstep, so their
  // HBM-bound epilogues do not all fall on the same moments.
  const int nmine = first < total ? (total - 1 - first) / stride + 1 : 0;
  const bool rev = Src::kDesync && (b & 1) != 0;
  auto tile_at = [&](int x) { return rev ? first + (nmine - 1 - (x - first) / stride) * stride : x; };

  // issuing side: the tile and stage whose DMAs go out next
  int it = first, is = 0, ins = 0, slot_issue = 0;
  TileOps iops{};
  // Zero until the first tile with a contraction is planned: a workgroup
  // whose tiles all have empty contractions issues only dummy stages, whose
  // zero-page selection holds only while every chunk offset (kA, kB) and
  // scale block (sBlk) of the plan is >= 0.
  DmaPlan<C> plan{};
  FastPlan<C> fplan{};
  // the stage read-ahead loop issues with recomputed lane offsets
  constexpr bool LEAN = FAST && C::SCHED == 8;
  LeanPlan<C> lplan{};
  if constexpr (LEAN) {
    const uint8_t* z = reinterpret_cast<const uint8_t*>(g_zero_page);
    lplan.a = lplan.b = lplan.as = lplan.bs = z;  // rows clamp to 0: offsets below 64 bytes
  } else if constexpr (FAST) {
    // dummy stages before any planned tile read the zero page at offset 0
    const uint8_t* z = reinterpret_cast<const uint8_t*>(g_zero_page);
    fplan.a = fplan.b = fplan.sb = z;
    unroll<C::DSA>([&](auto ic) { fplan.s[decltype(ic)::value] = z; });
  }
  auto load_issue_tile = [&]() {
    while (it < total) {
      iops = src.ops(tile_at(it), 0);
      ins = (iops.kc + C::BK - 1) / C::BK;
      if (ins > 0) break;
      it += stride;  // tiles with an empty contraction issue nothing
    }
    if (it < total) {
      if constexpr (LEAN) {
        plan_lean<C>(lplan, iops);
      } else {
        plan_dma<C>(plan, iops, lda, ldas, ldb, ldbs, w, lane);
        if constexpr (FAST) plan_fast<C>(fplan, plan, iops, ldas, ldbs, w);
      }
    }
  };
  auto issue_one = [&]() -> int {
    if (it >= total) return 0;
    issue_stage<C>(plan, iops, is, smem + slot_issue * C::STAGE_BYTES, w, ldas, ldbs);
    slot_issue = slot_issue + 1 == C::STAGES ? 0 : slot_issue + 1;
    if (++is == ins) {
      is = 0;
      it += stride;
      load_issue_tile();
    }
    return 1;
  };

  load_issue_tile();
  int ahead = 0;  // stages issued and not yet consumed
  int slot_comp = 0;
  if constexpr (C::SCHED == 7) {
    auto advance_issue = [&](bool dummy) {
      slot_issue = slot_issue + 1 == C::STAGES ? 0 : slot_issue + 1;
      if (!dummy && ++is == ins) {
        is = 0;
        it += stride;
        load_issue_tile();
      }
    };
    for (int q = 0; q < C::STAGES - 1; ++q) {
      const bool dummy = it >= total;
      if constexpr (FAST) issue_stage_fast<C>(fplan, dummy ? 0 : is, smem + slot_issue * C::STAGE_BYTES, w);
      else issue_stage<C>(plan, iops, is, smem + slot_issue * C::STAGE_BYTES, w, ldas, ldbs, dummy);
      advance_issue(dummy);
    }
    // stage 0 (of the first tile, or a dummy) has landed: its K step 0
    // operands go to registers
    KOps<C> f0, f1;
    // the zero page's address, held in registers (otherwise the compiler
    // reloads it from the GOT inside the loop, and that scalar load makes
    // the wave wait for every LDS read in flight)
    const uint8_t* zero = reinterpret_cast<const uint8_t*>(g_zero_page);
    asm volatile("" : "+s"(zero));
    const uint8_t* bsrc[C::DB];
    unroll<C::DB>([&](auto ic) { bsrc[decltype(ic)::value] = zero; });
    // fast issue: the pending B chunks' base and lane offsets
    const uint8_t* bbase = zero;
    uint32_t bvoff[C::DB];
    unroll<C::DB>([&](auto ic) { bvoff[decltype(ic)::value] = 0; });
    uint8_t* bdst = smem + slot_issue * C::STAGE_BYTES;
    wait_vmcnt<(C::STAGES - 2) * C::DPS>();
    raw_barrier();
    read_kops<C, 0>(smem, f0, wm, wn, h, l32);
    bool pending = false, pending_dummy = false;
    for (int ct = first; ct < total; ct += stride) {
      const TileOps cops = src.ops(tile_at(ct), 1);
      const int cns = (cops.kc + C::BK - 1) / C::BK;
      v16f acc[C::FM][C::FN];
      unroll<C::FM>([&](auto ic) { unroll<C::FN>([&](auto jc) { acc[ic][jc] = v16f{}; }); });
      for (int s = 0; s < cns; ++s) {
        // the issue state advances here (its branches stay out of the
        // step's straight-line block)
        if (pending) advance_issue(pending_dummy);
        const bool dummy = it >= total;
        uint8_t* dst = smem + slot_issue * C::STAGE_BYTES;
        const int slot_next = slot_comp + 1 == C::STAGES ? 0 : slot_comp + 1;
        // first half: the B chunks of the stage whose A chunks and scales
        // went out in the previous step's second half (same stage, same
        // slot; in the first step, zero-page DMAs into the slot the prologue
        // left empty, which that stage's own DMAs follow in issue order)
        ra_half<C, 1, 1, C::DB>(smem + slot_comp * C::STAGE_BYTES, f0, f1, acc, wm, wn, h, l32,
                                [&]() __attribute__((always_inline)) {
                                  if constexpr (FAST) {
                                    unroll<C::DB>([&](auto ic) {
                                      constexpr int i = decltype(ic)::value;
                                      dma16(bbase + bvoff[i], bdst + C::B_OFF + (i * C::NW + w) * 1024);
                                    });
                                  } else {
                                    issue_b_srcs<C>(bsrc, bdst, w);
                                  }
                                });
        __builtin_amdgcn_sched_barrier(0);
        // the next stage has landed (this wave's DMAs: STAGES-3 stages were
        // issued after it; the barrier covers the other waves')
        wait_vmcnt<(C::STAGES - 3) * C::DPS>();
        raw_barrier();
        __builtin_amdgcn_sched_barrier(0);
        ra_half<C, 0, 2, C::DPS - C::DB>(smem + slot_next * C::STAGE_BYTES, f1, f0, acc, wm, wn, h, l32,
                                         [&]() __attribute__((always_inline)) {
                                           if constexpr (FAST)
                                             issue_stage_fast<C, 0>(fplan, dummy ? 0 : is, dst, w);
                                           else
                                             issue_stage<C, 0>(plan, iops, is, dst, w, ldas, ldbs, dummy, zero);
                                         });
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (FAST) {
          bbase = fplan.b + (dummy ? 0 : is) * fplan.bstep;
          unroll<C::DB>([&](auto ic) { bvoff[decltype(ic)::value] = fplan.vB[decltype(ic)::value]; });
        } else {
          stage_b_srcs<C>(plan, iops, is, dummy, zero, bsrc);
        }
        bdst = dst;
        pending = true;
        pending_dummy = dummy;
        slot_comp = slot_next;
      }
      // The slot before slot_comp held the last stage consumed (before any,
      // the one slot the prologue left empty); its next DMA goes out after
      // the next barrier. Every wave's reads of it were consumed by MFMAs
      // issued before this barrier, so it is free for the epilogue.
      const int slot_free = slot_comp == 0 ? C::STAGES - 1 : slot_comp - 1;
      raw_barrier();
      src.epilogue(tile_at(ct), acc, smem + slot_free * C::STAGE_BYTES + w * C::EPI_BYTES, w, lane);
      // A tile with an empty contraction consumed no stage, so the next
      // step's first-half DMAs may target the slot its epilogue used (the
      // prologue's empty slot): every wave finishes the epilogue first.
      if (cns == 0) raw_barrier();
    }
    wait_vmcnt<0>();
    return;
  }
  if constexpr (C::SCHED == 8) {
    // Stage read-ahead with one K step per stage: every step waits for the
    // NEXT stage (STAGES-3 stages were issued after it), passes the barrier,
    // and then runs the MFMAs of the current stage (operands read during the
    // previous step) interleaved with the reads of the next stage and the
    // DMAs of a later stage into the slot of the previous one. The barrier
    // admits the reads (every wave's DMAs of the next stage have landed) and
    // frees that slot (every wave's reads of it were consumed by MFMAs issued
    // before the barrier). No LDS read sits between the barrier and the first
    // MFMA after it, and fragments alternate between two register sets.
    auto advance_issue = [&](bool dummy) {
      slot_issue = slot_issue + 1 == C::STAGES ? 0 : slot_issue + 1;
      if (!dummy && ++is == ins) {
        is = 0;
        it += stride;
        load_issue_tile();
      }
    };
    // uniform strides for the lean issue (the ABI keeps a tile's span below 2^31)
    const int ilda = __builtin_amdgcn_readfirstlane((int)lda), ildb = __builtin_amdgcn_readfirstlane((int)ldb);
    const int ildas = __builtin_amdgcn_readfirstlane((int)ldas), ildbs = __builtin_amdgcn_readfirstlane((int)ldbs);
    for (int q = 0; q < C::STAGES - 1; ++q) {
      const bool dummy = it >= total;
      if constexpr (LEAN)
        issue_stage_lean<C>(lplan, dummy ? 0 : is, smem + slot_issue * C::STAGE_BYTES, w, lane, ilda, ildb, ildas,
                            ildbs);
      else if constexpr (FAST) issue_stage_fast<C>(fplan, dummy ? 0 : is, smem + slot_issue * C::STAGE_BYTES, w);
      else issue_stage<C>(plan, iops, is, smem + slot_issue * C::STAGE_BYTES, w, ldas, ldbs, dummy);
      advance_issue(dummy);
    }
    const uint8_t* zero = reinterpret_cast<const uint8_t*>(g_zero_page);
    asm volatile("" : "+s"(zero));
    ROps<C> f;
    wait_vmcnt<(C::STAGES - 2) * C::DPS>();
    raw_barrier();
    read_b_part<C, 0, C::FN, true>(smem, f.b[0], f.sb[0], wn, h, l32);
    unroll<C::FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      read_a_frag<C>(smem, i, f.a[i], f.sa[i], wm, h, l32);
    });
    bool pending = false, pending_dummy = false;
    v16f acc[C::FM][C::FN];
    auto step = [&](auto pc) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      if (pending) advance_issue(pending_dummy);
      const bool dummy = it >= total;
      uint8_t* dst = smem + slot_issue * C::STAGE_BYTES;
      const int slot_next = slot_comp + 1 == C::STAGES ? 0 : slot_comp + 1;
      wait_vmcnt<(C::STAGES - 3) * C::DPS>();
      raw_barrier();
      __builtin_amdgcn_sched_barrier(0);
      ra_step<C, P>(smem + slot_next * C::STAGE_BYTES, f, acc, wm, wn, h, l32,
                    [&](auto q0c, auto q1c) __attribute__((always_inline)) {
                      constexpr int q0 = decltype(q0c)::value, q1 = decltype(q1c)::value;
                      if constexpr (LEAN) {
                        issue_stage_lean<C, q0, q1>(lplan, dummy ? 0 : is, dst, w, lane, ilda, ildb, ildas, ildbs);
                      } else if constexpr (q0 == 0) {
                        issue_stage<C>(plan, iops, is, dst, w, ldas, ldbs, dummy, zero);
                      }
                    });
      __builtin_amdgcn_sched_barrier(0);
      pending = true;
      pending_dummy = dummy;
      slot_comp = slot_next;
    };
    for (int ct = first; ct < total; ct += stride) {
      const TileOps cops = src.ops(tile_at(ct), 1);
      const int cns = (cops.kc + C::BK - 1) / C::BK;
      unroll<C::FM>([&](auto ic) { unroll<C::FN>([&](auto jc) { acc[ic][jc] = v16f{}; }); });
      int s = 0;
      for (; s + 2 <= cns; s += 2) {
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
      }
      if (s < cns) {
        step(std::integral_constant<int, 0>{});
        // the next stage's B fragments go back to the first set
        unroll<C::FN>([&](auto jc) { f.b[0][decltype(jc)::value] = f.b[1][decltype(jc)::value]; });
        f.sb[0] = f.sb[1];
      }
      // the slot of the last stage consumed (before any, the one the prologue
      // left empty) takes its next DMA after the next barrier: free for the
      // epilogue once every wave has issued its last MFMAs
      const int slot_free = slot_comp == 0 ? C::STAGES - 1 : slot_comp - 1;
      raw_barrier();
      src.epilogue(tile_at(ct), acc, smem + slot_free * C::STAGE_BYTES + w * C::EPI_BYTES, w, lane);
      if (cns == 0) raw_barrier();
    }
    wait_vmcnt<0>();
    return;
  }
  if constexpr (C::SCHED == 5) {
    // Every step issues exactly one stage (a dummy from the zero page once no
    // work is left), so STAGES-2 stages always follow the one awaited and the
    // wait is a constant; the DMAs go out inside the stage's MFMA block.
    auto advance_issue = [&](bool dummy) {
      slot_issue = slot_issue + 1 == C::STAGES ? 0 : slot_issue + 1;
      if (!dummy && ++is == ins) {
        is = 0;
        it += stride;
        load_issue_tile();
      }
    };
    for (int q = 0; q < C::STAGES - 1; ++q) {
      const bool dummy = it >= total;
      if constexpr (FAST) issue_stage_fast<C>(fplan, dummy ? 0 : is, smem + slot_issue * C::STAGE_BYTES, w);
      else issue_stage<C>(plan, iops, is, smem + slot_issue * C::STAGE_BYTES, w, ldas, ldbs, dummy);
      advance_issue(dummy);
    }
    bool pending = false, pending_dummy = false;
    for (int ct = first; ct < total; ct += stride) {
      const TileOps cops = src.ops(tile_at(ct), 1);
      const int cns = (cops.kc + C::BK - 1) / C::BK;
      v16f acc[C::FM][C::FN];
      unroll<C::FM>([&](auto ic) { unroll<C::FN>([&](auto jc) { acc[ic][jc] = v16f{}; }); });
      for (int s = 0; s < cns; ++s) {
        // the previous step's issue state advances here, ahead of the wait,
        // so that its branches (a new tile's set-up) do not split this
        // step's DMA + MFMA block
        if (pending) advance_issue(pending_dummy);
        const bool dummy = it >= total;
        uint8_t* dst = smem + slot_issue * C::STAGE_BYTES;
        wait_vmcnt<(C::STAGES - 2) * C::DPS>();
        raw_barrier();
        compute_stage<C>(smem + slot_comp * C::STAGE_BYTES, acc, wm, wn, h, l32,
                         [&]() __attribute__((always_inline)) {
                           if constexpr (FAST) issue_stage_fast<C>(fplan, dummy ? 0 : is, dst, w);
                           else issue_stage<C>(plan, iops, is, dst, w, ldas, ldbs, dummy);
                         });
        pending = true;
        pending_dummy = dummy;
        slot_comp = slot_comp + 1 == C::STAGES ? 0 : slot_comp + 1;
      }
      src.epilogue(tile_at(ct), acc, scratch, w, lane);
    }
    wait_vmcnt<0>();
    return;
  }
  for (int q = 0; q < C::STAGES - 1; ++q) ahead += issue_one();

  for (int ct = first; ct < total; ct += stride) {
    const TileOps cops = src.ops(tile_at(ct), 1);
    const int cns = (cops.kc + C::BK - 1) / C::BK;
    v16f acc[C::FM][C::FN];
    unroll<C::FM>([&](auto ic) { unroll<C::FN>([&](auto jc) { acc[ic][jc] = v16f{}; }); });
    v16f P[C::BLK ? C::FM : 1][C::BLK ? C::FN : 1];
    for (int s = 0; s < cns; ++s) {
      wait_stage<C>(ahead - 1);
      raw_barrier();
      // the slot refilled now held the stage every wave consumed last step
      ahead += issue_one();
      if constexpr (C::BLK) {
        const uint8_t* st = smem + slot_comp * C::STAGE_BYTES;
        if constexpr (C::PROMO == 1) {
          compute_stage_blk<C, true, true>(st, acc, P, wm, wn, h, l32);
        } else {
          if ((s & 1) == 0) compute_stage_blk<C, true, false>(st, acc, P, wm, wn, h, l32);
          else compute_stage_blk<C, false, true>(st, acc, P, wm, wn, h, l32);
        }
      } else {
        compute_stage<C>(smem + slot_comp * C::STAGE_BYTES, acc, wm, wn, h, l32);
      }
      slot_comp = slot_comp + 1 == C::STAGES ? 0 : slot_comp + 1;
      --ahead;
    }
    src.epilogue(tile_at(ct), acc, scratch, w, lane);
  }
  wait_vmcnt<0>();  // no DMA of this workgroup outlives it (every issued stage was waited for; kept explicit)
}

// ---------------------------------------------------------------------------
// epilogue: a 16-row half of one 32x32 fragment goes through the wave's
// scratch (row pitch 36 floats: 16-byte aligned rows, lane halves 16 banks
// apart), then each lane owns row l/4, columns 8*(l%4) .. +8 of the half for
// 16-byte global accesses
// ---------------------------------------------------------------------------
constexpr int kEpiPitch = 36;

// A raw buffer over `bytes` bytes from a wave-uniform base: accesses at
// offsets past the end read 0 and write nothing, which masks rows and
// columns outside an output without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_buffer(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
constexpr uint32_t kBufferOutside = 0x80000000u;  // an offset past every buffer's end
// Cache policy of accesses to data touched once (the non-temporal bit):
// the output stream then does not evict the operand panels the next tiles
// re-read from L2. Measured on the weight gradient's output: fc1 shapes
// 752 -> 675 us accumulating, 604 -> 443 us overwriting; blockwise
// 2.05 -> 1.92 ms.
constexpr int kStreamAux = 2;
// Accumulating weight-gradient epilogue: 16-row halves whose old output
// values are in flight while a half is stored (fc1: 1 half 660 us, 2 halves
// 652-656 us, 3 halves 647-655 us but the MXFP8 one at the a8w4 shapes 3.18
// -> 3.21 ms).
constexpr int kEpiLoadAhead = 2;

// Keeps an accumulator fragment in accumulation registers up to its use in
// an epilogue, for wave tiles of 256 accumulators per lane (128x128): without
// it the compiler copies every fragment into vector registers at the end of
// the stage loop, which needs as many vector registers as there are
// accumulators and spills the loop's state. Smaller wave tiles keep the
// compiler's placement (measured faster there).
template <class C>
__device__ __forceinline__ void pin_acc(v16f& v) {
  if constexpr (C::FM * C::FN * 16 > 128) asm volatile("" : "+a"(v));
}

template <int HF>
__device__ __forceinline__ void frag_half_rows(const v16f& v, float* scr, int lane, float (&o)[8]) {
  const int h = lane >> 5, l32 = lane & 31;
  unroll<8>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    const int rr = 8 * (q / 4) + 4 * h + (q % 4);
    scr[rr * kEpiPitch + l32] = v[HF * 8 + q];
  });
  const int rr = lane >> 2, cc = (lane & 3) * 8;
  const v4f lo = *reinterpret_cast<const v4f*>(scr + rr * kEpiPitch + cc);
  const v4f hi = *reinterpret_cast<const v4f*>(scr + rr * kEpiPitch + cc + 4);
  o[0] = lo[0]; o[1] = lo[1]; o[2] = lo[2]; o[3] = lo[3];
  o[4] = hi[0]; o[5] = hi[1]; o[6] = hi[2]; o[7] = hi[3];
}

typedef __bf16 v2bf16_t __attribute__((ext_vector_type(2)));
typedef float v2f_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32), 8 values -> 16 bytes
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t{a, b}), v2bf16_t));
}
__device__ __forceinline__ uint4 pack_bf16x8(const float (&o)[8]) {
  return make_uint4(cvt_bf16x2(o[0], o[1]), cvt_bf16x2(o[2], o[3]), cvt_bf16x2(o[4], o[5]), cvt_bf16x2(o[6], o[7]));
}

// Tile order inside an expert's R x Cn tile grid: groups of kTileGroup row
// tiles walked column by column (the group's rows fastest). The tiles that
// run at the same time (consecutive ids, 32 per XCD) then form a
// kTileGroup x 32/kTileGroup block instead of a run along one row of tiles,
// so an expert's weight tiles are re-read from beyond the XCD's L2 once per
// kTileGroup row tiles rather than once per 32/Cn. Measured at the fc1
// shapes: input gradient 342 -> 308 us (Cn = 16), forward and weight
// gradient unchanged; groups of 2 and 8 were slower. The MX weight gradients
// (fp32 main_grad read-modify-write) take groups of 5: fc1 670 -> 656 us,
// MXFP8 at the a8w4 shapes 3.20 -> 3.18 ms (groups of 3 and 6 in between, 12
// slower than 4); the blockwise one stays at 4.
constexpr int kTileGroup = 4, kTileGroupMxWgrad = 5;
template <int GROUP = kTileGroup>
__device__ __forceinline__ void grouped_tile(int local, int R, int Cn, int& rt, int& ct) {
  const int r0 = local / (GROUP * Cn) * GROUP;
  const int h = R - r0 < GROUP ? R - r0 : GROUP;
  const int in = local - r0 * Cn;
  ct = in / h;
  rt = r0 + (in - ct * h);
}

// ---------------------------------------------------------------------------
// forward / input gradient
// ---------------------------------------------------------------------------
// Row alignment mask of a rows-kernel tile start (MX: multiples of 4).
template <class C>
constexpr int kRowAlign = C::F32S ? 0 : 3;

// Number of BM-row tiles of an expert with m rows starting at row `start`.
template <class C>
__host__ __device__ inline int64_t expert_row_tiles(int64_t start, int64_t m) {
  return m > 0 ? (m + (start & kRowAlign<C>) + C::BM - 1) / C::BM : 0;
}

template <class C>
struct RowsSource {
  static constexpr bool kDesync = false;
  const RowsGemmParams& p;
  const int64_t* pref;       // LDS: first row of each expert's segment
  const int32_t* tile_offs;  // LDS
  int G, n_tiles, ntot;
  int cursor[2] = {-1, -1};  // segment cursors of the issuing and computing sides

  __device__ __forceinline__ int count() const { return ntot; }

  struct Pos { int g, mt, nt; };
  Pos cur{};                 // the computing side's last tile
  __device__ __forceinline__ Pos pos(int t, int side) {
    const int g = seek_segment(tile_offs, G + 1, t, cursor[side]);
    const int local = t - tile_offs[g];
    Pos q{g, 0, 0};
    grouped_tile(local, (tile_offs[g + 1] - tile_offs[g]) / n_tiles, n_tiles, q.mt, q.nt);
    if (side) cur = q;
    return q;
  }
  // Tile rows: MX tiles start at a multiple of 4 (the scale DMA moves four
  // rows per lane), so an expert's first tile may begin up to 3 rows before
  // its segment; rows outside [lo, hi) belong to other experts and are
  // computed but never stored.
  struct Rows { int64_t row0; int lo, hi; };
  __device__ __forceinline__ Rows rows(const Pos& q) const {
    const int64_t start = pref[q.g];
    const int64_t row0 = (start & ~(int64_t)kRowAlign<C>) + (int64_t)q.mt * C::BM;
    return Rows{row0, (int)(start - row0), (int)(start + p.sp.m[q.g] - row0)};
  }
  __device__ __forceinline__ TileOps ops(int t, int side) {
    const Pos q = pos(t, side);
    const Rows rw = rows(q);
    const int col0 = q.nt * C::BN;
    const int nleft = p.n_out - col0;
    TileOps o;
    o.a = p.a + data_off<C, false>(rw.row0, 0, p.lda);
    // A's scales are block-major ([blocks, rows]: u8, or fp32 for 1x128)
    o.as = p.as + (C::F32S ? rw.row0 * 4 : rw.row0);
    o.b = p.b + (int64_t)q.g * p.b_gstride + data_off<C, true>(col0, 0, p.ldb);
    o.bs = p.bs + (int64_t)q.g * p.bs_gstride +
           (C::F32S ? (int64_t)(col0 / C::BDIV) * p.ldbs : C::MFB ? (int64_t)col0 * 4 : (int64_t)col0);
    o.mrows = rw.hi < C::BM ? rw.hi : C::BM;
    o.nrows = nleft < C::BN ? nleft : C::BN;
    o.srows_a = (int)(p.ldas - rw.row0);  // MX: the padded row count is the block stride
    // MFMA layout: B's rows are padded to 32 (N and K are multiples of 32)
    o.srows_b = C::MFB ? (nleft + 31) / 32 * 128 : nleft;
    o.kc = p.kc;
    return o;
  }
  __device__ __forceinline__ void epilogue(int t, v16f (&acc)[C::FM][C::FN], uint8_t* scratch, int w, int lane) {
    (void)t;
    const Pos q = cur;
    const Rows rw = rows(q);
    const int64_t row0 = rw.row0;
    const int mlo = rw.lo, mleft = rw.hi;
    const int col0 = q.nt * C::BN;
    const int ncols = p.n_out - col0;
    const int wm = w / C::WN, wn = w % C::WN;
    float* scr = reinterpret_cast<float*>(scratch);
    const int rr = lane >> 2, cc = (lane & 3) * 8;
    unroll<C::FM>([&](auto ic) {
      unroll<C::FN>([&](auto jc) {
        constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
        unroll<2>([&](auto hc) {
          constexpr int hf = decltype(hc)::value;
          float o[8];
          pin_acc<C>(acc[i][j]);
          frag_half_rows<hf>(acc[i][j], scr, lane, o);
          const int row = wm * C::WTM + i * 32 + 16 * hf + rr;
          const int col = wn * C::WTN + j * 32 + cc;
          if (row >= mlo && row < mleft && col < ncols)
            *reinterpret_cast<uint4*>(p.c + (row0 + row) * p.ldc + col0 + col) = pack_bf16x8(o);
        });
      });
    });
  }
};

template <class C, bool FAST>
__device__ __forceinline__ void grouped_rows_body(const RowsGemmParams& p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int64_t pref[kMaxExperts + 1];
  __shared__ int64_t tpref[kMaxExperts + 1];
  __shared__ int64_t wtot[C::THREADS / 64];
  __shared__ int32_t tile_offs[kMaxExperts + 1];

  const int G = p.sp.G;
  const int n_tiles = (p.n_out + C::BN - 1) / C::BN;
  block_prefix64<C::THREADS>(G, [&](int g) { return (int64_t)p.sp.m[g]; }, pref, wtot);
  block_prefix64<C::THREADS>(G, [&](int g) { return expert_row_tiles<C>(pref[g], p.sp.m[g]); }, tpref, wtot);
  for (int g = threadIdx.x; g <= G; g += C::THREADS) tile_offs[g] = (int32_t)tpref[g] * n_tiles;
  __syncthreads();

  RowsSource<C> src{p, pref, tile_offs, G, n_tiles, tile_offs[G]};
  persistent_loop<C, FAST>(src, smem, p.lda, p.ldas, p.ldb, p.ldbs);
}

// The forward and the input gradient run the same body; each pass has its own
// kernel symbol so that traces and profiles report the two passes apart.
template <class C, bool FAST>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_fwd_kernel(const RowsGemmParams p) {
  grouped_rows_body<C, FAST>(p);
}
template <class C, bool FAST>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_dgrad_kernel(const RowsGemmParams p) {
  grouped_rows_body<C, FAST>(p);
}

// ---------------------------------------------------------------------------
// variable-K weight gradient
// ---------------------------------------------------------------------------
// Output mode of the weight gradient, a template parameter so a kernel holds
// only its own epilogue (the accumulating epilogues' loads into registers
// otherwise make the compiler drain the DMA ring at every stage head).
enum : int { kEpiF32Acc = 0, kEpiF32Set = 1, kEpiBf16Set = 2, kEpiBf16Acc = 3 };

template <class C, bool FAST, int EPI>
struct WgradSource {
  // Accumulating epilogues read and write the output (HBM-bound): desync the
  // XCDs (persistent_loop). Measured at the fc1 shapes, fp32 accumulate:
  // 700 -> 668 us; the overwriting blockwise weight gradient was slower
  // (1.71 -> 1.79 ms), so the other modes keep one order.
  static constexpr bool kDesync = EPI == kEpiF32Acc || EPI == kEpiBf16Acc;
  const WgradParams& p;
  const int64_t* pad_pref;   // LDS: padded segment offsets (natural expert order)
  const int32_t* tile_offs;  // LDS: tile offsets in longest-first order
  const int16_t* order;      // LDS: the expert at each position of that order
  int G, tc, ntot;
  int cursor[2] = {-1, -1};  // segment cursors of the issuing and computing sides

  __device__ __forceinline__ int count() const { return ntot; }

  struct Pos { int g, row0, col0; int64_t p0; int kc; };
  Pos cur{};                 // the computing side's last tile
  __device__ __forceinline__ Pos pos(int t, int side) {
    const int j = seek_segment(tile_offs, G + 1, t, cursor[side]);
    // the expert order from its LDS copy: a kernel-argument read with a
    // lane-varying index is a vector memory load whose wait drains every DMA
    // in flight once per tile
    const int g = order[j];
    const int local = t - tile_offs[j];
    int rt, ct;
    grouped_tile<C::F32S ? kTileGroup : kTileGroupMxWgrad>(local, (p.n_rows + C::BM - 1) / C::BM, tc, rt, ct);
    const int64_t p0 = pad_pref[g];
    const Pos q{g, rt * C::BM, ct * C::BN, p0, (int)(pad_pref[g + 1] - p0)};
    if (side) cur = q;
    return q;
  }
  __device__ __forceinline__ TileOps ops(int t, int side) {
    const Pos q = pos(t, side);
    TileOps o;
    // segment start: element bytes (E4M3: 1, E2M1: 1/2); scales, MX
    // block-major (block p0/32, row row0), blockwise block-major too (fp32,
    // block p0/128, row row0)
    o.a = p.a + data_off<C, false>(q.row0, C::AFP8 ? q.p0 : q.p0 / 2, p.lda);
    o.b = p.b + data_off<C, true>(q.col0, C::BFP8 ? q.p0 : q.p0 / 2, p.ldb);
    if constexpr (C::F32S) {
      o.as = p.as + q.p0 / 128 * p.ldas + (int64_t)q.row0 * 4;
      o.bs = p.bs + q.p0 / 128 * p.ldbs + (int64_t)q.col0 * 4;
    } else {
      o.as = p.as + q.p0 / 32 * p.ldas + q.row0;
      o.bs = p.bs + q.p0 / 32 * p.ldbs + q.col0;
    }
    const int rl = p.n_rows - q.row0, cl = p.n_cols - q.col0;
    o.mrows = rl < C::BM ? rl : C::BM;
    o.nrows = cl < C::BN ? cl : C::BN;
    o.srows_a = rl;  // n_rows and n_cols are multiples of 32, the block strides
    o.srows_b = cl;
    o.kc = q.kc;
    return o;
  }
  // The epilogue writes whole rows of the wave's tile, 16 rows (a half
  // fragment row) at a time: the half of every column fragment goes through
  // the wave's LDS scratch, then each lane takes CPL consecutive columns of
  // one row (16 bytes of output), so one store covers 64/(WTN/CPL) rows of
  // WTN contiguous columns (a CU stores contiguous runs about 3x faster than
  // 128-byte row pieces, measured). Accesses go through a buffer over the
  // half's valid rows, with columns past the output sent past its end: no
  // branches, so the compiler counts the outstanding memory operations
  // exactly; both are non-temporal. Accumulate: the old values of the next
  // kEpiLoadAhead halves are loaded before this half's stores, so loads and
  // stores overlap.
  template <bool BF16, bool ACC>
  __device__ __forceinline__ void store_tile(const Pos& q, v16f (&acc)[C::FM][C::FN], float* scr, int w, int lane) {
    constexpr int CPL = BF16 ? 8 : 4;   // columns per lane
    constexpr int ESZ = BF16 ? 2 : 4;   // output element bytes
    constexpr int LPR = C::WTN / CPL;   // lanes per row
    constexpr int RPI = 64 / LPR;       // rows per instruction
    constexpr int NI = 16 / RPI;        // instructions per half
    constexpr int NH = 2 * C::FM;       // halves per wave tile
    constexpr int P = C::EPI_PITCH;
    static_assert(64 % LPR == 0 && 16 % RPI == 0, "whole rows per instruction");
    const int rl = p.n_rows - q.row0, cl = p.n_cols - q.col0;
    const int wm = w / C::WN, wn = w % C::WN;
    // the lane's terms are recomputed per tile, not hoisted out of the tile
    // loop (where they would hold registers through the stage loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int h = ln >> 5, l32 = ln & 31;
    const int lr = ln / LPR, lc = (ln % LPR) * CPL;  // row within an instruction, first column
    const int col = wn * C::WTN + lc;
    const uint32_t row_bytes = (uint32_t)p.n_cols * ESZ;  // < 2^25: n_cols < 2^23
    const uint32_t coff = col < cl ? (uint32_t)col * ESZ : kBufferOutside;
    char* const tile = reinterpret_cast<char*>(p.c) + (((int64_t)q.g * p.n_rows + q.row0) * p.n_cols + q.col0) * ESZ;
    // half k: rows wm*WTM + 16k .. +16 of the tile (k = 2i + hf)
    auto half_buffer = [&](int k) {
      const int r0 = wm * C::WTM + 16 * k;
      const int n = rl - r0 < 0 ? 0 : (rl - r0 > 16 ? 16 : rl - r0);
      return uniform_buffer(tile + (int64_t)r0 * row_bytes, (uint32_t)n * row_bytes);  // <= 2^29 bytes
    };
    auto off = [&](int t) { return (uint32_t)(t * RPI + lr) * row_bytes + coff; };
    constexpr int D = kEpiLoadAhead < NH ? kEpiLoadAhead : NH;
    v4i old[D + 1][ACC ? NI : 1];
    auto load_half = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const __amdgpu_buffer_rsrc_t bk = half_buffer(k);
      unroll<NI>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        old[k % (D + 1)][t] = __builtin_amdgcn_raw_buffer_load_b128(bk, off(t), 0, kStreamAux);
      });
    };
    if constexpr (ACC) unroll<D>([&](auto kc) { load_half(kc); });
    unroll<NH>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int i = k / 2, hf = k % 2;
      if constexpr (ACC && k + D < NH) load_half(std::integral_constant<int, k + D>{});
      // register q of a fragment is row 8*(q/4) + 4*(lane/32) + q%4, column lane%32
      unroll<C::FN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        pin_acc<C>(acc[i][j]);
        unroll<8>([&](auto qc) {
          constexpr int qq = decltype(qc)::value;
          const int rr = 8 * (qq / 4) + 4 * h + (qq % 4);
          scr[rr * P + j * 32 + l32] = acc[i][j][hf * 8 + qq];
        });
      });
      const __amdgpu_buffer_rsrc_t b = half_buffer(k);
      unroll<NI>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const float* src = scr + (t * RPI + lr) * P + lc;
        float o[CPL];
        unroll<CPL / 4>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          const v4f v = *reinterpret_cast<const v4f*>(src + 4 * u);
          o[4 * u] = v[0]; o[4 * u + 1] = v[1]; o[4 * u + 2] = v[2]; o[4 * u + 3] = v[3];
        });
        v4i d;
        if constexpr (BF16) {
          if constexpr (ACC) {
            const v4i ov = old[k % (D + 1)][t];
            unroll<4>([&](auto ec) {
              constexpr int e = decltype(ec)::value;
              o[2 * e] += __uint_as_float((uint32_t)ov[e] << 16);
              o[2 * e + 1] += __uint_as_float((uint32_t)ov[e] & 0xffff0000u);
            });
          }
          const uint4 pk = pack_bf16x8(o);
          d = v4i{(int)pk.x, (int)pk.y, (int)pk.z, (int)pk.w};
        } else {
          if constexpr (ACC) {
            const v4i ov = old[k % (D + 1)][t];
            unroll<4>([&](auto ec) { o[decltype(ec)::value] += __int_as_float(ov[decltype(ec)::value]); });
          }
          d = v4i{__float_as_int(o[0]), __float_as_int(o[1]), __float_as_int(o[2]), __float_as_int(o[3])};
        }
        __builtin_amdgcn_raw_buffer_store_b128(d, b, off(t), 0, kStreamAux);
      });
    });
  }
  __device__ __forceinline__ void epilogue(int t, v16f (&acc)[C::FM][C::FN], uint8_t* scratch, int w, int lane) {
    (void)t;
    const Pos q = cur;
    float* scr = reinterpret_cast<float*>(scratch);
    store_tile<EPI == kEpiBf16Set || EPI == kEpiBf16Acc, EPI == kEpiF32Acc || EPI == kEpiBf16Acc>(q, acc, scr, w,
                                                                                                  lane);
  }
};

template <class C, bool FAST, int EPI>
__global__ __launch_bounds__(C::THREADS, C::OCC) void grouped_wgrad_kernel(const WgradParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int64_t pad_pref[kMaxExperts + 1];
  __shared__ int64_t tile_pref[kMaxExperts + 1];
  __shared__ int64_t wtot[C::THREADS / 64];
  __shared__ int32_t tile_offs[kMaxExperts + 1];
  __shared__ int16_t order[kMaxExperts];

  const int G = p.sp.G;
  for (int j = threadIdx.x; j < G; j += C::THREADS) order[j] = p.order[j];
  const int tr = (p.n_rows + C::BM - 1) / C::BM, tc = (p.n_cols + C::BN - 1) / C::BN;
  constexpr int PAD = C::F32S ? 128 : 32;  // segment pad multiple of the column-wise operands
  block_prefix64<C::THREADS>(G, [&](int g) { return (int64_t)((p.sp.m[g] + PAD - 1) & ~(PAD - 1)); }, pad_pref,
                             wtot);
  block_prefix64<C::THREADS>(G, [&](int j) {
    const int g = p.order[j];
    return (int64_t)((p.sp.m[g] > 0 || !p.accumulate) ? tr * tc : 0);
  }, tile_pref, wtot);
  for (int j = threadIdx.x; j <= G; j += C::THREADS) tile_offs[j] = (int32_t)tile_pref[j];
  __syncthreads();

  WgradSource<C, FAST, EPI> src{p, pad_pref, tile_offs, order, G, tc, tile_offs[G]};
  persistent_loop<C, FAST>(src, smem, p.lda, p.ldas, p.ldb, p.ldbs);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// a4w4 forward and input gradient: 8 waves (128x64 each), 4-stage ring,
// read-ahead schedule; weight gradient: 4 waves (128x128 each), same ring
using CfgA4 = TileCfg<256, 256, 2, 4, 128, 4, kA4W4, 1, 7>;
using CfgA4W = TileCfg<256, 256, 2, 2, 128, 4, kA4W4, 1, 7>;
// MXFP8 weight gradient (E4M3 x E4M3, UE8M0 per 32): 64-deep stages (16 KiB
// per operand) in a 3-stage ring, DMAs between the MFMAs
using CfgA8W = TileCfg<256, 256, 2, 4, 64, 3, kA8A8, 1, 5>;
// a8w4 forward: a 128-deep stage holds 32 KiB of E4M3 A rows, so the ring
// has two stages (the DMAs go out right after the barrier)
using CfgA8 = TileCfg<256, 256, 2, 4, 128, 2, kA8W4, 1, 3>;
// blockwise FP8: four waves (one per SIMD) each hold a 64x64 accumulator and
// its per-128 partial; B scale rows are shared by 128 weight rows in the
// forward, one per row in the weight gradient. Every blockwise operand is
// stored in 64-byte K blocks (KBlocked).
using CfgBlkF = KBlocked<TileCfg<128, 128, 2, 2, 128, 3, kBlkFp8, 1, 0, 128>>;
using CfgBlkW = KBlocked<TileCfg<128, 128, 2, 2, 128, 3, kBlkFp8, 1, 0, 1>>;
// blockwise FP8 with power-of-two scales: the a4w4 loop (8 waves, 256x256)
// with E4M3 on both sides; a 64-deep stage holds 16 KiB of each operand
using CfgP2F = KBlocked<TileCfg<256, 256, 2, 4, 64, 3, kBlkP2, 1, 5, 128>>;
using CfgP2W = KBlocked<TileCfg<256, 256, 2, 2, 64, 4, kBlkP2, 1, 8, 1>>;

template <class C, class K, class P>
static hipError_t launch_persistent(K kernel, const P& p, int64_t tiles, int num_cus, hipStream_t st) {
  const hipError_t e = ensure_dynamic_lds((const void*)kernel, C::SMEM_BYTES, st);
  if (e != hipSuccess) return e;
  int64_t grid = (int64_t)num_cus * C::OCC;
  if (tiles < grid) grid = tiles;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(C::THREADS), C::SMEM_BYTES, st, p);
  return hipGetLastError();
}

template <class C>
static int64_t rows_tiles(const RowsGemmParams& p) {
  int64_t mt = 0, start = 0;
  for (int g = 0; g < p.sp.G; ++g) {
    mt += expert_row_tiles<C>(start, p.sp.m[g]);
    start += p.sp.m[g];
  }
  return mt * ((p.n_out + C::BN - 1) / C::BN);
}

template <class C, bool FAST>
static hipError_t launch_rows_as(const RowsGemmParams& p, bool dgrad, int num_cus, hipStream_t st) {
  if (dgrad) return launch_persistent<C>(grouped_dgrad_kernel<C, FAST>, p, rows_tiles<C>(p), num_cus, st);
  return launch_persistent<C>(grouped_fwd_kernel<C, FAST>, p, rows_tiles<C>(p), num_cus, st);
}

// The read-ahead loop takes the fast DMA issue when every stage is full and
// the per-lane scale offsets ((SB-1) blocks of ld bytes plus a row) fit 32 bits.
template <class C>
static hipError_t launch_rows(const RowsGemmParams& p, bool dgrad, int num_cus, hipStream_t st) {
  if constexpr ((C::SCHED == 7 || C::SCHED == 8 || C::SCHED == 5) && !C::BLK) {
    constexpr int64_t kLim = (int64_t)1 << 30;
    if (p.kc % C::BK == 0 && p.ldas < kLim && p.ldbs < kLim) return launch_rows_as<C, true>(p, dgrad, num_cus, st);
  }
  return launch_rows_as<C, false>(p, dgrad, num_cus, st);
}

template <class C>
static hipError_t launch_rows_kb(const RowsGemmParams& p, bool dgrad, bool kblk, int num_cus, hipStream_t st) {
  return kblk ? launch_rows<KBlocked<C>>(p, dgrad, num_cus, st) : launch_rows<C>(p, dgrad, num_cus, st);
}

hipError_t launch_grouped_rows_mx(const RowsGemmParams& p, bool a_fp8, bool dgrad, bool mfma_b, bool kblk,
                                  int num_cus, hipStream_t st) {
  if (mfma_b)
    return a_fp8 ? launch_rows_kb<MfmaB<CfgA8>>(p, dgrad, kblk, num_cus, st)
                 : launch_rows_kb<MfmaB<CfgA4>>(p, dgrad, kblk, num_cus, st);
  return a_fp8 ? launch_rows_kb<CfgA8>(p, dgrad, kblk, num_cus, st) : launch_rows_kb<CfgA4>(p, dgrad, kblk, num_cus, st);
}

hipError_t launch_grouped_rows_blk(const RowsGemmParams& p, bool pow2, bool dgrad, int num_cus, hipStream_t st) {
  return pow2 ? launch_rows<CfgP2F>(p, dgrad, num_cus, st) : launch_rows<CfgBlkF>(p, dgrad, num_cus, st);
}

template <class C>
static hipError_t launch_wgrad(const WgradParams& p, int num_cus, hipStream_t st) {
  int64_t tiles = 0;
  const int64_t per = (int64_t)((p.n_rows + C::BM - 1) / C::BM) * ((p.n_cols + C::BN - 1) / C::BN);
  for (int g = 0; g < p.sp.G; ++g) tiles += (p.sp.m[g] > 0 || !p.accumulate) ? per : 0;
  if (tiles == 0) return hipSuccess;
  // fp32 row scales: segments are padded to 128, so with BK dividing 128
  // every stage is full and the fast issue applies
  constexpr bool FAST = C::F32S && !C::BLK && 128 % C::BK == 0;
  if (p.out_bf16) {
    if (p.accumulate) return launch_persistent<C>(grouped_wgrad_kernel<C, FAST, kEpiBf16Acc>, p, tiles, num_cus, st);
    return launch_persistent<C>(grouped_wgrad_kernel<C, FAST, kEpiBf16Set>, p, tiles, num_cus, st);
  }
  if (p.accumulate) return launch_persistent<C>(grouped_wgrad_kernel<C, FAST, kEpiF32Acc>, p, tiles, num_cus, st);
  return launch_persistent<C>(grouped_wgrad_kernel<C, FAST, kEpiF32Set>, p, tiles, num_cus, st);
}

hipError_t launch_grouped_wgrad_mx(const WgradParams& p, bool fp8, int num_cus, hipStream_t st) {
  if (fp8) return launch_wgrad<CfgA8W>(p, num_cus, st);
  return launch_wgrad<CfgA4W>(p, num_cus, st);
}

hipError_t launch_grouped_wgrad_blk(const WgradParams& p, bool pow2, int num_cus, hipStream_t st) {
  if (pow2) return launch_wgrad<CfgP2W>(p, num_cus, st);
  return launch_wgrad<CfgBlkW>(p, num_cus, st);
}

}  // namespace mxgg
