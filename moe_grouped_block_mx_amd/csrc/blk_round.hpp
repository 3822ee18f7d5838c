// Blockwise FP8 (E4M3, fp32 scale per 128-element block) scale rules and the
// fp32 -> E4M3 encoder ("Add ROCm Triton blockwise FP8 grouped GEMM": 1x128
// activation blocks, 128x128 weight blocks, power-of-two scales by default,
// block amax floored at 1e-4).
//
//   amax' = max(amax, fp32(1e-4))
//   power-of-two mode: t = largest integer with amax' * 2^t <= 448; codes =
//     RNE(x * 2^t) (exact product, never above 448); stored scale s = 2^-t.
//   fp32 mode: q = fp32(448 / amax'); codes = RNE-saturating E4M3 of
//     fp32(x * q); s = fp32(1 / q).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxgg {

constexpr uint32_t kBlkAmaxFloorBits = 0x38D1B717u;  // fp32 nearest to 1e-4

// amax' as fp32 bits from the bf16 bits of the block's largest magnitude (a
// bf16 value is exact in fp32, so the comparison is exact on the bits).
__host__ __device__ __forceinline__ uint32_t blk_amax_floored_bits(uint32_t amax_bf16_mag) {
  const uint32_t a = amax_bf16_mag << 16;
  return a > kBlkAmaxFloorBits ? a : kBlkAmaxFloorBits;
}

// t of the power-of-two mode. amax' = 1.m * 2^(fe-127) is a normal fp32;
// amax' * 2^t <= 448 = 1.75 * 2^8 holds for t = 135 - fe when 1.m <= 1.75
// (mantissa bits <= 0x600000), else for one less.
__host__ __device__ __forceinline__ int blk_pow2_t(uint32_t amaxp_bits) {
  const int fe = (int)(amaxp_bits >> 23);
  return (amaxp_bits & 0x7fffffu) <= 0x600000u ? 135 - fe : 134 - fe;
}

// fp32 bits of 2^-t (t in [-120, 22] for finite bf16 inputs: a normal fp32).
__host__ __device__ __forceinline__ uint32_t blk_pow2_scale_bits(int t) { return (uint32_t)(127 - t) << 23; }

// Round-to-nearest-even of v >> sh (0 <= sh < 32).
__host__ __device__ __forceinline__ uint32_t rne_shift(uint32_t v, int sh) {
  if (sh == 0) return v;
  const uint32_t half = 1u << (sh - 1);
  return (v + half - 1u + ((v >> sh) & 1u)) >> sh;
}

// fp32 -> E4M3 ("FN": bias 7, no infinities, max 448 = 0x7E), round to nearest
// even, saturating, sign kept. Finite inputs only.
__host__ __device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(uint32_t bits) {
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7fffffffu;
  const int fe = (int)(mag >> 23);
  if (fe == 0) return sign;  // zero or fp32 subnormal: far below half of 2^-9
  const uint32_t m24 = (mag & 0x7fffffu) | 0x800000u;  // 1.m as a 24-bit integer
  const int ex = fe - 127;
  uint32_t code;
  if (ex >= -6) {
    // normal binade: 3 mantissa bits; a carry out of the mantissa moves the
    // code to the next binade, which the code arithmetic does by itself
    const uint32_t m = rne_shift(m24, 20);  // in [8, 16]
    code = ((uint32_t)(ex + 7) << 3) + (m - 8u);
    if (ex > 8) code = 0x7Eu;
  } else {
    // subnormal E4M3: value = code * 2^-9, code = RNE(1.m * 2^(ex + 9))
    const int sh = 14 - ex;  // >= 21
    code = sh >= 32 ? 0u : rne_shift(m24, sh);
  }
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

}  // namespace mxgg
