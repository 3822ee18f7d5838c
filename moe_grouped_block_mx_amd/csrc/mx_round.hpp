// MX shared exponent and the operands of the hardware element conversion.
//
// The MX rule (OCP Microscaling v1.0; the tiny-scale clamp from the review
// thread on the page "route te.GroupedLinear through #723; a8w4 fwd-only"):
// shared exponent e = clamp(floor(log2 amax) - emax, -127, 127), e = -127 for
// an all-zero block; element code = round-to-nearest-even of |x| * 2^-e onto
// the element grid, saturated at the largest finite magnitude; sign copied.
//
// The shared exponent is computed exactly from the bf16 bits of amax. The
// elements are encoded by gfx950's v_cvt_scalef32_pk_{fp4,fp8}_bf16, which were
// checked against the rule on every finite bf16 pattern at every shared
// exponent: E2M1 matches exactly; E4M3 matches except that scaled magnitudes
// >= 464 become NaN instead of 448, which the clamp below removes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxgg {

// Element formats: mantissa bits, exponent of the smallest normal, largest
// finite magnitude code, exponent of the largest normal binade, sign bit.
struct E2M1Fmt { static constexpr int MB = 1, EMIN = 0, MAXC = 0x7, EMAX = 2, SIGN = 0x8; };
struct E4M3Fmt { static constexpr int MB = 3, EMIN = -6, MAXC = 0x7E, EMAX = 8, SIGN = 0x80; };

// floor(log2 |x|) of a nonzero bf16 magnitude (sign bit clear).
__host__ __device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
  const uint32_t E = mag >> 7;
  if (E) return (int)E - 127;
  return (31 - __builtin_clz(mag & 0x7fu)) - 133;  // subnormal: 0.m * 2^-126
}

// Shared exponent of a block from the bf16 bits of its largest magnitude.
template <class F>
__host__ __device__ __forceinline__ int mx_shared_exp(uint32_t amax_mag) {
  if (amax_mag == 0) return -127;
  int e = bf16_floor_log2(amax_mag) - F::EMAX;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// fp32 operand of the gfx950 scaled conversions: the UE8M0 scale 2^e carried
// in the exponent field (e = -127 is exponent field 0, which the conversion
// reads as 2^-127, not as a flushed denormal).
__host__ __device__ __forceinline__ uint32_t mx_scale_operand_bits(int e) { return (uint32_t)(e + 127) << 23; }

// bf16 bits of 448 * 2^e, the largest E4M3 magnitude at shared exponent e.
// The hardware E4M3 conversion rounds magnitudes at or above 464 (after
// scaling) to NaN instead of saturating, so inputs are first clamped to this
// value; below it round-to-nearest-even already gives 448, so the clamp only
// implements saturation. For e > 119 the bound exceeds every finite bf16.
__host__ __device__ __forceinline__ uint32_t e4m3_sat_limit_bits(int e) {
  return e > 119 ? 0x7f7fu : ((uint32_t)(e + 135) << 7) | 0x60u;
}

// Clamp both bf16 magnitudes of a packed pair to `limit` (sign kept).
__host__ __device__ __forceinline__ uint32_t clamp_bf16x2_mag(uint32_t w, uint32_t limit) {
  uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
  lo = lo < limit ? lo : limit;
  hi = hi < limit ? hi : limit;
  return (w & 0x80008000u) | lo | (hi << 16);
}

}  // namespace mxgg
