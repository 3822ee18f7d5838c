// MX element encoding on bf16 bit patterns, in integer arithmetic.
//
// The MX rule (OCP Microscaling v1.0; the tiny-scale clamp from the review
// thread on the page "route te.GroupedLinear through #723; a8w4 fwd-only"):
// shared exponent e = clamp(floor(log2 amax) - emax, -127, 127), e = -127 for
// an all-zero block; element code = round-to-nearest-even of |x| * 2^-e onto
// the element grid, saturated at the largest finite magnitude; sign copied.
//
// Everything below works on integers, so the result does not depend on the
// floating-point modes of the hardware (denormal flushing, conversion
// rounding): a bf16 magnitude is sig * 2^ex with an integer significand, the
// scaled value's binade L gives the grid quantum 2^Q, and the code is the
// rounded multiple of that quantum laid out as (binade, mantissa) bits.
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

// Magnitude code (no sign) of the bf16 magnitude `mag` scaled by 2^-e.
template <class F>
__host__ __device__ __forceinline__ uint32_t mx_encode_mag(uint32_t mag, int e) {
  if (mag == 0) return 0;
  const uint32_t E = mag >> 7;
  const int sig = E ? (int)(0x80u | (mag & 0x7fu)) : (int)(mag & 0x7fu);
  const int ex = E ? (int)E - 134 : -133;          // |x| = sig * 2^ex
  const int L = (31 - __builtin_clz((uint32_t)sig)) + ex - e;         // floor(log2(|x| 2^-e))
  const int Q = (L > F::EMIN ? L : F::EMIN) - F::MB;  // grid quantum exponent
  const int sh = ex - e - Q;                        // n = sig * 2^sh
  uint32_t n;
  if (sh >= 0) {
    n = (uint32_t)sig << sh;                        // exact (small values only)
  } else {
    int r = -sh;
    r = r > 31 ? 31 : r;
    const uint32_t us = (uint32_t)sig;
    const uint32_t q = us >> r;
    const uint32_t rem = us & ((1u << r) - 1u);
    const uint32_t half = 1u << (r - 1);
    n = q + ((rem > half) | ((rem == half) & (q & 1u)));
  }
  // grid position -> code: binade index above the subnormal binade, plus n
  uint32_t code = ((uint32_t)(Q - (F::EMIN - F::MB)) << F::MB) + n;
  return code > (uint32_t)F::MAXC ? (uint32_t)F::MAXC : code;
}

template <class F>
__host__ __device__ __forceinline__ uint32_t mx_encode(uint32_t bits, int e) {
  const uint32_t sign = (bits & 0x8000u) ? (uint32_t)F::SIGN : 0u;
  return sign | mx_encode_mag<F>(bits & 0x7fffu, e);
}

}  // namespace mxgg
