"""Element and scale formats, built from their bit-field definitions.

Test infrastructure only (see the package docstring).

Sources: the OCP Microscaling Formats (MX) v1.0 specification (E2M1 element,
UE8M0 scale, block size 32) and the OCP 8-bit Floating Point specification
(E4M3 "FN" variant: bias 7, no infinities, S.1111.111 is NaN, largest finite
magnitude 448). The pages name these formats -- "Integrate MXFP4 hipblaslt GEMM
support" (E2M1 data with UE8M0 block-32 scales) and "route te.GroupedLinear
through #723; a8w4 fwd-only" (E4M3 elements, 448 as the largest value in the
tiny-scale review thread) -- but print no table, so the tables here are
generated from the definitions and pinned in tests against the values the
specifications list.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "E2M1", "E4M3", "FORMATS", "MiniFloat",
    "bf16_bits_to_f64", "ue8m0_to_f64",
]


class MiniFloat:
    """A sign / exponent / mantissa format with subnormals and no infinities.

    ``values[c]`` is the real value of code ``c`` (NaN for NaN codes).
    ``emax`` is the exponent of the largest normal binade, used by the MX
    shared-exponent rule.
    """

    def __init__(self, name: str, ebits: int, mbits: int, bias: int,
                 nan_codes: tuple[int, ...]):
        self.name = name
        self.ebits = ebits
        self.mbits = mbits
        self.bias = bias
        self.nbits = 1 + ebits + mbits
        self.sign_bit = 1 << (ebits + mbits)
        ncodes = 1 << self.nbits
        vals = np.empty(ncodes, dtype=np.float64)
        for c in range(ncodes):
            sign = -1.0 if c & self.sign_bit else 1.0
            e = (c >> mbits) & ((1 << ebits) - 1)
            m = c & ((1 << mbits) - 1)
            if e == 0:  # subnormal: 0.m * 2^(1-bias)
                mag = (m / (1 << mbits)) * 2.0 ** (1 - bias)
            else:       # normal: 1.m * 2^(e-bias)
                mag = (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)
            vals[c] = sign * mag
        for c in nan_codes:
            vals[c] = np.nan
        self.values = vals
        # Non-negative finite magnitudes, indexed by the magnitude code
        # (the code with the sign bit clear). Codes are increasing in value.
        pos = vals[: self.sign_bit]
        finite = np.isfinite(pos)
        self.mag_values = pos[finite].copy()
        self.max_mag_code = int(np.flatnonzero(finite)[-1])
        self.max_value = float(pos[self.max_mag_code])
        # exponent of the largest normal binade
        self.emax = int(np.floor(np.log2(self.max_value)))

    def __repr__(self) -> str:
        return f"MiniFloat({self.name})"


# E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; all 16 codes finite.
E2M1 = MiniFloat("e2m1", ebits=2, mbits=1, bias=1, nan_codes=())
# E4M3 (OCP "FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; only
# S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
E4M3 = MiniFloat("e4m3", ebits=4, mbits=3, bias=7, nan_codes=(0x7F, 0xFF))

FORMATS = {"mxfp4": E2M1, "mxfp8": E4M3}


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64.

    A bf16 pattern is the upper half of the fp32 pattern with the same value,
    so widening the bits and reinterpreting is exact, subnormals included.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ue8m0_to_f64(byte: np.ndarray) -> np.ndarray:
    """UE8M0 scale value 2^(b-127); 0xFF is NaN."""
    b = np.asarray(byte, dtype=np.int64)
    out = np.ldexp(1.0, b - 127).astype(np.float64)
    return np.where(b == 0xFF, np.nan, out)
