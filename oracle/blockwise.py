"""DeepSeek-style blockwise FP8 (E4M3) quantization, in fp64 / fp32.

Test infrastructure only (see the package docstring).

Source: "Add ROCm Triton blockwise FP8 grouped GEMM" -- activations are
quantized 1x128 along K, weights in 128x128 blocks, and the wgrad operands
1x128 along M per expert segment padded to 128 (the segment-padded column-wise
operand); the recipe uses power-of-two scales by default (the review thread on
threading the recipe's power-of-two flag into the Triton launchers); the
kernels floor each block's amax at 1e-4 (the NUM_XCDS / amax-clamp commit
notes).

Readings taken where the page gives no formula:

* the amax floor is the fp32 value nearest 1e-4, since the kernels work in
  fp32;
* power-of-two mode: the stored scale is s = 2^-t with t the largest integer
  such that amax' * 2^t <= 448 (no element overflows before saturation);
  codes = RNE-saturating E4M3 of x * 2^t (exact);
* fp32 mode (flag off): q = fp32(448 / amax'), codes = RNE-saturating E4M3 of
  fp32(x * q), s = fp32(1 / q). This mode is our own reading; its pins are
  what the arithmetic fixes (power-of-two amax makes every step exact; the
  amax element lands on 448; half-step reconstruction bound), see
  tests/test_oracle_blockwise.py. Whether the product x * q is rounded to
  fp32 (as the kernels do) is not distinguishable by those pins.

Dequantized value = value(code) * s. The grouped products reuse
``oracle.grouped`` on the dequantized operands (segment pad 128).
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3, bf16_bits_to_f64
from .mx import round_to_format, segpad_offsets

BLK = 128
AMAX_FLOOR = float(np.float32(1e-4))

__all__ = [
    "BLK", "AMAX_FLOOR", "pow2_exponent", "quantize_1x128", "quantize_128x128",
    "quantize_colwise_segpad_128", "dequantize_1x128", "dequantize_128x128",
]


def pow2_exponent(amax: np.ndarray) -> np.ndarray:
    """t = max { integer t : max(amax, floor) * 2^t <= 448 }."""
    a = np.maximum(np.asarray(amax, dtype=np.float64), AMAX_FLOOR)
    _, E = np.frexp(a)                    # a = f * 2^E, f in [0.5, 1)
    t0 = 9 - E.astype(np.int64)           # a * 2^t0 = f * 512 < 512
    fits = np.ldexp(a, t0) <= E4M3.max_value
    return np.where(fits, t0, t0 - 1).astype(np.int64)


def _quant_groups(xb: np.ndarray, amax: np.ndarray, pow2: bool):
    """xb: values with a trailing block axis; amax broadcastable to xb."""
    if pow2:
        t = pow2_exponent(amax)
        y = np.ldexp(xb, t)
        s = np.ldexp(1.0, -t).astype(np.float32)
    else:
        a = np.maximum(amax, AMAX_FLOOR).astype(np.float32)
        q = (np.float32(448.0) / a).astype(np.float32)
        y = (xb.astype(np.float32) * q).astype(np.float32).astype(np.float64)
        s = (np.float32(1.0) / q).astype(np.float32)
    return round_to_format(y, E4M3), s


def quantize_1x128(x_bits: np.ndarray, pow2: bool = True):
    """bf16 [R, C] -> E4M3 codes [R, C] and fp32 scales [R, C/128]."""
    x = bf16_bits_to_f64(x_bits)
    R, C = x.shape
    if C % BLK:
        raise ValueError("cols must be a multiple of 128")
    xb = x.reshape(R, C // BLK, BLK)
    amax = np.max(np.abs(xb), axis=-1, keepdims=True)
    codes, s = _quant_groups(xb, amax, pow2)
    return codes.reshape(R, C), s.reshape(R, C // BLK)


def quantize_128x128(w_bits: np.ndarray, pow2: bool = True):
    """bf16 [R, C] (R, C multiples of 128) -> codes [R, C], scales [R/128, C/128]."""
    w = bf16_bits_to_f64(w_bits)
    R, C = w.shape
    if R % BLK or C % BLK:
        raise ValueError("rows and cols must be multiples of 128")
    wb = w.reshape(R // BLK, BLK, C // BLK, BLK)
    amax = np.max(np.abs(wb), axis=(1, 3), keepdims=True)
    codes, s = _quant_groups(wb, amax, pow2)
    return codes.reshape(R, C), s.reshape(R // BLK, C // BLK)


def quantize_colwise_segpad_128(x_bits: np.ndarray, m_splits, pow2: bool = True):
    """bf16 [R, C] -> codes [C, Mpad] and scales [C, Mpad/128], segments of
    each expert transposed and zero-padded to a multiple of 128."""
    x = bf16_bits_to_f64(x_bits)
    R, C = x.shape
    row_offs, pad_offs = segpad_offsets(m_splits, BLK)
    if row_offs[-1] != R:
        raise ValueError("sum(m_splits) != rows")
    mpad = int(pad_offs[-1])
    xt = np.zeros((C, mpad), dtype=np.float64)
    for g in range(len(row_offs) - 1):
        r0, r1 = row_offs[g], row_offs[g + 1]
        xt[:, pad_offs[g]:pad_offs[g] + (r1 - r0)] = x[r0:r1].T
    xb = xt.reshape(C, mpad // BLK, BLK)
    amax = np.max(np.abs(xb), axis=-1, keepdims=True)
    codes, s = _quant_groups(xb, amax, pow2)
    return codes.reshape(C, mpad), s.reshape(C, mpad // BLK)


def dequantize_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = E4M3.values[np.asarray(codes, dtype=np.uint8)]
    return vals * np.repeat(np.asarray(scales, dtype=np.float64), BLK, axis=-1)


def dequantize_128x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    vals = E4M3.values[np.asarray(codes, dtype=np.uint8)]
    s = np.asarray(scales, dtype=np.float64)
    s_full = np.repeat(np.repeat(s, BLK, axis=0), BLK, axis=1)
    return vals * s_full
