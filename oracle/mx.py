"""MX (block-32, UE8M0-scaled) quantization and dequantization, in fp64.

Test infrastructure only (see the package docstring).

The rule (OCP Microscaling v1.0, section "Conversion from vectors of scalar
floats", which is the rule the grouped MXFP4 / a8w4 pages rely on):

* a block is 32 consecutive elements along the contraction axis;
* amax = max |x_i| over the block;
* shared exponent e = floor(log2 amax) - emax_elem, with emax_elem = 2 for
  E2M1 and 8 for E4M3; the exponent is clamped to [-127, 127] (the clamp at
  -127 and "rescale first" behaviour follow the review thread on tiny block
  scales on the page "route te.GroupedLinear through #723; a8w4 fwd-only");
  an all-zero block takes e = -127 (our reading of the zero-block case that
  thread leaves open: the formula's own limit);
* each element is scaled by 2^-e (exact) and rounded to the nearest value of
  the element format, ties to the even code, saturating at +-6 (E2M1) or
  +-448 (E4M3); the sign bit is kept, so a negative input that rounds to zero
  gives negative zero;
* the stored scale byte is e + 127.

Row-wise layout ("Triton mxfp4 (and a8w4) grouped GEMM kernel", row operand):
data u8[rows, cols/2] for E2M1 (element 2j in bits 3:0 of byte j, element
2j+1 in bits 7:4) or u8[rows, cols] for E4M3, scales u8[rows, cols/32].

Column-wise segment-padded layout (same page, the padded column operand used by
the variable-K weight gradient): the rows of each expert segment are
transposed, blocks of 32 start at the segment start, rows past the segment end
inside the last block are zeros; output data u8[cols, Mpad/2] (E2M1) or
u8[cols, Mpad], scales u8[cols, Mpad/32], Mpad = sum_g ceil(m_g/32)*32.
"""
from __future__ import annotations

import numpy as np

from .formats import FORMATS, MiniFloat, bf16_bits_to_f64

BLOCK = 32

__all__ = [
    "BLOCK", "shared_exponent", "round_to_format", "quantize_blocks",
    "quantize_rowwise", "dequantize_rowwise", "pack_codes", "unpack_codes",
    "segpad_offsets", "quantize_colwise_segpad", "dequantize_colwise_segpad",
]


def _fmt(fmt) -> MiniFloat:
    return FORMATS[fmt] if isinstance(fmt, str) else fmt


def shared_exponent(amax: np.ndarray, f: MiniFloat) -> np.ndarray:
    """e = clamp(floor(log2 amax) - emax, -127, 127); e = -127 when amax == 0.

    floor(log2 a) is taken exactly from the binary exponent: frexp writes
    a = m * 2^E with m in [0.5, 1), so floor(log2 a) = E - 1.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)
    e = np.clip(E.astype(np.int64) - 1 - f.emax, -127, 127)
    return np.where(amax == 0.0, -127, e).astype(np.int64)


def round_to_format(y: np.ndarray, f: MiniFloat) -> np.ndarray:
    """Element codes: nearest finite value of ``f``, ties to the even code,
    saturating at the largest finite magnitude; sign bit copied from ``y``."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("non-finite input to the MX oracle")
    mags = f.mag_values                      # ascending, index == magnitude code
    a = np.abs(y)
    hi = np.searchsorted(mags, a, side="left")   # first magnitude >= a
    hi = np.minimum(hi, len(mags) - 1)           # beyond the max: saturate
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    # nearest; on an exact tie take the even magnitude code
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    # a value at or above the largest magnitude maps to it
    code = np.where(a >= mags[-1], len(mags) - 1, code).astype(np.int64)
    sign = np.signbit(y).astype(np.int64)
    return (code | (sign * f.sign_bit)).astype(np.uint8)


def quantize_blocks(x: np.ndarray, f: MiniFloat):
    """Quantize fp64 values whose last axis holds whole 32-element blocks.

    Returns (codes uint8 with the shape of x, scale bytes uint8 with the last
    axis divided by 32).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (x.shape[-1] // BLOCK, BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    e = shared_exponent(amax, f)
    y = np.ldexp(xb, -e[..., None])               # exact: power-of-two scaling
    codes = round_to_format(y, f).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def pack_codes(codes: np.ndarray, f: MiniFloat) -> np.ndarray:
    """E2M1: two codes per byte, even element in the low nibble. E4M3: as is."""
    codes = np.asarray(codes, dtype=np.uint8)
    if f.nbits == 8:
        return codes
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_codes(q: np.ndarray, f: MiniFloat) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8)
    if f.nbits == 8:
        return q
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def quantize_rowwise(x_bits: np.ndarray, fmt):
    """Row-wise MX quantization of a bf16 [rows, cols] matrix along cols.

    Returns (data, scales) in the row-wise layout of the module docstring.
    """
    f = _fmt(fmt)
    x = bf16_bits_to_f64(x_bits)
    if x.ndim != 2:
        raise ValueError("expects a 2-D matrix")
    codes, scales = quantize_blocks(x, f)
    return pack_codes(codes, f), scales


def dequantize_rowwise(q: np.ndarray, scales: np.ndarray, fmt) -> np.ndarray:
    """v = value(code) * 2^(byte-127), as fp64 [rows, cols]."""
    f = _fmt(fmt)
    codes = unpack_codes(q, f)
    vals = f.values[codes]
    e = np.asarray(scales, dtype=np.int64) - 127
    e_full = np.repeat(e, BLOCK, axis=-1)
    return np.ldexp(vals, e_full)


def segpad_offsets(m_splits, pad: int = BLOCK):
    """Row offsets (length G+1) and padded offsets (each segment rounded up to
    a multiple of ``pad``)."""
    m = np.asarray(m_splits, dtype=np.int64)
    if np.any(m < 0):
        raise ValueError("negative split")
    row_offs = np.concatenate([[0], np.cumsum(m)])
    padded = -(-m // pad) * pad
    pad_offs = np.concatenate([[0], np.cumsum(padded)])
    return row_offs, pad_offs


def quantize_colwise_segpad(x_bits: np.ndarray, m_splits, fmt, pad: int = BLOCK):
    """Column-wise MX quantization of bf16 [rows, cols] per expert segment.

    For expert g, rows [row_offs[g], row_offs[g+1]) are transposed into
    columns [pad_offs[g], pad_offs[g] + m_g) of a [cols, Mpad] matrix whose
    remaining columns in the segment are zero; that matrix is then quantized
    along its rows in blocks of 32 (``pad`` is a multiple of 32, so no block
    crosses a segment boundary).
    """
    f = _fmt(fmt)
    if pad % BLOCK:
        raise ValueError("pad must be a multiple of 32")
    x = bf16_bits_to_f64(x_bits)
    rows, cols = x.shape
    row_offs, pad_offs = segpad_offsets(m_splits, pad)
    if row_offs[-1] != rows:
        raise ValueError("sum(m_splits) != rows")
    mpad = int(pad_offs[-1])
    xt = np.zeros((cols, mpad), dtype=np.float64)
    for g in range(len(row_offs) - 1):
        r0, r1 = row_offs[g], row_offs[g + 1]
        p0 = pad_offs[g]
        xt[:, p0:p0 + (r1 - r0)] = x[r0:r1, :].T
    codes, scales = quantize_blocks(xt, f)
    return pack_codes(codes, f), scales


def dequantize_colwise_segpad(q: np.ndarray, scales: np.ndarray, fmt) -> np.ndarray:
    """fp64 [cols, Mpad] (the padded, transposed operand)."""
    return dequantize_rowwise(q, scales, fmt)
