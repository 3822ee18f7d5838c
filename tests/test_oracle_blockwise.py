"""Pins for oracle.blockwise. Power-of-two mode: brute force of the exponent
rule, the amax floor, block sharing, the segment-pad mapping and an exact
blockwise product. The fp32-scale mode (our reading of a step the page leaves
open) is pinned by what the arithmetic fixes: blocks whose amax is a power of
two make every fp32 step exact, so the codes must be the E4M3 round-to-nearest-
even of the exact products (found here by a search over the E4M3 value table)
and the scale the fp32 nearest to 1/q; for any block the amax element lands
on 448 and every element reconstructs within half an E4M3 step of its scaled
value (plus the fp32 rounding of q and x*q)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import blockwise as bw
from oracle import grouped
from oracle.formats import E4M3, bf16_bits_to_f64
from synth import fp32_to_bf16_bits


def _brute_t(amax: float) -> int:
    a = Fraction(max(amax, float(np.float32(1e-4))))
    t = -300
    while a * Fraction(2) ** (t + 1) <= 448:
        t += 1
    return t


def test_pow2_exponent_brute_force():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        [0.0, 1e-9, 1e-4, 448.0, 448.0001, 449.0, 480.0, 512.0, 0.875, 0.8751, 1.0, 3.3e38],
        np.exp(rng.uniform(-20, 80, size=200)),
    ])
    got = bw.pow2_exponent(vals)
    for v, t in zip(vals, got):
        assert int(t) == _brute_t(float(v)), v


def test_zero_block_uses_amax_floor():
    x = np.zeros((2, 128), dtype=np.uint16)
    q, s = bw.quantize_1x128(x)
    assert np.all(q == 0)
    assert np.all(s == np.float32(2.0 ** -22))   # 1e-4 * 2^22 = 419 <= 448 < 838


def test_1x128_max_element_and_rounding():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    xb = fp32_to_bf16_bits(x)
    q, s = bw.quantize_1x128(xb)
    xv = bf16_bits_to_f64(xb)
    for r in range(4):
        for b in range(2):
            blk = xv[r, b * 128:(b + 1) * 128]
            t = _brute_t(float(np.abs(blk).max()))
            assert s[r, b] == np.float32(2.0 ** -t)
            for i in range(128):
                y = Fraction(float(blk[i])) * Fraction(2) ** t
                # nearest E4M3 value, exact, ties to even, all |y| <= 448 here
                best = None
                for c in range(0x7F):
                    v = Fraction(float(E4M3.values[c]))
                    d = abs(abs(y) - v)
                    if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                        best = (d, c)
                code = best[1] | (0x80 if xb[r, b * 128 + i] & 0x8000 else 0)
                assert int(q[r, b * 128 + i]) == code


def test_128x128_shares_one_scale_per_block():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    w[5, 7] = 3.0          # dominates block (0, 0) only
    wb = fp32_to_bf16_bits(w)
    q, s = bw.quantize_128x128(wb)
    assert s.shape == (2, 2)
    assert s[0, 0] == np.float32(2.0 ** -_brute_t(3.0))
    wv = bf16_bits_to_f64(wb)
    for i in range(2):
        for j in range(2):
            blk = wv[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert s[i, j] == np.float32(2.0 ** -_brute_t(float(np.abs(blk).max())))
    d = bw.dequantize_128x128(q, s)
    # relative error of E4M3 (3 mantissa bits) is at most 2^-4 for normal codes
    big = np.abs(wv) > 2.0 ** -6 * s.max()
    assert np.all(np.abs(d - wv)[big] <= np.abs(wv)[big] * 2.0 ** -4)


def test_colwise_segpad_128_mapping():
    rng = np.random.default_rng(4)
    splits = [130, 0, 5]
    x = fp32_to_bf16_bits(rng.standard_normal((sum(splits), 16)).astype(np.float32))
    q, s = bw.quantize_colwise_segpad_128(x, splits)
    assert q.shape == (16, 256 + 128) and s.shape == (16, 3)
    qr, sr = bw.quantize_1x128(x.T.copy()[:, :128])      # expert 0, first block
    assert np.array_equal(q[:, :128], qr) and np.array_equal(s[:, :1], sr)
    # expert 0 second block: 2 real rows then zeros
    blk = np.zeros((16, 128), dtype=np.uint16)
    blk[:, :2] = x[128:130].T
    qb, sb = bw.quantize_1x128(blk)
    assert np.array_equal(q[:, 128:256], qb) and np.array_equal(s[:, 1:2], sb)
    blk = np.zeros((16, 128), dtype=np.uint16)
    blk[:, :5] = x[130:135].T
    qb, sb = bw.quantize_1x128(blk)
    assert np.array_equal(q[:, 256:], qb) and np.array_equal(s[:, 2:], sb)


def test_blockwise_fwd_small_exact():
    rng = np.random.default_rng(6)
    splits = [3, 0, 2]
    G, N, K = 3, 128, 256
    a = fp32_to_bf16_bits(rng.standard_normal((5, K)).astype(np.float32))
    w = fp32_to_bf16_bits((rng.standard_normal((G * N, K)) * 0.02).astype(np.float32))
    aq, as_ = bw.quantize_1x128(a)
    wq, ws = bw.quantize_128x128(w)
    A = bw.dequantize_1x128(aq, as_)
    W = bw.dequantize_128x128(wq, ws).reshape(G, N, K)
    y = grouped.grouped_fwd(A, W, splits)
    # exact reference with fractions for a few outputs
    for (m, g, n) in [(0, 0, 0), (2, 0, 127), (3, 2, 64), (4, 2, 5)]:
        ref = sum(Fraction(float(A[m, k])) * Fraction(float(W[g, n, k])) for k in range(K))
        assert Fraction(float(y[m, n])) == ref


def test_fp32_scale_mode_sanity():
    # parity unpinned: only checks the definition's own consequences
    x = fp32_to_bf16_bits(np.linspace(-3, 3, 128, dtype=np.float32)[None, :])
    q, s = bw.quantize_1x128(x, pow2=False)
    assert int(q[0, -1]) == 0x7E          # amax * (448/amax) = 448 exactly
    assert s[0, 0] == np.float32(1.0) / (np.float32(448.0) / np.float32(3.0))


# ---------------------------------------------------------------------------
# fp32-scale mode pins
# ---------------------------------------------------------------------------
_E4M3_MAGS = [Fraction(float(v)) for v in E4M3.mag_values]   # increasing, code = index


def _e4m3_rne_code(y: Fraction) -> int:
    """Nearest E4M3 magnitude by search, ties to the even code, saturating at
    448; the sign bit from y."""
    a = abs(y)
    if a >= _E4M3_MAGS[-1]:
        c = len(_E4M3_MAGS) - 1
    else:
        hi = next(i for i, v in enumerate(_E4M3_MAGS) if v >= a)
        lo = max(hi - 1, 0)
        dl, dh = a - _E4M3_MAGS[lo], _E4M3_MAGS[hi] - a
        c = lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)
    return c | (0x80 if y < 0 and c else 0)


def _nearest_f32(r: Fraction) -> float:
    """The fp32 nearest to the positive rational r, by comparing neighbours."""
    f = np.float32(float(r))
    best = None
    for cand in (np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - r)
        if best is None or d < best[0]:
            best = (d, cand)
    return float(best[1])


def _bf16_block(rng, amax_exp):
    """128 bf16 values below 2^amax_exp with one element exactly +-2^amax_exp."""
    x = rng.uniform(-1, 1, size=128).astype(np.float32) * np.float32(2.0 ** amax_exp)
    b = fp32_to_bf16_bits(x)
    v = bf16_bits_to_f64(b)
    b[np.abs(v) >= 2.0 ** amax_exp] = fp32_to_bf16_bits(np.float32(0.5 * 2.0 ** amax_exp))
    b[int(rng.integers(0, 128))] = fp32_to_bf16_bits(np.float32((1 if rng.random() < 0.5 else -1) * 2.0 ** amax_exp))
    return b


@pytest.mark.parametrize("amax_exp", [-12, -3, 0, 1, 5, 9, 20])
def test_fp32_mode_power_of_two_amax_is_exact_rne(amax_exp):
    rng = np.random.default_rng(100 + amax_exp)
    b = _bf16_block(rng, amax_exp)
    q, s = bw.quantize_1x128(b[None, :], pow2=False)
    x = bf16_bits_to_f64(b)
    qv = Fraction(448) / Fraction(2) ** amax_exp          # exact in fp32 (7 * 2^k)
    for i in range(128):
        assert int(q[0, i]) == _e4m3_rne_code(Fraction(float(x[i])) * qv), i
    assert float(s[0, 0]) == _nearest_f32(1 / qv)


def test_fp32_mode_amax_to_448_and_half_step_bound():
    rng = np.random.default_rng(7)
    for trial in range(40):
        scale = float(2.0 ** rng.uniform(-20, 20))
        x = fp32_to_bf16_bits((rng.standard_normal(128) * scale).astype(np.float32))
        q, s = bw.quantize_1x128(x[None, :], pow2=False)
        xv = bf16_bits_to_f64(x)
        codes = q[0].astype(np.int64)
        i = int(np.argmax(np.abs(xv)))
        floor = Fraction(float(bw.AMAX_FLOOR))
        amax = max(Fraction(float(np.abs(xv).max())), floor)
        if amax > floor:
            assert codes[i] & 0x7F == 0x7E                   # the amax element lands on 448
        assert np.all(codes & 0x7F <= 0x7E)                  # nothing beyond 448, no NaN code
        sf = Fraction(float(s[0, 0]))
        for k in range(128):
            y = Fraction(float(xv[k])) * 448 / amax             # exact scaled value
            c = int(codes[k]) & 0x7F
            lo = _E4M3_MAGS[max(c - 1, 0)]
            hi = _E4M3_MAGS[min(c + 1, len(_E4M3_MAGS) - 1)]
            half_step = max(_E4M3_MAGS[c] - lo, hi - _E4M3_MAGS[c]) / 2
            err = abs(Fraction(float(E4M3.values[int(codes[k])])) * sf - Fraction(float(xv[k])))
            # half an E4M3 step of the scaled value, plus the fp32 roundings of q,
            # x*q and 1/q (three relative 2^-24 terms of the scaled value)
            bound = (half_step + 3 * abs(y) / 2 ** 23) * sf * (1 + Fraction(1, 2 ** 20))
            assert err <= bound, (trial, k)


# ---------------------------------------------------------------------------
# dequantization pins ("Add ROCm Triton blockwise FP8 grouped GEMM": 1x128
# activation scales along K, 128x128 weight blocks; dequantized = code * s)
# ---------------------------------------------------------------------------
def _e4m3_by_fields(code: int) -> Fraction:
    """E4M3 "FN" value from its bit fields (sign, 4-bit exponent with bias 7,
    3-bit mantissa; exponent field 0 is subnormal), written out here rather
    than read from the oracle's table."""
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _finite_e4m3_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01          # the two NaN codes become 448-adjacent finite ones
    return c


def test_dequantize_1x128_each_element_is_code_times_its_row_block_scale():
    rng = np.random.default_rng(21)
    R, C = 3, 384
    codes = _finite_e4m3_codes(rng, (R, C))
    # every (row, block) scale distinct, powers of two and general fp32
    scales = np.array([[2.0 ** -7, 3.0, 0.15625], [1.7e-3, 2.0 ** 5, 0.9],
                       [6.5e4, 2.0 ** -20, 1.1]], dtype=np.float32)
    d = bw.dequantize_1x128(codes, scales)
    assert d.shape == (R, C)
    for r in range(R):
        for c in range(C):
            ref = _e4m3_by_fields(int(codes[r, c])) * Fraction(float(scales[r, c // 128]))
            # a 4-bit significand times a 24-bit one: exact in fp64
            assert Fraction(float(d[r, c])) == ref, (r, c)


def test_dequantize_128x128_each_element_uses_its_block_scale():
    rng = np.random.default_rng(22)
    codes = _finite_e4m3_codes(rng, (256, 384))
    scales = np.array([[2.0 ** -3, 5.0, 0.3], [7.0, 2.0 ** 9, 1e-3]], dtype=np.float32)
    d = bw.dequantize_128x128(codes, scales)
    for (r, c) in [(0, 0), (127, 127), (128, 0), (0, 128), (255, 383), (129, 260), (17, 300), (200, 131)]:
        ref = _e4m3_by_fields(int(codes[r, c])) * Fraction(float(scales[r // 128, c // 128]))
        assert Fraction(float(d[r, c])) == ref, (r, c)


@pytest.mark.parametrize("t", [-20, -5, 0, 3, 17])
def test_dequantize_1x128_round_trip_is_exact_on_the_scaled_e4m3_grid(t):
    # x = E4M3 value * 2^-t with one element at 448 * 2^-t: the block's
    # power-of-two exponent is t, every x * 2^t is an E4M3 value, so
    # quantize-then-dequantize must give x back bit for bit
    rng = np.random.default_rng(300 + t)
    codes = _finite_e4m3_codes(rng, (2, 256))
    codes[(codes & 0x7F) == 0x7E] -= 1                      # at most one amax element per block
    codes[0, 5], codes[1, 200] = 0x7E, 0xFE               # +448 in block 0 of row 0, -448 in block 1 of row 1
    codes[0, 130], codes[1, 64] = 0x7E, 0xFE
    x = np.array([[float(_e4m3_by_fields(int(c)) * Fraction(2) ** -t) for c in row] for row in codes])
    xb = fp32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(xb), x)        # 4-bit significands fit bf16
    q, s = bw.quantize_1x128(xb)
    assert np.all(s == np.float32(2.0 ** -t))
    assert np.array_equal(bw.dequantize_1x128(q, s), x)


def test_dequantize_1x128_reconstructs_within_half_an_e4m3_step():
    rng = np.random.default_rng(23)
    xb = fp32_to_bf16_bits((rng.standard_normal((4, 512)) * np.float32(2.0 ** 7)).astype(np.float32))
    q, s = bw.quantize_1x128(xb)
    d = bw.dequantize_1x128(q, s)
    x = bf16_bits_to_f64(xb)
    for r in range(4):
        for c in range(512):
            sc = Fraction(float(s[r, c // 128]))
            mag = int(q[r, c]) & 0x7F
            lo = _E4M3_MAGS[max(mag - 1, 0)]
            hi = _E4M3_MAGS[min(mag + 1, len(_E4M3_MAGS) - 1)]
            half_step = max(_E4M3_MAGS[mag] - lo, hi - _E4M3_MAGS[mag]) / 2
            assert abs(Fraction(float(d[r, c])) - Fraction(float(x[r, c]))) <= half_step * sc, (r, c)
