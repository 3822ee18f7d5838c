"""Pins for oracle.blockwise (power-of-two mode); the fp32-scale mode is our own
reading and is only sanity-checked here (parity unpinned)."""
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
