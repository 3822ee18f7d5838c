"""Pins for oracle.grouped: exact brute force with fractions on tiny shapes,
reductions to dense products, and the accumulate / empty-expert rules."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import grouped, mx
from oracle.formats import bf16_bits_to_f64
from synth import fp32_to_bf16_bits

E2M1_MAG = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
            Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _e4m3_frac(c):
    s = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 0xF, c & 7
    if e == 0:
        return s * Fraction(m, 8) / 64
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _deq_fraction(q, s, fmt):
    """Dequantize a row-wise operand to a list-of-lists of Fractions."""
    rows = q.shape[0]
    cols = q.shape[1] * (2 if fmt == "mxfp4" else 1)
    out = []
    for r in range(rows):
        row = []
        for c in range(cols):
            if fmt == "mxfp4":
                byte = int(q[r, c // 2])
                code = (byte >> 4) if c % 2 else (byte & 0xF)
                v = E2M1_MAG[code & 7] * (-1 if code & 8 else 1)
            else:
                v = _e4m3_frac(int(q[r, c]))
            row.append(v * Fraction(2) ** (int(s[r, c // 32]) - 127))
        out.append(row)
    return out


def _inputs(rng, shape, std=1.0):
    return fp32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


@pytest.mark.parametrize("afmt", ["mxfp4", "mxfp8"])
def test_fwd_brute_force(afmt):
    rng = np.random.default_rng(11)
    splits = [3, 0, 8, 5]
    G, K, N = 4, 64, 6
    M = sum(splits)
    a = _inputs(rng, (M, K))
    w = _inputs(rng, (G * N, K), 0.3)
    aq, as_ = mx.quantize_rowwise(a, afmt)
    wq, ws = mx.quantize_rowwise(w, "mxfp4")
    A = _deq_fraction(aq, as_, afmt)
    W = _deq_fraction(wq, ws, "mxfp4")
    got = grouped.grouped_fwd(mx.dequantize_rowwise(aq, as_, afmt),
                              mx.dequantize_rowwise(wq, ws, "mxfp4").reshape(G, N, K),
                              splits)
    r = 0
    for g, m in enumerate(splits):
        for i in range(m):
            for n in range(N):
                ref = sum(A[r + i][k] * W[g * N + n][k] for k in range(K))
                assert Fraction(got[r + i, n]) == ref
        r += m


def test_dgrad_brute_force():
    rng = np.random.default_rng(12)
    splits = [5, 2, 0]
    G, K, N = 3, 32, 64           # contraction over N
    M = sum(splits)
    dy = _inputs(rng, (M, N))
    w = _inputs(rng, (G * N, K), 0.3)
    dyq, dys = mx.quantize_rowwise(dy, "mxfp4")
    # W quantized along N: column-wise segment-padded with splits [N]*G
    wcq, wcs = mx.quantize_colwise_segpad(w, [N] * G, "mxfp4")
    assert wcq.shape == (K, G * N // 2)
    DY = _deq_fraction(dyq, dys, "mxfp4")
    WC = _deq_fraction(wcq, wcs, "mxfp4")      # [K][G*N]
    got = grouped.grouped_dgrad(mx.dequantize_rowwise(dyq, dys, "mxfp4"),
                                mx.dequantize_rowwise(wcq, wcs, "mxfp4"), splits)
    r = 0
    for g, m in enumerate(splits):
        for i in range(m):
            for k in range(K):
                ref = sum(DY[r + i][n] * WC[k][g * N + n] for n in range(N))
                assert Fraction(got[r + i, k]) == ref
        r += m


@pytest.mark.parametrize("accumulate", [False, True])
def test_wgrad_brute_force(accumulate):
    rng = np.random.default_rng(13)
    splits = [9, 0, 33, 4]
    G, N, K = 4, 3, 10
    M = sum(splits)
    dy = _inputs(rng, (M, N))
    x = _inputs(rng, (M, K))
    dq, ds = mx.quantize_colwise_segpad(dy, splits, "mxfp4")
    xq, xs = mx.quantize_colwise_segpad(x, splits, "mxfp4")
    DY = _deq_fraction(dq, ds, "mxfp4")   # [N][Mpad]
    X = _deq_fraction(xq, xs, "mxfp4")    # [K][Mpad]
    main0 = rng.standard_normal((G, N, K)).astype(np.float32)
    got = grouped.grouped_wgrad(mx.dequantize_rowwise(dq, ds, "mxfp4"),
                                mx.dequantize_rowwise(xq, xs, "mxfp4"), splits,
                                main_grad0=main0.astype(np.float64), accumulate=accumulate)
    p0 = 0
    for g, m in enumerate(splits):
        mp = -(-m // 32) * 32
        for n in range(N):
            for k in range(K):
                ref = sum(DY[n][p0 + t] * X[k][p0 + t] for t in range(mp))
                if accumulate:
                    ref += Fraction(float(main0[g, n, k]))
                assert Fraction(got[g, n, k]) == ref, (g, n, k)
        p0 += mp


def test_grouped_equals_concatenated_dense_and_G1():
    rng = np.random.default_rng(14)
    splits = [0, 17, 0, 40, 1]
    K, N = 64, 16
    a = rng.standard_normal((sum(splits), K))
    w = rng.standard_normal((len(splits), N, K))
    y = grouped.grouped_fwd(a, w, splits)
    off = np.concatenate([[0], np.cumsum(splits)])
    for g in range(len(splits)):
        np.testing.assert_array_equal(y[off[g]:off[g + 1]], a[off[g]:off[g + 1]] @ w[g].T)
    y1 = grouped.grouped_fwd(a, w[1:2], [sum(splits)])
    np.testing.assert_array_equal(y1, a @ w[1].T)


def test_lossless_inputs_reduce_to_plain_matmul():
    # values already on the MXFP4 grid, each block holding the max code 6*2^e
    rng = np.random.default_rng(15)
    splits = [32, 0, 64]
    K, N, G = 64, 8, 3
    def on_grid(shape):
        mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
        v = mags[rng.integers(0, 8, size=shape)] * rng.choice([-1, 1], size=shape)
        v[..., ::32] = 6.0                      # block max at 6 -> e = 0 after scaling
        e = rng.integers(-4, 5, size=shape[:-1] + (shape[-1] // 32,))
        return v * np.repeat(2.0 ** e, 32, axis=-1)
    a = on_grid((sum(splits), K))
    w = on_grid((G * N, K))
    ab, wb = fp32_to_bf16_bits(a.astype(np.float32)), fp32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(ab), a)
    aq, as_ = mx.quantize_rowwise(ab, "mxfp4")
    wq, ws = mx.quantize_rowwise(wb, "mxfp4")
    np.testing.assert_array_equal(mx.dequantize_rowwise(aq, as_, "mxfp4"), a)
    y = grouped.grouped_fwd(mx.dequantize_rowwise(aq, as_, "mxfp4"),
                            mx.dequantize_rowwise(wq, ws, "mxfp4").reshape(G, N, K), splits)
    ref = np.concatenate([a[:32] @ w[:8].T, a[32:] @ w[16:24].T])
    np.testing.assert_array_equal(y, ref)


def test_wgrad_accumulate_minus_overwrite_is_main0_and_empty_rules():
    rng = np.random.default_rng(16)
    splits = [0, 40, 0, 24]
    N, K = 4, 8
    mpad = sum(-(-m // 32) * 32 for m in splits)
    dyc = rng.standard_normal((N, mpad))
    xc = rng.standard_normal((K, mpad))
    main0 = rng.standard_normal((4, N, K))
    acc = grouped.grouped_wgrad(dyc, xc, splits, main0, accumulate=True)
    ovw = grouped.grouped_wgrad(dyc, xc, splits, None, accumulate=False)
    np.testing.assert_array_equal(acc - ovw, main0 + ovw - ovw)
    np.testing.assert_array_equal(acc[0], main0[0])
    np.testing.assert_array_equal(acc[2], main0[2])
    assert np.all(ovw[0] == 0) and np.all(ovw[2] == 0)
