"""Pins for oracle.mx: the pages' worked example, exact brute force with
fractions, closed forms and invariants of the MX rule."""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.formats import E2M1, E4M3
from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# an exact, slow, independent restatement of the rule (fractions, no numpy)
# ----------------------------------------------------------------------------

def _bf16_fraction(b: int) -> Fraction:
    s = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    assert e != 0xFF
    if e == 0:
        return s * Fraction(m, 2 ** 133)
    return s * Fraction(128 + m) * Fraction(2) ** (e - 134)


def _magnitudes(name):
    """Finite non-negative magnitudes by code, from the spec's field layout."""
    if name == "e2m1":
        return [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
                Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            if e == 0:
                out.append(Fraction(m, 8) * Fraction(1, 64))
            else:
                out.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return out


def _brute_block(bits, name):
    mags = _magnitudes(name)
    emax = 2 if name == "e2m1" else 8
    sign_bit = 0x8 if name == "e2m1" else 0x80
    xs = [_bf16_fraction(int(b)) for b in bits]
    amax = max(abs(x) for x in xs)
    if amax == 0:
        e = -127
    else:
        L = 0
        while Fraction(2) ** L > amax:
            L -= 1
        while Fraction(2) ** (L + 1) <= amax:
            L += 1
        e = min(max(L - emax, -127), 127)
    codes = []
    for b, x in zip(bits, xs):
        y = abs(x) / Fraction(2) ** e
        if y >= mags[-1]:
            k = len(mags) - 1
        else:
            best = min(abs(y - v) for v in mags)
            ks = [i for i, v in enumerate(mags) if abs(y - v) == best]
            k = ks[0] if len(ks) == 1 else [i for i in ks if i % 2 == 0][0]
        codes.append(k | (sign_bit if int(b) & 0x8000 else 0))
    return codes, e + 127


def _random_bf16_blocks(rng, nblocks):
    """Blocks with a spread of binades, subnormals, zeros and exact ties."""
    out = []
    for i in range(nblocks):
        kind = i % 5
        if kind == 0:       # wide random exponents incl. subnormals
            e = rng.integers(0, 255, size=32)
            m = rng.integers(0, 128, size=32)
        elif kind == 1:     # one binade region, common case
            e = rng.integers(120, 132, size=32)
            m = rng.integers(0, 128, size=32)
        elif kind == 2:     # near the bottom of the range
            e = rng.integers(0, 4, size=32)
            m = rng.integers(0, 128, size=32)
        elif kind == 3:     # near the top of the range
            e = rng.integers(250, 255, size=32)
            m = rng.integers(0, 128, size=32)
        else:               # exact E2M1 midpoints after scale 2^0 (amax 4)
            vals = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 3.0, 0.5, 1.5,
                             0.125, 2.25, 2.75, 3.25, 3.75, 1.0] * 2, dtype=np.float32)
            b = (vals.view(np.uint32) >> 16).astype(np.uint16)
            s = rng.integers(0, 2, size=32).astype(np.uint16) << 15
            out.append(b | s)
            continue
        s = rng.integers(0, 2, size=32)
        b = (s << 15) | (e << 7) | m
        zero = rng.random(32) < 0.1
        b = np.where(zero, s << 15, b)
        out.append(b.astype(np.uint16))
    return np.stack(out)


@pytest.mark.parametrize("name", ["e2m1", "e4m3"])
def test_rowwise_matches_exact_brute_force(name):
    rng = np.random.default_rng(123)
    blocks = _random_bf16_blocks(rng, 40)           # 40 blocks = 5 rows x 256
    x = blocks.reshape(5, 256)
    fmt = "mxfp4" if name == "e2m1" else "mxfp8"
    q, s = mx.quantize_rowwise(x, fmt)
    f = E2M1 if name == "e2m1" else E4M3
    codes = mx.unpack_codes(q, f)
    for r in range(5):
        for j in range(8):
            bc, bs = _brute_block(x[r, j * 32:(j + 1) * 32], name)
            assert int(s[r, j]) == bs, (r, j)
            assert [int(c) for c in codes[r, j * 32:(j + 1) * 32]] == bc, (r, j)


def test_worked_example_tiny_scale():
    kv = {}
    with open(os.path.join(GOLDEN, "tiny_scale_e4m3.txt")) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k] = v
    bits = np.array([int(t, 16) for t in kv["block_bf16"].split()], dtype=np.uint16)
    q, s = mx.quantize_rowwise(bits[None, :], kv["format"])
    assert int(s[0, 0]) - 127 == int(kv["scale_exponent"])
    assert E4M3.values[q[0, 0]] == float(kv["element0_value"])
    assert np.all(q[0, 1:] == 0)
    # the same block in E2M1 keeps the value too: 2^-126 * 2^127 = 2 -> code 0x4
    q4, s4 = mx.quantize_rowwise(bits[None, :], "mxfp4")
    assert s4[0, 0] == 0 and (q4[0, 0] & 0xF) == 0x4


def test_closed_form_all_ones():
    ones = np.full((2, 64), 0x3F80, dtype=np.uint16)
    q, s = mx.quantize_rowwise(ones, "mxfp4")
    assert np.all(q == 0x66) and np.all(s == 125)       # 1 * 2^2 = 4 = code 6
    q8, s8 = mx.quantize_rowwise(ones, "mxfp8")
    assert np.all(q8 == 0x78) and np.all(s8 == 119)     # 1 * 2^8 = 256 = 0x78


def test_e2m1_rounding_intervals():
    # RNE intervals implied by the E2M1 magnitudes 0,.5,1,1.5,2,3,4,6
    cases = {0.0: 0, 0.25: 0, 0.2500001: 1, 0.74999: 1, 0.75: 2, 1.25: 2,
             1.2500001: 3, 1.75: 4, 2.5: 4, 2.5000001: 5, 3.5: 6, 5.0: 6,
             5.0000001: 7, 6.0: 7, 1e9: 7}
    ys = np.array(list(cases.keys()))
    got = mx.round_to_format(ys, E2M1)
    assert [int(c) for c in got] == list(cases.values())
    neg = mx.round_to_format(-ys, E2M1)
    assert [int(c) for c in neg] == [c | 8 for c in cases.values()]


def test_e4m3_rounding_saturation_and_ties():
    f = E4M3
    ys = np.array([448.0, 464.0, 480.0, 1e6, 1.0 + 1 / 16, 1.0 + 3 / 16,
                   2.0 ** -10, 2.0 ** -10 + 2.0 ** -20, 3 * 2.0 ** -10])
    got = [int(c) for c in mx.round_to_format(ys, f)]
    # 464 is the midpoint of 448 (0x7E) and the NaN slot: saturates to 448
    assert got[:4] == [0x7E, 0x7E, 0x7E, 0x7E]
    assert got[4] == 0x38          # 1+1/16: tie between 0x38 (even) and 0x39
    assert got[5] == 0x3A          # 1+3/16: tie between 0x39 and 0x3A (even)
    assert got[6] == 0x00          # 2^-10: half the smallest subnormal -> 0
    assert got[7] == 0x01
    assert got[8] == 0x02          # 1.5 * 2^-9: tie -> even code 2


def test_zero_blocks():
    z = np.zeros((1, 32), dtype=np.uint16)
    q, s = mx.quantize_rowwise(z, "mxfp4")
    assert np.all(q == 0) and s[0, 0] == 0
    nz = np.full((1, 32), 0x8000, dtype=np.uint16)
    q, s = mx.quantize_rowwise(nz, "mxfp4")
    assert np.all(q == 0x88) and s[0, 0] == 0
    q, s = mx.quantize_rowwise(nz, "mxfp8")
    assert np.all(q == 0x80) and s[0, 0] == 0


def test_subnormal_input_block():
    x = np.zeros((1, 32), dtype=np.uint16)
    x[0, 0] = 0x0001            # 2^-133
    q, s = mx.quantize_rowwise(x, "mxfp8")
    assert s[0, 0] == 0 and q[0, 0] == 0x08     # 2^-133 * 2^127 = 2^-6
    q, s = mx.quantize_rowwise(x, "mxfp4")
    assert s[0, 0] == 0 and q[0, 0] == 0        # 2^-6 rounds to 0 in E2M1


def test_pack_nibble_order():
    codes = np.array([[1, 2, 3, 4, 0xF, 0x8]], dtype=np.uint8)
    assert list(mx.pack_codes(codes, E2M1)[0]) == [0x21, 0x43, 0x8F]
    assert np.array_equal(mx.unpack_codes(mx.pack_codes(codes, E2M1), E2M1), codes)


def _bf16(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_invariants(fmt):
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((8, 128)).astype(np.float32))
    q, s = mx.quantize_rowwise(x, fmt)
    d = mx.dequantize_rowwise(q, s, fmt)
    # idempotence: quantizing the dequantized values reproduces them
    d_bits = _bf16(d.astype(np.float32))
    assert np.array_equal(mx.bf16_bits_to_f64(d_bits), d)    # exact in bf16
    q2, s2 = mx.quantize_rowwise(d_bits, fmt)
    assert np.array_equal(mx.dequantize_rowwise(q2, s2, fmt), d)
    # sign symmetry
    qn, sn = mx.quantize_rowwise(x ^ np.uint16(0x8000), fmt)
    assert np.array_equal(sn, s)
    f = E2M1 if fmt == "mxfp4" else E4M3
    assert np.array_equal(mx.unpack_codes(qn, f), mx.unpack_codes(q, f) ^ f.sign_bit)
    # power-of-two equivariance (no clamping for these magnitudes)
    for j in (-5, 3):
        xj = _bf16((mx.bf16_bits_to_f64(x) * 2.0 ** j).astype(np.float32))
        qj, sj = mx.quantize_rowwise(xj, fmt)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj.astype(int), s.astype(int) + j)
    # permutation equivariance inside a block
    perm = rng.permutation(32)
    xp = x.copy()
    xp[:, :32] = x[:, :32][:, perm]
    qp, sp = mx.quantize_rowwise(xp, fmt)
    assert np.array_equal(sp, s)
    assert np.array_equal(mx.unpack_codes(qp, f)[:, :32], mx.unpack_codes(q, f)[:, :32][:, perm])


def test_large_exponent_clamp_top():
    # amax near the bf16 maximum: e = 127 - 2 = 125 for E2M1 (no clamp needed)
    x = np.zeros((1, 32), dtype=np.uint16)
    x[0, 0] = 0x7F7F
    q, s = mx.quantize_rowwise(x, "mxfp4")
    assert int(s[0, 0]) == 127 + 125
    assert (q[0, 0] & 0xF) == 0x7   # (2-2^-7)*2^127 / 2^125 = 7.97 -> saturates to 6


@pytest.mark.parametrize("pad", [32, 128])
def test_colwise_segpad_layout(pad):
    rng = np.random.default_rng(5)
    splits = [40, 0, 7, 33, 64]
    rows, cols = sum(splits), 64
    x = _bf16(rng.standard_normal((rows, cols)).astype(np.float32))
    q, s = mx.quantize_colwise_segpad(x, splits, "mxfp4", pad=pad)
    padded = [-(-m // pad) * pad for m in splits]
    mpad = sum(padded)
    assert q.shape == (cols, mpad // 2) and s.shape == (cols, mpad // 32)
    codes = mx.unpack_codes(q, E2M1)
    # rebuild each block independently: column c, expert g, block j
    r0 = p0 = 0
    for m, pm in zip(splits, padded):
        for j in range(pm // 32):
            for c in range(cols):
                blk = np.zeros(32, dtype=np.uint16)
                lo = j * 32
                hi = min(m, lo + 32)
                if hi > lo:
                    blk[:hi - lo] = x[r0 + lo:r0 + hi, c]
                bc, bs = _brute_block(blk, "e2m1")
                got_c = [int(v) for v in codes[c, p0 + lo:p0 + lo + 32]]
                assert got_c == bc and int(s[c, (p0 + lo) // 32]) == bs
        r0 += m
        p0 += pm


def test_segpad_pad_invariance():
    rng = np.random.default_rng(9)
    splits = [70, 3, 0, 128]
    x = _bf16(rng.standard_normal((sum(splits), 32)).astype(np.float32))
    q32, s32 = mx.quantize_colwise_segpad(x, splits, "mxfp8", pad=32)
    q128, s128 = mx.quantize_colwise_segpad(x, splits, "mxfp8", pad=128)
    _, p32 = mx.segpad_offsets(splits, 32)
    _, p128 = mx.segpad_offsets(splits, 128)
    for g, m in enumerate(splits):
        nb = -(-m // 32)
        a = q32[:, p32[g]:p32[g] + nb * 32]
        b = q128[:, p128[g]:p128[g] + nb * 32]
        assert np.array_equal(a, b)
        assert np.array_equal(s32[:, p32[g] // 32:p32[g] // 32 + nb],
                              s128[:, p128[g] // 32:p128[g] // 32 + nb])
        # the extra padding of the 128 layout is zero codes
        assert np.all(q128[:, p128[g] + nb * 32:p128[g + 1]] == 0)
