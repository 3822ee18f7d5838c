"""The library's blockwise-FP8 scale rule and its fp32 -> E4M3 encoder,
compiled for the host, against the oracle: floored amax, power-of-two
exponent and scale over every finite bf16 magnitude; E4M3 codes over every
binade that reaches E4M3 (normal, subnormal, underflow, saturation), at random
mantissas, at every rounding midpoint and one ulp either side of it."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import blockwise as ob
from oracle import mx
from oracle.formats import E4M3, bf16_bits_to_f64

HERE = os.path.dirname(os.path.abspath(__file__))


def _fp32_cases():
    rng = np.random.default_rng(7)
    out = []
    for fe in range(90, 146):                      # 2^-37 .. 2^18: underflow .. saturation
        mant = rng.integers(0, 1 << 23, size=2048, dtype=np.uint32)
        out.append((np.uint32(fe) << np.uint32(23)) | mant)
        # E4M3 keeps 3 mantissa bits in normal binades, fewer below 2^-6:
        # every midpoint between neighbours, and one fp32 ulp either side
        for keep in range(0, 4):
            step = np.uint32(1) << np.uint32(23 - keep)
            mids = (np.arange(1 << keep, dtype=np.uint32) * step) + (step >> np.uint32(1))
            for d in (-1, 0, 1):
                out.append((np.uint32(fe) << np.uint32(23)) | ((mids.astype(np.int64) + d) & 0x7FFFFF).astype(np.uint32))
    v = np.concatenate(out).astype(np.uint32)
    v = np.concatenate([v, v | np.uint32(0x80000000), np.array([0, 0x80000000, 1, 0x807FFFFF], dtype=np.uint32)])
    return v


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    cxx = shutil.which("hipcc")
    if cxx is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("blkr")
    exe = str(d / "blk_round_dump")
    subprocess.run([cxx, "-O2", "-std=c++17", "-o", exe, os.path.join(HERE, "host", "blk_round_dump.cpp")],
                   check=True, capture_output=True)
    vals = _fp32_cases()
    fin = str(d / "in.f32")
    vals.tofile(fin)
    out = str(d / "dump.bin")
    subprocess.run([exe, fin, out], check=True)
    raw = np.fromfile(out, dtype=np.uint8)
    rule = raw[:3 * 32768 * 4].view(np.uint32).reshape(32768, 3)
    codes = raw[3 * 32768 * 4:]
    return rule, vals, codes


def test_pow2_rule_every_bf16_magnitude(dump):
    rule, _, _ = dump
    mags = np.arange(32768, dtype=np.uint16)
    finite = (mags >> 7) != 0xFF
    amax = bf16_bits_to_f64(mags[finite])
    a_f = rule[finite, 0].view(np.float32).astype(np.float64)
    assert np.array_equal(a_f, np.maximum(amax, ob.AMAX_FLOOR))
    t = rule[finite, 1].view(np.int32).astype(np.int64)
    assert np.array_equal(t, ob.pow2_exponent(amax))
    s = rule[finite, 2].view(np.float32).astype(np.float64)
    assert np.array_equal(s, np.ldexp(1.0, -t))


def test_e4m3_encoder_matches_oracle_rounding(dump):
    _, vals, codes = dump
    y = vals.view(np.float32).astype(np.float64)
    ref = mx.round_to_format(y, E4M3)
    bad = np.nonzero(ref != codes)[0]
    assert bad.size == 0, [(hex(int(vals[i])), y[i], int(codes[i]), int(ref[i])) for i in bad[:5]]


def test_e4m3_encoder_covers_the_edges(dump):
    _, vals, codes = dump
    v = set(int(c) for c in codes)
    # saturation, the largest normal, the smallest normal, subnormals, signed zero
    assert {0x7E, 0xFE, 0x08, 0x01, 0x81, 0x00, 0x80} <= v
    assert 0x7F not in v and 0xFF not in v
