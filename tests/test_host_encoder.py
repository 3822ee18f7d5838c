"""The library's MX element encoder (compiled for the host) against the oracle
over every finite bf16 magnitude and every shared exponent in [-127, 127]."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import mx
from oracle.formats import E2M1, E4M3, bf16_bits_to_f64

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    cxx = shutil.which("hipcc")
    if cxx is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("enc")
    exe = str(d / "mx_encode_dump")
    subprocess.run([cxx, "-O2", "-std=c++17", "-o", exe,
                    os.path.join(HERE, "host", "mx_encode_dump.cpp")],
                   check=True, capture_output=True)
    out = str(d / "codes.bin")
    subprocess.run([exe, out], check=True)
    raw = np.fromfile(out, dtype=np.uint8)
    se = raw[:2 * 32768 * 2].view(np.int16).reshape(2, 32768)
    codes = raw[2 * 32768 * 2:].reshape(2, 255, 32768)
    return se, codes


def test_shared_exponent_all_magnitudes(dump):
    se, _ = dump
    mags = np.arange(32768, dtype=np.uint16)
    finite = (mags >> 7) != 0xFF
    amax = bf16_bits_to_f64(mags[finite])
    for k, f in enumerate((E2M1, E4M3)):
        ref = mx.shared_exponent(amax, f)
        assert np.array_equal(se[k][finite], ref)


@pytest.mark.parametrize("k,f", [(0, E2M1), (1, E4M3)])
def test_encode_all_magnitudes_all_exponents(dump, k, f):
    _, codes = dump
    mags = np.arange(32768, dtype=np.uint16)
    finite = (mags >> 7) != 0xFF
    x = bf16_bits_to_f64(mags[finite])
    for i, e in enumerate(range(-127, 128)):
        ref = mx.round_to_format(np.ldexp(x, -e), f)
        got = codes[k, i][finite]
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (e, hex(int(mags[finite][bad[0]])), int(got[bad[0]]), int(ref[bad[0]]))
