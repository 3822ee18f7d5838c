"""The library's MX shared-exponent rule and E4M3 saturation bound, compiled
for the host, against the oracle: shared exponent over every finite bf16
magnitude, clamp bound equal to 448 * 2^e, scale operand equal to 2^e."""
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
    d = tmp_path_factory.mktemp("mxr")
    exe = str(d / "mx_round_dump")
    subprocess.run([cxx, "-O2", "-std=c++17", "-o", exe, os.path.join(HERE, "host", "mx_round_dump.cpp")],
                   check=True, capture_output=True)
    out = str(d / "dump.bin")
    subprocess.run([exe, out], check=True)
    raw = np.fromfile(out, dtype=np.uint8)
    se = raw[:2 * 32768 * 2].view(np.int16).reshape(2, 32768)
    rest = raw[2 * 32768 * 2:].view(np.uint32)
    return se, rest[:255], rest[255:510]


def test_shared_exponent_all_magnitudes(dump):
    se, _, _ = dump
    mags = np.arange(32768, dtype=np.uint16)
    finite = (mags >> 7) != 0xFF
    amax = bf16_bits_to_f64(mags[finite])
    for k, f in enumerate((E2M1, E4M3)):
        assert np.array_equal(se[k][finite], mx.shared_exponent(amax, f))


def test_e4m3_saturation_bound(dump):
    _, lim, _ = dump
    for i, e in enumerate(range(-127, 128)):
        v = float(bf16_bits_to_f64(np.array([lim[i]], dtype=np.uint16))[0])
        if e <= 119:
            assert v == 448.0 * 2.0 ** e, e
        else:
            assert lim[i] == 0x7F7F       # no finite bf16 exceeds 448 * 2^e
        # every magnitude above the bound rounds to 448 * 2^e under the rule
        assert E4M3.values[mx.round_to_format(np.array([v * 2.0 ** -e]), E4M3)[0]] == 448.0 or e > 119


def test_scale_operand_is_2_pow_e(dump):
    _, _, scl = dump
    for i, e in enumerate(range(-127, 128)):
        # exponent field e + 127, mantissa 0; e = -127 is field 0 (read as 2^-127 by the conversion)
        assert scl[i] == (e + 127) << 23
