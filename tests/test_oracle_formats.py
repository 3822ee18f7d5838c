"""Pins for oracle.formats against values the OCP specifications list."""
import math

import numpy as np

from oracle.formats import E2M1, E4M3, bf16_bits_to_f64, ue8m0_to_f64


def test_e2m1_table_matches_ocp_list():
    # OCP MX v1.0, FP4 E2M1 value table: magnitudes of codes 0..7
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(E2M1.values[:8]) == expect
    assert list(E2M1.values[8:]) == [-v for v in expect]
    assert math.copysign(1.0, E2M1.values[8]) == -1.0       # 0x8 is -0
    assert E2M1.emax == 2 and E2M1.max_value == 6.0 and E2M1.max_mag_code == 7


def test_e4m3_spot_values():
    v = E4M3.values
    assert v[0x38] == 1.0
    assert v[0x40] == 2.0
    assert v[0x7E] == 448.0
    assert v[0x08] == 2.0 ** -6          # smallest normal
    assert v[0x01] == 2.0 ** -9          # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert v[0x78] == 256.0
    assert v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert math.copysign(1.0, v[0x80]) == -1.0 and v[0x80] == 0.0
    assert E4M3.emax == 8 and E4M3.max_mag_code == 0x7E


def test_e4m3_structure():
    v = E4M3.values
    assert np.isfinite(v).sum() == 254
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)      # magnitude codes increase with value
    assert np.array_equal(v[0x80:0xFF], -pos)
    # within each binade the spacing is 2^(e-3) (3 mantissa bits)
    for e in range(1, 15):
        seg = pos[e * 8:(e + 1) * 8]
        assert np.allclose(np.diff(seg), 2.0 ** (e - 7 - 3))


def test_bf16_decode():
    bits = np.array([0x3F80, 0x0001, 0x8000, 0x7F7F, 0x4040, 0xBF00, 0x0080], dtype=np.uint16)
    v = bf16_bits_to_f64(bits)
    assert v[0] == 1.0
    assert v[1] == 2.0 ** -133
    assert v[2] == 0.0 and math.copysign(1.0, v[2]) == -1.0
    assert v[3] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert v[4] == 3.0
    assert v[5] == -0.5
    assert v[6] == 2.0 ** -126


def test_ue8m0():
    b = np.array([0, 1, 127, 128, 254, 255])
    v = ue8m0_to_f64(b)
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126 and v[2] == 1.0
    assert v[3] == 2.0 and v[4] == 2.0 ** 127 and np.isnan(v[5])
