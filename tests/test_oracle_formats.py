"""Pins of the oracle's format decoders and its bf16 rounding.

Truth comes from outside the oracle: torch's float8_e4m3fn / float8_e8m0fnu /
bfloat16 casts (library routines), the exact embedding of every E2M1 value
into E4M3 (both are OCP minifloats), and a brute-force nearest-neighbour
search over all finite bf16 values.
"""
import math

import numpy as np
import pytest
import torch

import _bf16


def test_e4m3_all_codes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.dec_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # closed forms: largest finite, smallest subnormal, NaN codes
    assert orc.dec_e4m3(0x7E) == 448.0 and orc.dec_e4m3(0xFE) == -448.0
    assert orc.dec_e4m3(0x01) == 2.0 ** -9
    assert math.isnan(orc.dec_e4m3(0x7F)) and math.isnan(orc.dec_e4m3(0xFF))


def test_e8m0_all_codes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([orc.dec_e8m0(c) for c in range(256)])
    assert math.isnan(got[255]) and math.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert orc.dec_e8m0(127) == 1.0


def _e2m1_as_e4m3(code):
    # E2M1 (bias 1) value (1+m/2)*2^(e-1) is E4M3 (bias 7) with exponent
    # field e+6 and mantissa m<<2; the subnormal 0.5 is E4M3 exponent 6.
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0:
        mag = 0 if m == 0 else (6 << 3)
    else:
        mag = ((e + 6) << 3) | (m << 2)
    return (s << 7) | mag


def test_e2m1_all_codes(orc):
    codes = np.array([_e2m1_as_e4m3(c) for c in range(16)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.dec_e2m1(c) for c in range(16)])
    assert np.array_equal(got, ref)
    assert sorted(set(np.abs(got).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_bf16_decode_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.dec_bf16(int(c)) for c in codes[::7]])
    sub = ref[::7]
    assert np.array_equal(np.isnan(got), np.isnan(sub))
    ok = ~np.isnan(sub)
    assert np.array_equal(got[ok], sub[ok])


@pytest.fixture(scope="module")
def bf16_table():
    """All finite non-negative bf16 values, ascending, with their codes."""
    return _bf16.table()


_brute_rne = _bf16.brute_rne


def test_bf16_rne_brute_force(orc, bf16_table):
    codes, vals = bf16_table
    rng = np.random.default_rng(11)
    samples = []
    samples += list(rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 39, 3000))
    # exact midpoints and their fp64 neighbours (ties to even)
    idx = rng.integers(0, len(vals) - 1, 2000)
    for i in idx:
        mid = (vals[i] + vals[i + 1]) / 2
        samples += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid]
    # subnormal range, the largest finite values and overflow
    samples += [2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -140]
    samples += [vals[-1], vals[-1] * (1 + 2.0 ** -9), 2.0 ** 128, 1e300, -1e300, 0.0, -0.0]
    for v in samples:
        got = orc.bf16_rne(float(v))
        want = _brute_rne(float(v), codes, vals)
        assert got == want, (v, hex(got), hex(want))
    assert orc.bf16_rne(float("nan")) & 0x7FFF > 0x7F80
    assert orc.bf16_rne(float("inf")) == 0x7F80 and orc.bf16_rne(float("-inf")) == 0xFF80
