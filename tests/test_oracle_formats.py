"""Pins for the oracle's element formats (CPU only).

Each check ties the oracle to something other than itself: the value set
printed on the 7minutos.es NVFP4 page, a library conversion (torch's
float8_e4m3fn / bfloat16), or an exact brute force with rational arithmetic.
"""

import bisect
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.conftest import read_golden

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def finite_bf16_values():
    v = F.bf16_bits_to_f32(ALL_BF16)
    keep = np.isfinite(v)
    return ALL_BF16[keep], v[keep].astype(np.float64)


def test_e2m1_value_set_matches_page():
    printed = sorted(float(x) for x in read_golden("e2m1_values.txt"))
    pos = [F.e2m1_value(c) for c in range(8)]
    neg = [F.e2m1_value(c) for c in range(8, 16)]
    assert pos == printed                      # codes 0..7 in ascending order
    assert [-p for p in pos] == neg            # sign bit = bit 3
    assert np.signbit(F.e2m1_value(8))         # -0


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))
    assert F.E4M3_TABLE[0x7E] == 448.0 and F.E4M3_TABLE[0x08] == 2.0 ** -6
    assert F.E4M3_TABLE[0x01] == 2.0 ** -9


def test_e8m0_scales_are_powers_of_two():
    vals = F.E8M0_TABLE[:255]
    m, _ = np.frexp(vals)
    assert np.all(m == 0.5)                    # every scale is a power of two
    assert np.all(vals[1:] / vals[:-1] == 2.0)  # one binade per code
    assert vals[127] == 1.0 and np.isnan(F.E8M0_TABLE[255])


def _brute_nearest(values, grid_vals, grid_codes, vmax):
    """Nearest grid value with rational arithmetic; ties -> even code; |v| > vmax -> vmax."""
    out = []
    for v in values:
        a = Fraction(abs(float(v)))
        if a >= Fraction(vmax):
            out.append(grid_codes[-1])
            continue
        i = bisect.bisect_left(grid_vals, a)
        if grid_vals[i] == a:
            out.append(grid_codes[i])
            continue
        lo, hi = grid_vals[i - 1], grid_vals[i]
        dlo, dhi = a - lo, hi - a
        if dlo < dhi:
            out.append(grid_codes[i - 1])
        elif dhi < dlo:
            out.append(grid_codes[i])
        else:
            out.append(grid_codes[i - 1] if grid_codes[i - 1] % 2 == 0 else grid_codes[i])
    return np.array(out, dtype=np.int64)


def test_e4m3_rne_sat_exhaustive_bf16_vs_rational_brute_force():
    bits, v = finite_bf16_values()
    grid_codes = list(range(0x7F))
    grid_vals = [Fraction(F.e4m3_value(c)) for c in grid_codes]
    mag_codes = _brute_nearest(v, grid_vals, grid_codes, 448.0)
    expect = mag_codes | (np.signbit(v).astype(np.int64) << 7)
    got = F.encode_e4m3(v).astype(np.int64)
    assert np.array_equal(got, expect)


def test_e4m3_in_range_matches_torch_conversion():
    _, v = finite_bf16_values()
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.encode_e4m3(v), ref)


def test_e2m1_rne_sat_exhaustive_bf16_vs_rational_brute_force():
    bits, v = finite_bf16_values()
    grid_codes = list(range(8))
    grid_vals = [Fraction(F.e2m1_value(c)) for c in grid_codes]
    mag_codes = _brute_nearest(v, grid_vals, grid_codes, 6.0)
    expect = mag_codes | (np.signbit(v).astype(np.int64) << 3)
    assert np.array_equal(F.encode_e2m1(v).astype(np.int64), expect)


def test_e2m1_ties_go_to_even_code():
    # midpoints between neighbouring magnitudes, and saturation past 6
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 1e30, -0.25, -5.0])
    codes = F.encode_e2m1(v)
    assert list(codes) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 0x8, 0xE]


def test_round_trip_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert int(F.encode_e4m3(np.array([F.e4m3_value(c)]))[0]) == c
    for c in range(16):
        assert int(F.encode_e2m1(np.array([F.e2m1_value(c)]))[0]) == c


def test_f32_to_bf16_matches_torch():
    g = np.random.default_rng(7)
    v = np.concatenate([
        g.standard_normal(200000).astype(np.float32),
        (g.standard_normal(20000) * 1e-39).astype(np.float32),   # FP32 subnormals
        np.array([3.3895314e38, -3.4e38, 0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                 dtype=np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_bits(v), ref)


def test_f32_to_bf16_infinities_overflow_and_ties():
    # IEEE binary32 bit patterns rounded to their top 16 bits, nearest-even:
    #   +-Inf stay +-Inf (0x7F80 / 0xFF80); FLT_MAX 0x7F7FFFFF rounds up past the BF16
    #   maximum 0x7F7F to Inf; 0x7F7F8000 is a tie whose lower neighbour 0x7F7F is odd, so
    #   it goes up to Inf; 0x3F808000 is a tie between 0x3F80 (even) and 0x3F81, so it stays;
    #   0x3F818000 is a tie between 0x3F81 (odd) and 0x3F82, so it goes up; 0x3F807FFF is
    #   below the tie; the smallest FP32 subnormal 0x00000001 rounds to +0.
    bits = np.array([0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x3F808000,
                     0x3F818000, 0x3F807FFF, 0x00000001, 0x80000001], dtype=np.uint32)
    got = F.f32_to_bf16_bits(bits.view(np.float32))
    assert [int(b) for b in got] == [0x7F80, 0xFF80, 0x7F80, 0xFF80, 0x7F80, 0x3F80, 0x3F82, 0x3F80,
                                     0x0000, 0x8000]


def test_nonfinite_inputs_are_rejected():
    with pytest.raises(ValueError):
        F.encode_e4m3(np.array([np.nan]))
    with pytest.raises(ValueError):
        F.encode_e2m1(np.array([np.inf]))
