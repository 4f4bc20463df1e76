"""Pins for the oracle's scalar rules: E2M1 coding, E8M0 and UE4M3/UE5M3 scales.

Each rule is checked against something other than the oracle's own code: an
independent formulation (np.rint on the grid spacing, integer bit arithmetic),
a library routine (torch's float8_e4m3fn cast), exact rational arithmetic, or
the constants the pages state (tests/golden/page_constants.json).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def all_finite_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def rint_code(y: np.ndarray) -> np.ndarray:
    """E2M1 code by a second formulation: the grid spacing is 0.5 below 2, 1
    below 4 and 2 above; np.rint (ties to even multiple) on |y|/spacing; an even
    multiple of the spacing is an even code in every range; clamp at 6."""
    a = np.minimum(np.abs(y), 6.0)
    q = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(a / q) * q, 6.0)
    mag = np.searchsorted(GRID, r)  # r is on the grid
    assert np.all(GRID[mag] == r)
    return (np.signbit(y).astype(np.uint8) << 3) | mag.astype(np.uint8)


def test_e2m1_exhaustive_bf16_times_scales(orc):
    """All finite bf16 values x times 2^-E for a spread of exponents E: oracle
    code == np.rint formulation (ties, saturation, signed zero included)."""
    x = all_finite_bf16_as_f32().astype(np.float64)
    for E in list(range(-135, -115)) + list(range(-10, 11)) + list(range(115, 128)):
        y = np.ldexp(x, -E)
        np.testing.assert_array_equal(orc.e2m1_codes(y), rint_code(y), err_msg=f"E={E}")


def test_e2m1_ties_and_signs(orc):
    # exact ties go to the even code; magnitudes past 6 saturate; -0 keeps its sign
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6), (7.0, 7),
             (1e30, 7), (0.0, 0), (-0.0, 8), (-0.25, 8), (-0.2500001, 9), (5.000001, 7),
             (-6.0, 15)]
    for y, c in cases:
        assert orc.e2m1_code(y) == c, y
    for c in range(16):
        v = orc.e2m1_value(c)
        assert abs(v) == GRID[c & 7] and (c < 8 or v <= 0)


def floor_log2_bits(m: np.ndarray) -> np.ndarray:
    """floor(log2 m) of positive float32 by integer bit arithmetic."""
    b = m.view(np.uint32).astype(np.int64)
    e = (b >> 23) & 0xFF
    man = b & 0x7FFFFF
    sub = np.array([int(v).bit_length() - 1 - 149 for v in man[e == 0]], dtype=np.int64)
    out = e - 127
    out[e == 0] = sub
    return out


def test_e8m0_exhaustive_positive_bf16(orc):
    x = all_finite_bf16_as_f32()
    m = x[x > 0]
    want = np.clip(floor_log2_bits(m) - 2, -127, 127)
    np.testing.assert_array_equal(orc.e8m0_exponents(m), want)
    assert orc.e8m0_exponent(0.0) == -127


def test_e8m0_fp32_subnormals_and_random(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(1, 0x7F800000, size=200000, dtype=np.uint32)
    m = bits.view(np.float32)
    want = np.clip(floor_log2_bits(m) - 2, -127, 127)
    np.testing.assert_array_equal(orc.e8m0_exponents(m), want)
    # math.frexp agrees on the exponent
    for v in m[:2000]:
        assert orc.e8m0_exponent(v) == max(min(math.frexp(float(v))[1] - 3, 127), -127)


def test_e8m0_floor_not_ceil(orc):
    # max 1.875: floor(log2) = 0 -> E = -2 (byte 0x7D); a ceil rule would give -1
    assert orc.e8m0_exponent(1.875) == -2
    assert orc.e8m0_exponent(4.0) == 0 and orc.e8m0_exponent(7.999) == 0


def ue4m3_reference(s: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn cast (round to nearest even, non-saturating) after
    clamping to the largest finite value 448."""
    t = torch.from_numpy(np.minimum(s, np.float32(448.0)).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def ue4m3_sweep_points():
    vals = np.array([sorted({j * 2.0 ** -9 for j in range(8)} |
                            {(1 + j / 8) * 2.0 ** (e - 7) for e in range(1, 16) for j in range(8)
                             if not (e == 15 and j == 7)})])[0]
    mids = 0.5 * (vals[1:] + vals[:-1])
    pts = [np.float32(v) for v in np.concatenate([vals, mids, [464.0, 470.0, 480.0, 1e6]])]
    base = np.array(pts, dtype=np.float32)
    near = [np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(0))]
    rng = np.random.default_rng(3)
    rnd = (rng.random(300000) * 470.0).astype(np.float32)
    small = (rng.random(100000) * 0.02).astype(np.float32)
    bf = all_finite_bf16_as_f32()
    bf = bf[~np.signbit(bf) & (bf < 1e5)]  # block scales are never negative (m = max |x|)
    return np.concatenate([base, *near, rnd, small, bf])


def test_ue4m3_against_torch_cast(orc):
    s = ue4m3_sweep_points()
    np.testing.assert_array_equal(orc.ue4m3_bytes(s), ue4m3_reference(s))


def test_ue4m3_values_and_page_constants(orc):
    const = json.load(open(GOLDEN))
    nz = [orc.ue4m3_value(b) for b in range(1, 0x7F)]
    assert min(nz) == 2.0 ** const["ue4m3_min_nonzero_scale"]["value_log2"]
    assert max(nz) == 448.0
    # the byte is the E4M3 bit pattern with a clear sign bit
    for b in range(0x7F):
        want = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
        assert orc.ue4m3_value(b) == want
    # zero-rounding boundary: s = 2^-10 ties between 0 and 2^-9 and goes to code 0
    assert orc.ue4m3_byte(2.0 ** -10) == 0
    assert orc.ue4m3_byte(float(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))) == 1


def ue5m3_bits_reference(s: np.ndarray) -> np.ndarray:
    """UE5M3 by bit arithmetic: round the binary32 significand to 3 bits (ties to
    even) above 2^-14; multiples of 2^-17 (np.rint) below; saturate at 61440."""
    s = s.astype(np.float32)
    b = s.view(np.uint32).astype(np.int64)
    lsb = (b >> 20) & 1
    r = (b + 0x7FFFF + lsb) >> 20
    normal = r - (112 << 3)
    sub = np.rint(s.astype(np.float64) * 2.0 ** 17).astype(np.int64)
    out = np.where(s < 2.0 ** -14, sub, normal)
    return np.minimum(out, 0xF7).astype(np.uint8)


def test_ue5m3_against_bit_formulation(orc):
    const = json.load(open(GOLDEN))
    rng = np.random.default_rng(5)
    s = np.concatenate([(rng.random(200000) * 70000).astype(np.float32),
                        (rng.random(200000) * 1e-3).astype(np.float32),
                        np.float32(2.0) ** rng.integers(-19, 17, 50000).astype(np.float32)
                        * (1 + rng.integers(0, 16, 50000) / np.float32(16))])
    s = s.astype(np.float32)
    np.testing.assert_array_equal(orc.ue5m3_bytes(s), ue5m3_bits_reference(s))
    nz = [orc.ue5m3_value(b) for b in range(1, 0xF8)]
    assert min(nz) == 2.0 ** const["ue5m3_min_nonzero_scale"]["value_log2"]
    assert max(nz) == 61440.0


def rn32(q: Fraction) -> float:
    """Round an exact rational to the nearest binary32 (ties to even), normal range."""
    neg = q < 0
    q = abs(q)
    e = math.floor(math.log2(q.numerator) - math.log2(q.denominator))
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    scaled = q / Fraction(2) ** (e - 23)  # in [2^23, 2^24)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(Fraction(n) * Fraction(2) ** (e - 23))
    return -v if neg else v


def test_nv_element_codes_use_correctly_rounded_division(orc):
    """Codes of a UE4M3 block equal the codes of RN32(x/d) with the quotient
    rounded by hand from its exact rational value."""
    rng = np.random.default_rng(11)
    g = np.float32(0.0137)
    n_blk = 400
    x = (rng.standard_normal((n_blk, 16)) * 0.05).astype(np.float32)
    # put exact E2M1 midpoints times d into some blocks to stress ties
    r = orc.quantize(x, orc.FMT_UE4M3, 16, orc.GMODE_GIVEN, g=float(g))
    codes = np.empty((n_blk, 16), np.uint8)
    codes[:, 0::2] = r["codes"] & 0xF
    codes[:, 1::2] = r["codes"] >> 4
    for i in range(n_blk):
        sb = int(r["scales"][i, 0])
        shat = np.float32(orc.ue4m3_value(sb))
        d = np.float32(shat * g)
        for j in range(16):
            if d == 0:
                want = 8 if np.signbit(x[i, j]) else 0
            else:
                y = rn32(Fraction(float(x[i, j])) / Fraction(float(d))) if x[i, j] != 0 else float(x[i, j])
                want = rint_code(np.array([y]))[0]
            assert codes[i, j] == want, (i, j)


def test_bf16_rounding_against_torch(orc):
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.integers(0, 0x7F7FFFFF, 100000, dtype=np.uint32)).view(np.float32),
                        (np.arange(0, 65536, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    v = v[np.isfinite(v)]
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.to_bf16_bits(v), want)
