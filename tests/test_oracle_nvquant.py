"""Pins for the oracle's NV quantizer (fp32 -> E2M1 codes + E4M3 block scales per 16,
with a caller-supplied fp32 global scale g).

The rule (a reading: the pages fix none) is written out in oracle.c: per 16-element
block, sv = amax / (6 g) in fp32, the scale is the E4M3 code nearest to sv (ties to
the even code, saturating at 448), and each element is x * min(1 / (e4m3(s) g), FLT_MAX)
in fp32, rounded to the nearest E2M1 value (ties to the even mantissa bit, saturating at
6, zero +0).
Each pin checks it against something other than the oracle's own search:
- the E4M3 values printed by the format's definition (0x38 = 1, 0x7E = 448, ...) and
  exact round trips of all 126 positive finite scale codes;
- every midpoint between neighbouring scale codes, which must go to the even code;
- exact round trips of values on the E2M1 grid, and every E2M1 tie;
- the rounding error bound of round-to-nearest on both grids, and saturation;
- the zero, underflowing and non-finite blocks, and negative zero.
"""
import numpy as np
import pytest

import datagen

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # E2M1 magnitudes, codes 0..7


def e4m3_positive():
    """Values of the finite non-negative E4M3FN codes 0x00..0x7E, from the format's
    definition (bias 7, 3 mantissa bits, subnormals below 2^-6), not from the oracle."""
    v = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        v.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(v)


E4 = e4m3_positive()


def dequant(codes, scales, g):
    c = datagen.unpack_nibbles(codes).astype(np.int64)
    mag = GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    s = np.repeat(E4[scales.astype(np.int64)], 16, axis=1)
    return mag * s * np.float64(np.float32(g))


def test_e4m3_table_anchors(oracle_lib):
    assert E4[0x38] == 1.0 and E4[0x7E] == 448.0 and E4[0x01] == 2.0 ** -9
    assert E4[0x28] == 0.25 and E4[0x48] == 4.0 and E4[0x08] == 2.0 ** -6
    assert np.all(np.diff(E4) > 0)


def test_every_scale_code_round_trips(oracle_lib):
    # g = 1 and amax = 6 * e4m3(c): both fp32 operations are exact, so sv = e4m3(c)
    codes = np.arange(1, 0x7F)
    x = np.zeros((len(codes), 16), np.float32)
    x[:, 3] = (6.0 * E4[codes]).astype(np.float32)
    x[:, 7] = -x[:, 3] * np.float32(0.25)
    _, s = oracle_lib.nv_quantize(x, 1.0)
    assert np.array_equal(s[:, 0].astype(np.int64), codes)


def test_scale_ties_go_to_the_even_code(oracle_lib):
    # midpoints between neighbouring finite codes, scaled by 6 (exact in fp32)
    lo = np.arange(0, 0x7E)
    mid = (E4[lo] + E4[lo + 1]) / 2
    x = np.zeros((len(lo), 16), np.float32)
    x[:, 0] = (6.0 * mid).astype(np.float32)
    assert np.array_equal(x[:, 0].astype(np.float64), 6.0 * mid)      # the midpoints are exact
    _, s = oracle_lib.nv_quantize(x, 1.0)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(s[:, 0].astype(np.int64), want)


def test_scale_is_nearest_and_saturates(oracle_lib):
    rng = np.random.default_rng(3)
    amax = (rng.uniform(0.5, 1.0, 400) * np.ldexp(1.0, rng.integers(-14, 14, 400))).astype(np.float32)
    g = np.float32(0.37)
    x = np.zeros((400, 16), np.float32)
    x[:, 11] = amax
    _, s = oracle_lib.nv_quantize(x, g)
    sv = (amax / np.float32(np.float32(6.0) * g)).astype(np.float64)
    got = E4[s[:, 0].astype(np.int64)]
    best = np.abs(E4[None, :] - np.minimum(sv, 448.0)[:, None]).min(axis=1)
    assert np.all(np.abs(got - np.minimum(sv, 448.0)) == best)
    big = np.zeros((2, 16), np.float32)
    big[0, 0], big[1, 0] = 6 * 449.0, np.float32(3e38)
    _, s2 = oracle_lib.nv_quantize(big, 1.0)
    assert list(s2[:, 0]) == [0x7E, 0x7E]


def test_elements_saturate_however_large(oracle_lib):
    # with the scale saturated at 448, x / d can be far above 6: the code is still 6
    x = np.zeros((3, 16), np.float32)
    x[0, 2] = np.float32(3e38)
    x[1, 0], x[1, 1] = 6 * 500.0, -6 * 500.0
    x[2, 5] = -np.float32(1e30)
    codes, s = oracle_lib.nv_quantize(x, 1.0)
    assert np.all(s[:, 0] == 0x7E)
    c = datagen.unpack_nibbles(codes)[:, :16]
    assert c[0, 2] == 7 and c[1, 0] == 7 and c[1, 1] == 15 and c[2, 5] == 15
    assert c[0, [0, 1, 3]].tolist() == [0, 0, 0]


def test_grid_values_round_trip(oracle_lib):
    # scale code 0x38 (1.0) with g = 1/4: d = 0.25 exactly, and x = 0.25 * grid value
    rng = np.random.default_rng(5)
    c = rng.integers(0, 16, (64, 16))
    c[:, 0] = 7                                          # |6| fixes amax = 1.5: sv = 1.5 / 1.5 = 1.0
    mag = GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    x = (mag * 0.25).astype(np.float32)
    codes, s = oracle_lib.nv_quantize(x, 0.25)
    assert np.all(s == 0x38)
    want = np.where((c & 7) == 0, 0, c)                  # zero magnitudes come out +0
    assert np.array_equal(datagen.unpack_nibbles(codes).astype(np.int64), want)


def test_element_ties_go_to_even(oracle_lib):
    # midpoints of the E2M1 grid at d = 1 (scale 0x38, g = 1; amax 6 fixes sv = 1)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.0
    x[0, 1:8] = mids
    x[0, 8:15] = -np.array(mids, np.float32)
    codes, s = oracle_lib.nv_quantize(x, 1.0)
    assert s[0, 0] == 0x38
    got = datagen.unpack_nibbles(codes)[0].astype(np.int64)
    assert list(got[1:8]) == want
    assert list(got[8:15]) == [w | 8 if w else 0 for w in want]


def test_error_bound(oracle_lib):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 256)) * np.ldexp(1.0, rng.integers(-6, 6, (64, 1)))).astype(np.float32)
    g = np.float32(np.abs(x).max() / (448.0 * 6.0))
    codes, s = oracle_lib.nv_quantize(x, g)
    xd = dequant(codes, s, g)
    d = np.repeat(E4[s.astype(np.int64)], 16, axis=1) * np.float64(g)
    y = np.abs(x.astype(np.float64)) / d
    # half the local grid step (0.25 below 2, 0.5 below 4, 1 above), relative to d,
    # plus the fp32 rounding of y; saturation at 6 adds |y| - 6
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    bound = (half + np.maximum(y - 6.0, 0.0) + 1e-6 * y) * d
    assert np.all(np.abs(x - xd) <= bound)
    # the block scale keeps |y| <= 6 within the E4M3 rounding of sv (relative 1/16)
    assert np.all(y <= 6.0 * (1 + 1 / 16) + 1e-6)


def test_zero_underflow_nonfinite_and_negative_zero(oracle_lib):
    x = np.zeros((5, 32), np.float32)
    x[1, :16] = np.float32(1e-30)                        # sv underflows E4M3: scale 0, codes 0
    x[2, 3] = np.inf
    x[2, 17] = 1.0
    x[3, 5] = np.nan
    x[4, :16] = -0.0
    x[4, 0] = -np.float32(6.0)                           # sv = 1; other entries -0
    codes, s = oracle_lib.nv_quantize(x, 1.0)
    assert s[0, 0] == 0 and not codes[0].any()
    assert s[1, 0] == 0 and not codes[1, :8].any()
    assert s[2, 0] == 0x7F and not codes[2, :8].any() and s[2, 1] != 0x7F
    assert s[3, 0] == 0x7F and not codes[3, :8].any()
    c4 = datagen.unpack_nibbles(codes)[4, :16]
    assert c4[0] == 15 and not c4[1:].any()              # -6 is code 15; -0 comes out +0


def test_rejects_bad_arguments(oracle_lib):
    x = np.ones((2, 16), np.float32)
    for g in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            oracle_lib.nv_quantize(x, g)
    with pytest.raises(ValueError):
        oracle_lib.nv_quantize(np.ones((2, 24), np.float32), 1.0)


def test_decisions_in_fp32(oracle_lib):
    # amax chosen so that amax / (6 g) lands within one fp32 ulp of a scale midpoint:
    # the fp32 quotient decides the code (the fp64 quotient would decide differently)
    g = np.float32(0.1)
    six_g = np.float32(np.float32(6.0) * g)
    mid = (E4[0x40] + E4[0x41]) / 2                      # between 2.0 and 2.25
    found = False
    for k in range(-40, 41):
        amax = np.float32(np.float64(mid) * np.float64(six_g)) + np.float32(k) * np.spacing(np.float32(mid * six_g))
        sv32 = np.float32(amax / six_g)
        sv64 = np.float64(amax) / (6.0 * np.float64(g))
        if (sv32 == mid) != (sv64 == mid) or ((sv32 > mid) != (sv64 > mid)):
            x = np.zeros((1, 16), np.float32)
            x[0, 0] = amax
            _, s = oracle_lib.nv_quantize(x, g)
            want = 0x40 if sv32 < mid else (0x41 if sv32 > mid else 0x40)
            assert s[0, 0] == want
            found = True
    assert found, "no amax near the midpoint separates fp32 from fp64"
