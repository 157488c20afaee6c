"""Pins for the oracle's MX quantizer (fp32 -> E2M1 codes + E8M0 block scales).

The rule (a reading: the pages fix none) is the max-abs rule written out in
oracle.c.  Each pin checks it against something other than the oracle:
- the threshold-count formula of the input generators (a second implementation
  of the same rule, by a different method);
- the scale exponent read straight from the fp32 bit fields of the block maximum;
- exact round trips of values that lie on the E2M1 grid;
- the rounding error bound of round-to-nearest on the grid, and saturation;
- every tie, which must go to the code with an even mantissa bit;
- covariance under scaling by powers of two;
- the zero, non-finite and clamped-exponent blocks.
"""
import numpy as np
import pytest

import datagen

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # E2M1 magnitudes, codes 0..7


def dequant(codes, scales):
    """Value of every element: sign * GRID[magnitude] * 2^(e - 127)."""
    c = datagen.unpack_nibbles(codes).astype(np.int64)
    mag = GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    e = np.repeat(scales.astype(np.int64), 32, axis=1)
    return np.ldexp(mag, e - 127)


@pytest.mark.parametrize("dist", ["normal", "wide", "tiny"])
def test_matches_threshold_formula(oracle_lib, dist):
    rng = np.random.default_rng({"normal": 1, "wide": 2, "tiny": 3}[dist])
    x = rng.standard_normal((16, 256)).astype(np.float32)
    if dist == "wide":
        x *= np.ldexp(1.0, rng.integers(-20, 20, (16, 256))).astype(np.float32)
    if dist == "tiny":
        x *= np.float32(2.0 ** -60)
    c, s = oracle_lib.mx_quantize(x)
    c2, s2 = datagen.quantize_mx(x)
    assert np.array_equal(s, s2)
    assert np.array_equal(c, c2)


def test_exponent_from_bit_fields(oracle_lib):
    rng = np.random.default_rng(4)
    amax = (rng.uniform(1.0, 2.0, 64) * np.ldexp(1.0, rng.integers(-100, 100, 64))).astype(np.float32)
    x = np.zeros((64, 32), np.float32)
    x[:, 5] = -amax
    x[:, 9] = amax * np.float32(0.3)
    _, s = oracle_lib.mx_quantize(x)
    biased = (amax.view(np.uint32) >> 23) & 0xFF          # floor(log2 amax) + 127
    assert np.array_equal(s[:, 0].astype(np.int64), biased.astype(np.int64) - 2)


def test_grid_values_round_trip(oracle_lib):
    rng = np.random.default_rng(5)
    rows = 32
    e = rng.integers(100, 150, rows)
    codes = rng.integers(0, 16, (rows, 32))
    codes[:, 0] = rng.choice([6, 7, 14, 15], rows)        # a magnitude of 4 or 6 fixes the exponent
    codes[codes == 8] = 0                                  # -0 comes back as +0
    x = (GRID[codes & 7] * np.where(codes & 8, -1.0, 1.0) * np.ldexp(1.0, e - 127)[:, None]).astype(np.float32)
    c, s = oracle_lib.mx_quantize(x)
    assert np.array_equal(s[:, 0], e.astype(np.uint8))
    assert np.array_equal(datagen.unpack_nibbles(c), codes.astype(np.uint8))


def test_error_bound_and_saturation(oracle_lib):
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((64, 128)) * np.ldexp(1.0, rng.integers(-5, 5, (64, 1)))).astype(np.float32)
    c, s = oracle_lib.mx_quantize(x)
    dq = dequant(c, s)
    unit = np.ldexp(1.0, np.repeat(s.astype(np.int64), 32, axis=1) - 127)
    y = np.abs(x.astype(np.float64)) / unit                # scaled magnitude, in [0, 8)
    assert y.max() < 8.0
    half_gap = np.where(y < 2.0, 0.25, np.where(y < 4.0, 0.5, 1.0))
    inside = y <= 6.0
    assert np.all(np.abs(dq - x)[inside] <= (half_gap * unit)[inside])
    assert np.all(np.abs(dq)[~inside] == (6.0 * unit)[~inside])     # saturated to +-6


def test_ties_go_to_even_code(oracle_lib):
    # One block with amax = 4 (scale 2^0) holding every midpoint of the grid.
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]                           # the neighbour with mantissa bit 0
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 4.0
    x[0, 1:8] = mids
    x[0, 8:15] = [-v for v in mids]
    c, s = oracle_lib.mx_quantize(x)
    assert s[0, 0] == 127
    got = datagen.unpack_nibbles(c)[0]
    assert list(got[1:8]) == want
    assert list(got[8:15]) == [w | 8 if w else 0 for w in want]


@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_covariance(oracle_lib, k):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((8, 96)).astype(np.float32)
    c0, s0 = oracle_lib.mx_quantize(x)
    c1, s1 = oracle_lib.mx_quantize((x * np.float32(2.0 ** k)).astype(np.float32))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(np.int64), s0.astype(np.int64) + k)


def test_special_blocks(oracle_lib):
    x = np.zeros((5, 32), np.float32)
    x[1, 3] = np.inf
    x[2, 7] = np.nan
    x[2, 8] = 1.0
    x[3, 0] = 4.0
    x[3, 1] = -0.1                                         # rounds to zero: +0, not -0
    x[4, 0] = np.float32(2.0 ** -140)                      # exponent clamps at 0
    c, s = oracle_lib.mx_quantize(x)
    assert s[0, 0] == 127 and not c[0].any()
    assert s[1, 0] == 0xFF and not c[1].any()
    assert s[2, 0] == 0xFF and not c[2].any()
    assert datagen.unpack_nibbles(c)[3, 1] == 0
    assert s[4, 0] == 0
    big = np.full((1, 32), np.float32(3.0e38))
    _, sb = oracle_lib.mx_quantize(big)
    assert sb[0, 0] == 127 + 127 - 2                       # floor(log2 3e38) = 127
