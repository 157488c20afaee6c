"""Pins for the oracle's NV quantizer (fp32 -> E2M1 codes + E4M3 block scales per 16,
with a caller-supplied fp32 global scale g).

The rule (a reading: the pages fix none) is written out in oracle.c: per 16-element
block, the scale is the E4M3 code nearest to the exact quotient amax / (6 g) (ties to
the even code, saturating at 448), and each element is the E2M1 value nearest to the
exact quotient x / (e4m3(s) g) (ties to the even mantissa bit, saturating at 6, zero
+0).  The oracle takes both quotients in fp64 and argues that this decides every code
exactly.  Each pin checks it against something other than the oracle's own search:
- exact rational arithmetic (fractions.Fraction) on blocks built to sit on, and one
  fp32 ulp either side of, every rounding boundary of both grids, for global scales
  from the subnormal range to near FLT_MAX;
- the E4M3 values printed by the format's definition (0x38 = 1, 0x7E = 448, ...) and
  exact round trips of all 126 positive finite scale codes;
- every midpoint between neighbouring scale codes, which must go to the even code;
- exact round trips of values on the E2M1 grid, and every E2M1 tie;
- the rounding error bound of round-to-nearest on both grids, and saturation;
- the zero, underflowing and non-finite blocks, and negative zero.
"""
from fractions import Fraction

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
    for i in range(400):
        sv = Fraction(float(amax[i])) / (6 * Fraction(float(g)))
        assert s[i, 0] == ref_nearest(sv, E4_EXACT), i
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


# ---- exact rational reference ----------------------------------------------------------

E2M1_EXACT = [Fraction(v) for v in GRID]
E4_EXACT = [Fraction(float(v)) for v in E4]


def ref_nearest(v, grid):
    """Index of the grid value nearest to the Fraction v >= 0 (grid ascending), a tie
    going to the even index; v past the last value saturates to it."""
    if v >= grid[-1]:
        return len(grid) - 1
    return min(range(len(grid)), key=lambda i: (abs(v - grid[i]), i & 1))


def ref_nv_block(xs, g):
    """The rule in exact rational arithmetic, for one 16-element fp32 block."""
    if not np.all(np.isfinite(xs)):
        return 0x7F, [0] * 16
    gq = Fraction(float(g))
    amax = max(abs(Fraction(float(v))) for v in xs)
    s = ref_nearest(amax / (6 * gq), E4_EXACT)
    if E4_EXACT[s] == 0:
        return s, [0] * 16
    d = E4_EXACT[s] * gq
    codes = []
    for v in xs:
        y = Fraction(float(v)) / d
        c = ref_nearest(abs(y), E2M1_EXACT)
        codes.append(c | 8 if (c and y < 0) else c)
    return s, codes


def _f32_around(q, k):
    """fp32 values next to the exact positive rational q: the largest fp32 <= q, the
    smallest >= q, and k more ulps on each side (positive, finite)."""
    if q >= Fraction(float(np.finfo(np.float32).max)):
        return []
    lo = np.float32(float(q))
    while Fraction(float(lo)) > q:
        lo = np.nextafter(lo, np.float32(0))
    while Fraction(float(np.nextafter(lo, np.float32(np.inf)))) <= q:
        lo = np.nextafter(lo, np.float32(np.inf))
    out = []
    v = lo
    for _ in range(k):
        v = np.nextafter(v, np.float32(0))
    for _ in range(2 * k + 2):
        if np.isfinite(v) and v > 0:
            out.append(v)
        v = np.nextafter(v, np.float32(np.inf))
    return out


E2M1_MIDS = [(E2M1_EXACT[i] + E2M1_EXACT[i + 1]) / 2 for i in range(7)]
E4_MIDS = [(E4_EXACT[i] + E4_EXACT[i + 1]) / 2 for i in range(0x7E)]


def _boundary_blocks(rng, g):
    """Blocks whose elements sit on and around E2M1 boundaries of their block scale, and
    blocks whose maximum sits on and around an E4M3 boundary of amax / (6 g)."""
    gq = Fraction(float(g))
    blocks = []
    for s in rng.choice(np.arange(1, 0x7F), 6, replace=False):
        with np.errstate(over="ignore"):
            top = np.float32(float(6 * E4_EXACT[s] * gq))      # amax near 6 e4m3(s) g
        if not (np.isfinite(top) and top > 0):
            continue
        vals = []
        for mu in E2M1_MIDS + E2M1_EXACT[1:7]:
            vals += _f32_around(mu * E4_EXACT[s] * gq, 1)
        vals = [v for v in vals if v <= top]
        rng.shuffle(vals)
        for i in range(0, len(vals), 15):
            blk = np.zeros(16, np.float32)
            part = np.array(vals[i:i + 15], np.float32)
            part *= np.where(rng.integers(0, 2, part.size) == 1, -1, 1).astype(np.float32)
            blk[1:1 + part.size] = part
            blk[0] = top
            blocks.append(blk)
    for j in rng.choice(len(E4_MIDS), 12, replace=False):
        for amax in _f32_around(E4_MIDS[j] * 6 * gq, 2):
            blk = (rng.uniform(-1, 1, 16) * np.float64(amax)).astype(np.float32)
            blk[rng.integers(0, 16)] = amax
            blocks.append(blk)
    return blocks


@pytest.mark.parametrize("g", [1.0, 0.1, 0.37, 3.0e-3, 1.7e-39, 4.0e-43, 2.5e35, 1.0e38, 3.0e38])
def test_decisions_on_exact_quotients(oracle_lib, g):
    """Every scale and code equals the exact rational rule, on blocks built around the
    rounding boundaries of both grids (where a quotient rounded to fp32, or taken
    through an fp32 reciprocal, decides differently), for global scales from the fp32
    subnormal range to past FLT_MAX / 6."""
    g = np.float32(g)
    rng = np.random.default_rng(int(np.float32(g).view(np.uint32)))
    blocks = _boundary_blocks(rng, g)
    assert len(blocks) > 20
    x = np.stack(blocks)
    codes, s = oracle_lib.nv_quantize(x, g)
    c = datagen.unpack_nibbles(codes)
    for i, blk in enumerate(blocks):
        want_s, want_c = ref_nv_block(blk, g)
        assert s[i, 0] == want_s, (i, blk)
        assert list(c[i]) == want_c, (i, blk)


def test_decisions_on_random_blocks(oracle_lib):
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((64, 64)) * np.ldexp(1.0, rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    x[3, :16] = 0.0
    x[5, 16:32] = x[5, 16:32] * np.float32(1e-35)
    for g in (np.float32(np.abs(x).max() / (448 * 6)), np.float32(0.01), np.float32(7.3e-40)):
        codes, s = oracle_lib.nv_quantize(x, g)
        c = datagen.unpack_nibbles(codes)
        for r in range(64):
            for b in range(4):
                want_s, want_c = ref_nv_block(x[r, 16 * b:16 * b + 16], g)
                assert s[r, b] == want_s and list(c[r, 16 * b:16 * b + 16]) == want_c, (g, r, b)


def test_exact_quotient_differs_from_fp32_arithmetic(oracle_lib):
    """The boundary blocks really separate the exact rule from fp32 arithmetic: for
    some elements, x * fl(1 / fl(e4m3(s) g)) and fl(x / fl(e4m3(s) g)) round to other
    E2M1 codes than the exact quotient (so a pin built on them can tell them apart)."""
    differ_recip = differ_div = 0
    for g in (np.float32(0.1), np.float32(0.37), np.float32(3.0e-3)):
        rng = np.random.default_rng(int(g.view(np.uint32)))
        for blk in _boundary_blocks(rng, g):
            s, want = ref_nv_block(blk, g)
            if not E4_EXACT[s]:
                continue
            d32 = np.float32(np.float32(E4[s]) * g)
            inv = np.float32(np.float32(1.0) / d32)
            for v, w in zip(blk, want):
                y1 = Fraction(float(np.float32(v * inv)))
                y2 = Fraction(float(np.float32(v / d32)))
                c1 = ref_nearest(abs(y1), E2M1_EXACT)
                c2 = ref_nearest(abs(y2), E2M1_EXACT)
                differ_recip += int(c1 != (w & 7))
                differ_div += int(c2 != (w & 7))
    assert differ_recip > 0 and differ_div > 0


def test_scale_rule_past_six_g_overflow(oracle_lib):
    """g above FLT_MAX / 6: 6 g is not an fp32 value, but the exact quotient amax / (6 g)
    is an ordinary number, and the scale follows it."""
    g = np.float32(1.0e38)
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = np.float32(3.4e38)
    x[0, 1] = np.float32(-1.0e38)
    codes, s = oracle_lib.nv_quantize(x, g)
    want_s, want_c = ref_nv_block(x[0], g)
    assert 0 < want_s < 0x40 and s[0, 0] == want_s
    assert list(datagen.unpack_nibbles(codes)[0]) == want_c
