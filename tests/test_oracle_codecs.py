"""Pins for the oracle's scalar decoders, against sources other than the oracle.

- E4M3FN and E8M0: every code against torch's own float8 decoders
  (torch.float8_e4m3fn, torch.float8_e8m0fnu), an independent implementation.
- E2M1: the sixteen values written as a literal list (the textbook value set
  of the 4-bit 1-2-1 format: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), plus anchors.
- INT4: numpy int8 sign extension.
- bf16: torch.bfloat16 over all 65536 bit patterns.
"""
import math

import numpy as np
import pytest
import torch

E2M1_LITERAL = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_matches_literal_value_set(oracle_lib):
    got = [oracle_lib.e2m1(c) for c in range(16)]
    assert got == E2M1_LITERAL
    # signs, including negative zero for code 8
    assert [math.copysign(1.0, v) for v in got] == [1.0] * 8 + [-1.0] * 8


def test_e2m1_anchors(oracle_lib):
    vals = [oracle_lib.e2m1(c) for c in range(16)]
    assert max(vals) == 6.0 and min(vals) == -6.0
    assert len({abs(v) for v in vals}) == 8
    assert oracle_lib.e2m1(1) == 0.5          # the only subnormal
    assert oracle_lib.e2m1(2) == 1.0          # exponent field 1 = 2^0
    # only the low nibble matters
    assert oracle_lib.e2m1(0x17) == 6.0


def test_e4m3fn_all_codes_match_torch(oracle_lib):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_lib.e4m3fn(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                     # 0x7F and 0xFF only
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3fn_anchors(oracle_lib):
    assert oracle_lib.e4m3fn(0x38) == 1.0
    assert oracle_lib.e4m3fn(0x7E) == 448.0
    assert oracle_lib.e4m3fn(0x01) == 2.0 ** -9
    assert oracle_lib.e4m3fn(0x28) == 0.25
    assert oracle_lib.e4m3fn(0x48) == 4.0
    pos = [oracle_lib.e4m3fn(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))   # strictly monotone


def test_e8m0_all_codes_match_torch(oracle_lib):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle_lib.e8m0(e) for e in range(256)])
    assert math.isnan(got[255]) and math.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert oracle_lib.e8m0(127) == 1.0
    for e in range(254):
        assert oracle_lib.e8m0(e + 1) == 2.0 * oracle_lib.e8m0(e)


def test_int4_sign_extension(oracle_lib):
    ref = (np.arange(16, dtype=np.uint8) << 4).view(np.int8) >> 4
    got = [oracle_lib.int4(n) for n in range(16)]
    assert got == ref.tolist()
    assert got[7] == 7 and got[8] == -8 and got[15] == -1


def test_bf16_all_patterns_match_torch(oracle_lib):
    pats = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle_lib.bf16(int(u)) for u in pats[::7]])
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan])


@pytest.mark.parametrize("bad", [0xFF])
def test_special_codes_propagate_nan(oracle_lib, bad):
    """E8M0 0xFF is NaN; an MX product touching it is NaN in that row only."""
    rng = np.random.default_rng(3)
    from datagen import random_mx
    d = random_mx(2, 3, 64, rng)
    d["sfA"][1, 0] = bad
    D, S = oracle_lib.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"])
    assert not np.isnan(D[0]).any()
    assert np.isnan(D[1]).all()
