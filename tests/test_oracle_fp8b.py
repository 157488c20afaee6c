"""Pins for the oracle's FP8 blockwise-scaled GEMM, each against something other than
the oracle: torch's own E4M3 decoder with a numpy GEMM, exact rational arithmetic,
and identities that follow from the definition
  D[m][n] = sum_g sA[m][g] * sB[n][g] * sum_{k in group g} e4m3(A[m][k]) * e4m3(B[n][k]).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen


def e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def test_unit_scales_are_a_plain_gemm(oracle_lib):
    d = datagen.make_shape("fp8b", 9, 11, 384, seed=3)
    ones_a = np.ones_like(d["sA"])
    ones_b = np.ones_like(d["sB"])
    D, _ = oracle_lib.fp8b_gemm(d["A"], ones_a, d["B"], ones_b)
    ref = e4m3_values(d["A"]) @ e4m3_values(d["B"]).T
    assert np.array_equal(D, ref)      # every partial sum is exact in fp64


def test_group_scales_weight_their_own_group(oracle_lib):
    d = datagen.make_shape("fp8b", 4, 6, 512, seed=4)
    a, b = e4m3_values(d["A"]), e4m3_values(d["B"])
    ref = np.zeros((4, 6))
    for g in range(4):
        ks = slice(128 * g, 128 * (g + 1))
        ref += np.outer(d["sA"][:, g].astype(np.float64), d["sB"][:, g].astype(np.float64)) * (a[:, ks] @ b[:, ks].T)
    D, _ = oracle_lib.fp8b_gemm(d["A"], d["sA"], d["B"], d["sB"])
    assert np.allclose(D, ref, rtol=1e-13, atol=0.0)


@pytest.mark.parametrize("signs", ["positive", "negative"])
def test_exact_rational_brute_force(oracle_lib, signs):
    d = datagen.make_shape("fp8b", 2, 3, 256, seed=5)
    if signs == "negative":
        d["sA"][0, 1] *= -1
        d["sB"][1, 0] *= -1
        d["sB"][2, :] *= -1
    a, b = e4m3_values(d["A"]), e4m3_values(d["B"])
    D, S = oracle_lib.fp8b_gemm(d["A"], d["sA"], d["B"], d["sB"])
    for m in range(2):
        for n in range(3):
            exact = Fraction(0)
            mag = Fraction(0)
            for k in range(256):
                g = k // 128
                t = (Fraction(float(d["sA"][m, g])) * Fraction(float(d["sB"][n, g])) *
                     Fraction(a[m, k]) * Fraction(b[n, k]))
                exact += t
                mag += abs(t)
            assert abs(Fraction(D[m, n]) - exact) <= Fraction(1e-14) * mag
            assert abs(Fraction(S[m, n]) - mag) <= Fraction(1e-14) * mag
    assert np.all(S >= np.abs(D))


def test_group_boundary_straddle(oracle_lib):
    A = np.zeros((1, 256), np.uint8)
    B = np.zeros((1, 256), np.uint8)
    A[0, 127], B[0, 127] = 0x40, 0x44     # 2.0 * 3.0 in group 0
    A[0, 128], B[0, 128] = 0x38, 0x48     # 1.0 * 4.0 in group 1
    sA = np.array([[0.5, 3.0]], np.float32)
    sB = np.array([[2.0, 0.25]], np.float32)
    D, S = oracle_lib.fp8b_gemm(A, sA, B, sB)
    assert D[0, 0] == 0.5 * 2.0 * 6.0 + 3.0 * 0.25 * 4.0
    assert S[0, 0] == D[0, 0]


def test_transpose_identity(oracle_lib):
    d = datagen.make_shape("fp8b", 5, 7, 256, seed=6)
    D, S = oracle_lib.fp8b_gemm(d["A"], d["sA"], d["B"], d["sB"])
    Dt, St = oracle_lib.fp8b_gemm(d["B"], d["sB"], d["A"], d["sA"])
    assert np.array_equal(Dt, D.T) and np.array_equal(St, S.T)


@pytest.mark.parametrize("seed", [7, 8])
def test_sampled_equals_full(oracle_lib, seed):
    d = datagen.make_shape("fp8b", 6, 5, 384, seed=seed)
    d["sA"][::2] *= -1            # negative scales: S must stay a sum of magnitudes
    d["sB"][:, 1] *= -1
    D, S = oracle_lib.fp8b_gemm(d["A"], d["sA"], d["B"], d["sB"])
    ms = np.array([0, 5, 3, 2])
    ns = np.array([4, 0, 2, 2])
    Ds, Ss = oracle_lib.sampled("fp8b", d, ms, ns)
    assert np.array_equal(Ds, D[ms, ns]) and np.array_equal(Ss, S[ms, ns])
    assert np.all(Ss >= np.abs(Ds)) and np.all(S >= np.abs(D))
