"""At the workloads' own sizes, the fp64 oracle must equal the exact result.

For MXFP4 and NVFP4 every term a_hat * b_hat is an integer times a fixed power
of two, so the whole product can be computed exactly with integer-valued
matrices: scale each decoded operand to integers (E2M1 x 2 is an integer, E8M0
is a power of two, E4M3 x 2^9 is an integer), multiply the integer matrices in
fp64 BLAS -- exact in any summation order while every partial sum stays below
2^53, which the test asserts from the operand bounds -- and scale back.  This
is a second implementation that shares nothing with oracle.c (decodes come
from a literal E2M1 list and torch's float8 decoders); the oracle must match it
bit for bit.  For W4A8 the exact value at sampled outputs is formed with
Python fractions; the oracle must equal it correctly rounded (only the final
multiply by the fp32 row scale rounds).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
from datagen import unpack_nibbles

E2M1_X2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _int_operand_mx(X, sf):
    """Integer matrix Xi and power p with decoded X = Xi * 2^p."""
    codes = unpack_nibbles(X)
    e = sf.astype(np.int64)
    emin = int(e.min())
    shift = np.repeat(e - emin, 32, axis=1)
    Xi = E2M1_X2[codes] << shift
    return Xi, emin - 127 - 1


def _int_operand_nv(X, sf):
    codes = unpack_nibbles(X)
    s = np.repeat(E4M3[sf] * 512.0, 16, axis=1)         # E4M3 x 2^9: integer-valued
    assert np.array_equal(s, np.round(s))
    Xi = E2M1_X2[codes] * s.astype(np.int64)
    return Xi, -9 - 1


def _exact_product(Ai, pa, Bi, pb):
    K = Ai.shape[1]
    bound = int(np.abs(Ai).max()) * int(np.abs(Bi).max()) * K
    assert bound < 2 ** 53, "integer partial sums would not be exact in fp64"
    return np.ldexp(Ai.astype(np.float64) @ Bi.astype(np.float64).T, pa + pb)


@pytest.mark.parametrize("name,rows", [
    ("mxfp4_256", None),
    ("nvfp4_1024", None),
    ("mxfp4_gemv_8x14336x4096", None),
    ("mxfp4_8192", (4096, 4104)),
])
def test_oracle_equals_exact_integer_product(oracle_lib, name, rows):
    d = datagen.make(name)
    r0, r1 = rows if rows is not None else (0, d["M"])
    if d["kind"] == "nv":
        Ai, pa = _int_operand_nv(d["A"][r0:r1], d["sfA"][r0:r1])
        Bi, pb = _int_operand_nv(d["B"], d["sfB"])
        ref = _exact_product(Ai, pa, Bi, pb) * (float(d["gA"]) * float(d["gB"]))
    else:
        Ai, pa = _int_operand_mx(d["A"][r0:r1], d["sfA"][r0:r1])
        Bi, pb = _int_operand_mx(d["B"], d["sfB"])
        ref = _exact_product(Ai, pa, Bi, pb)
    D, S = oracle_lib.run("nv" if d["kind"] == "nv" else "mx", d, rows=(r0, r1))
    assert np.array_equal(D, ref)
    assert np.all(S >= np.abs(D))


def test_w4a8_oracle_is_exact_then_one_rounding(oracle_lib):
    d = datagen.make("w4a8_256x8192x8192")
    rng = np.random.default_rng(99)
    ms = rng.integers(0, d["M"], 48)
    ns = rng.integers(0, d["N"], 48)
    D, S = oracle_lib.sampled("w4a8", d, ms, ns)
    q = None
    for i, (m, n) in enumerate(zip(ms, ns)):
        a = E4M3[d["A"][m]]
        q = ((unpack_nibbles(d["B"][n:n + 1])[0] << 4).astype(np.uint8).view(np.int8) >> 4)
        parts = (a * 512.0).astype(np.int64).reshape(-1, 128) * q.astype(np.int64).reshape(-1, 128)
        gsum = parts.sum(axis=1)                       # exact integers (x 2^9)
        sB = torch.from_numpy(d["sB"][n].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        tot = sum((Fraction(float(s)) * int(g) for s, g in zip(sB, gsum)), Fraction(0)) / 512
        exact = Fraction(float(d["sa"][m])) * tot
        assert D[i] == float(exact), (m, n)
