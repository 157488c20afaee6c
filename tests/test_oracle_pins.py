"""Pins for the oracle's products, each against something other than the oracle.

- Exact brute force with fractions.Fraction on tiny shapes, decoding through
  sources independent of oracle.c (a literal E2M1 value list, torch's float8
  decoders for E4M3 / E8M0, numpy sign extension for INT4, torch bf16).
- Special cases that reduce to a textbook product (unit scales => plain GEMM of
  decoded values, checked with numpy's matmul).
- Invariants fixed by the mathematics: doubling one block's scale doubles that
  block's contribution only, sign flip, zero codes, K-split additivity, K-block
  permutation, the transpose identity (page 2: a column-major N x M result has
  the bytes of a row-major M x N one).
- The per-slice scale-block counts the pages state (tests/golden/scale_blocks.json),
  and a straddle case that pins the block index at its boundary.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from datagen import pack_nibbles, random_mx, random_nv, random_w4a8, unpack_nibbles

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
E8M0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "scale_blocks.json")


def _int4(n):
    return int(((np.uint8(n) << 4).astype(np.uint8).view(np.int8)) >> 4)


def _bf16(u):
    return float(torch.tensor([int(u)], dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
                 .to(torch.float64)[0])


# ---- independent exact references -----------------------------------------------------

def exact_fp4(A, sfA, B, sfB, V, scale_table, g=Fraction(1)):
    a = unpack_nibbles(A)
    b = unpack_nibbles(B)
    M, K = a.shape
    N = b.shape[0]
    D = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += (Fraction(E2M1[a[m, k]]) * Fraction(scale_table[sfA[m, k // V]])
                      * Fraction(E2M1[b[n, k]]) * Fraction(scale_table[sfB[n, k // V]]))
            D[m][n] = s * g
    return D


def exact_fp4_mag(A, sfA, B, sfB, V, scale_table, g=Fraction(1)):
    """S = sum_k |a_hat * b_hat| * |g| for the block-scaled FP4 product, exactly."""
    a = unpack_nibbles(A)
    b = unpack_nibbles(B)
    M, K = a.shape
    N = b.shape[0]
    return [[sum((abs(Fraction(E2M1[a[m, k]]) * Fraction(scale_table[sfA[m, k // V]])
                      * Fraction(E2M1[b[n, k]]) * Fraction(scale_table[sfB[n, k // V]]))
                  for k in range(K)), Fraction(0)) * abs(g)
             for n in range(N)] for m in range(M)]


def exact_w4a8(A, sa, B, sB, magnitude=False):
    """D (or, with magnitude=True, S = the same sum over |every factor|), exactly."""
    q = unpack_nibbles(B)
    M, K = A.shape
    N = q.shape[0]
    f = abs if magnitude else (lambda v: v)
    D = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                part = sum((f(Fraction(E4M3[A[m, k]]) * _int4(q[n, k]))
                            for k in range(128 * g, 128 * g + 128)), Fraction(0))
                tot += f(Fraction(_bf16(sB[n, g]))) * part
            D[m][n] = f(Fraction(float(sa[m]))) * tot
    return D


def _assert_exact(D, ref):
    for m in range(len(ref)):
        for n in range(len(ref[0])):
            r = ref[m][n]
            assert Fraction(D[m, n]) == r or abs(Fraction(D[m, n]) - r) <= abs(r) * Fraction(1, 2 ** 52), (m, n)


@pytest.mark.parametrize("K", [32, 64, 128])
@pytest.mark.parametrize("seed", [0, 1])
def test_mx_bruteforce_fraction(oracle_lib, K, seed):
    rng = np.random.default_rng(seed)
    d = random_mx(3, 2, K, rng, exp_lo=120, exp_hi=134)
    D, S = oracle_lib.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"])
    ref = exact_fp4(d["A"], d["sfA"], d["B"], d["sfB"], 32, E8M0)
    # every term is a dyadic rational on a small grid: fp64 must be exact here
    for m in range(3):
        for n in range(2):
            assert Fraction(D[m, n]) == ref[m][n]
    assert np.all(S >= np.abs(D))


@pytest.mark.parametrize("K", [16, 32, 64])
@pytest.mark.parametrize("g", [(1.0, 1.0), (2.0, 0.375), (3.0, -0.5)])
def test_nv_bruteforce_fraction(oracle_lib, K, g):
    rng = np.random.default_rng(K)
    d = random_nv(2, 3, K, rng, gA=g[0], gB=g[1])
    # also use the full finite E4M3 range for the scales, subnormals included, and
    # negative scale codes in B
    d["sfA"] = rng.integers(0, 0x7F, d["sfA"].shape, dtype=np.uint8)
    d["sfB"] = d["sfB"] | (rng.integers(0, 2, d["sfB"].shape, dtype=np.uint8) << 7)
    D, S = oracle_lib.nv_gemm(d["A"], d["sfA"], d["gA"], d["B"], d["sfB"], d["gB"])
    g_exact = Fraction(float(d["gA"])) * Fraction(float(d["gB"]))
    ref = exact_fp4(d["A"], d["sfA"], d["B"], d["sfB"], 16, E4M3, g_exact)
    _assert_exact(D, ref)
    # S carries |gA * gB| and |every scale|: negative scale codes are in sfA's range
    _assert_exact(S, exact_fp4_mag(d["A"], d["sfA"], d["B"], d["sfB"], 16, E4M3, g_exact))
    assert np.all(S >= np.abs(D))


@pytest.mark.parametrize("K", [128, 256])
@pytest.mark.parametrize("signs", ["positive", "negative"])
def test_w4a8_bruteforce_fraction(oracle_lib, K, signs):
    rng = np.random.default_rng(K + 7)
    d = random_w4a8(2, 3, K, rng)
    if signs == "negative":
        # a negative row scale, and group scales of either sign (bf16 sign bit)
        d["sa"][0] = -d["sa"][0]
        d["sB"] = d["sB"] | (rng.integers(0, 2, d["sB"].shape).astype(np.uint16) << 15)
        d["sB"][0, 0] |= 0x8000
    D, S = oracle_lib.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    _assert_exact(D, exact_w4a8(d["A"], d["sa"], d["B"], d["sB"]))
    _assert_exact(S, exact_w4a8(d["A"], d["sa"], d["B"], d["sB"], magnitude=True))
    assert np.all(S >= np.abs(D))


def test_e2m1_pair_products_exhaustive(oracle_lib):
    """All 16 x 16 code pairs at K = V with a single nonzero k: D = e2m1(a) * e2m1(b)."""
    K = 32
    a = np.zeros((16, K), np.uint8)
    b = np.zeros((16, K), np.uint8)
    a[:, 5] = np.arange(16)
    b[:, 5] = np.arange(16)
    ones = np.full((16, 1), 127, np.uint8)
    D, S = oracle_lib.mx_gemm(pack_nibbles(a), ones, pack_nibbles(b), ones)
    ref = np.array(E2M1)[:, None] * np.array(E2M1)[None, :]
    assert np.array_equal(D, ref)
    assert np.array_equal(S, np.abs(ref))


# ---- special cases that reduce to a textbook product -----------------------------------

@pytest.mark.parametrize("kind", ["mx", "nv"])
def test_unit_scales_reduce_to_plain_gemm(oracle_lib, kind):
    rng = np.random.default_rng(11)
    M, N, K = 7, 9, 256
    if kind == "mx":
        d = random_mx(M, N, K, rng)
        d["sfA"][:] = 127
        d["sfB"][:] = 127
        D, _ = oracle_lib.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"])
    else:
        d = random_nv(M, N, K, rng)
        d["sfA"][:] = 0x38
        d["sfB"][:] = 0x38
        D, _ = oracle_lib.nv_gemm(d["A"], d["sfA"], 1.0, d["B"], d["sfB"], 1.0)
    a = np.array(E2M1)[unpack_nibbles(d["A"])]
    b = np.array(E2M1)[unpack_nibbles(d["B"])]
    assert np.array_equal(D, a @ b.T)


def test_w4a8_unit_scales_reduce_to_plain_gemm(oracle_lib):
    rng = np.random.default_rng(12)
    d = random_w4a8(5, 6, 256, rng)
    d["sa"][:] = 1.0
    d["sB"][:] = 0x3F80            # bf16 1.0
    D, _ = oracle_lib.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    a = E4M3[d["A"]]
    q = ((unpack_nibbles(d["B"]) << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.float64)
    assert np.array_equal(D, a @ q.T)


# ---- invariants ---------------------------------------------------------------------------

def test_mx_block_doubling_changes_only_that_block(oracle_lib):
    rng = np.random.default_rng(21)
    M, N, K = 4, 5, 256
    d = random_mx(M, N, K, rng)
    D0, _ = oracle_lib.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"])
    m, j = 2, 3
    sf2 = d["sfA"].copy()
    sf2[m, j] += 1
    D1, _ = oracle_lib.mx_gemm(d["A"], sf2, d["B"], d["sfB"])
    # contribution of block j of row m: zero every other block of A
    a = unpack_nibbles(d["A"])
    only = np.zeros_like(a)
    only[:, 32 * j:32 * (j + 1)] = a[:, 32 * j:32 * (j + 1)]
    C, _ = oracle_lib.mx_gemm(pack_nibbles(only), d["sfA"], d["B"], d["sfB"])
    expect = D0.copy()
    expect[m] += C[m]
    assert np.array_equal(D1, expect)
    rows = [r for r in range(M) if r != m]
    assert np.array_equal(D1[rows], D0[rows])


def test_nv_block_doubling(oracle_lib):
    rng = np.random.default_rng(22)
    d = random_nv(3, 4, 128, rng)
    D0, _ = oracle_lib.nv_gemm(d["A"], d["sfA"], 1.0, d["B"], d["sfB"], 1.0)
    n, j = 1, 5
    sf2 = d["sfB"].copy()
    sf2[n, j] += 8                # exponent field + 1: exactly twice the value
    assert E4M3[sf2[n, j]] == 2 * E4M3[d["sfB"][n, j]]
    D1, _ = oracle_lib.nv_gemm(d["A"], d["sfA"], 1.0, d["B"], sf2, 1.0)
    b = unpack_nibbles(d["B"])
    only = np.zeros_like(b)
    only[:, 16 * j:16 * (j + 1)] = b[:, 16 * j:16 * (j + 1)]
    C, _ = oracle_lib.nv_gemm(d["A"], d["sfA"], 1.0, pack_nibbles(only), d["sfB"], 1.0)
    expect = D0.copy()
    expect[:, n] += C[:, n]
    assert np.array_equal(D1, expect)


def test_w4a8_group_scale_doubling(oracle_lib):
    rng = np.random.default_rng(23)
    d = random_w4a8(3, 4, 384, rng)
    D0, _ = oracle_lib.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    n, g = 2, 1
    sB2 = d["sB"].copy()
    sB2[n, g] += 0x80             # bf16 exponent + 1
    D1, _ = oracle_lib.w4a8_gemm(d["A"], d["sa"], d["B"], sB2)
    q = unpack_nibbles(d["B"])
    only = np.zeros_like(q)
    only[:, 128 * g:128 * (g + 1)] = q[:, 128 * g:128 * (g + 1)]
    C, _ = oracle_lib.w4a8_gemm(d["A"], d["sa"], pack_nibbles(only), d["sB"])
    expect = D0.copy()
    expect[:, n] += C[:, n]
    np.testing.assert_allclose(D1, expect, rtol=2 ** -50, atol=0)
    others = [c for c in range(4) if c != n]
    assert np.array_equal(D1[:, others], D0[:, others])


def test_w4a8_row_scale_is_a_row_multiplier(oracle_lib):
    rng = np.random.default_rng(24)
    d = random_w4a8(3, 4, 256, rng)
    D0, _ = oracle_lib.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    sa2 = d["sa"].copy()
    sa2[1] *= 4
    D1, _ = oracle_lib.w4a8_gemm(d["A"], sa2, d["B"], d["sB"])
    assert np.array_equal(D1[1], 4 * D0[1])
    assert np.array_equal(D1[[0, 2]], D0[[0, 2]])


def test_sign_flip_and_zero(oracle_lib):
    rng = np.random.default_rng(31)
    d = random_mx(3, 4, 128, rng)
    D0, _ = oracle_lib.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"])
    a = unpack_nibbles(d["A"])
    a[1] ^= 8
    D1, _ = oracle_lib.mx_gemm(pack_nibbles(a), d["sfA"], d["B"], d["sfB"])
    assert np.array_equal(D1[1], -D0[1]) and np.array_equal(D1[[0, 2]], D0[[0, 2]])
    Dz, Sz = oracle_lib.mx_gemm(np.zeros_like(d["A"]), d["sfA"], d["B"], d["sfB"])
    assert not Dz.any() and not Sz.any()


def test_k_split_additivity_and_block_permutation(oracle_lib):
    rng = np.random.default_rng(32)
    M, N, K = 4, 3, 256
    d = random_mx(M, N, K, rng)
    D, _ = oracle_lib.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"])
    h = K // 2
    D1, _ = oracle_lib.mx_gemm(d["A"][:, :h // 2], d["sfA"][:, :h // 32], d["B"][:, :h // 2], d["sfB"][:, :h // 32])
    D2, _ = oracle_lib.mx_gemm(d["A"][:, h // 2:], d["sfA"][:, h // 32:], d["B"][:, h // 2:], d["sfB"][:, h // 32:])
    assert np.array_equal(D, D1 + D2)   # exact: all partial sums are exact dyadics
    perm = rng.permutation(K // 32)
    a = unpack_nibbles(d["A"]).reshape(M, K // 32, 32)[:, perm].reshape(M, K)
    b = unpack_nibbles(d["B"]).reshape(N, K // 32, 32)[:, perm].reshape(N, K)
    Dp, _ = oracle_lib.mx_gemm(pack_nibbles(a), d["sfA"][:, perm], pack_nibbles(b), d["sfB"][:, perm])
    assert np.array_equal(D, Dp)


def test_zero_padding_blocks(oracle_lib):
    rng = np.random.default_rng(33)
    d = random_nv(2, 3, 64, rng)
    D, _ = oracle_lib.nv_gemm(d["A"], d["sfA"], 1.0, d["B"], d["sfB"], 1.0)
    pad = lambda x, s: np.concatenate([x, s], axis=1)
    A2 = pad(d["A"], np.zeros((2, 16), np.uint8))
    B2 = pad(d["B"], np.zeros((3, 16), np.uint8))
    sA2 = pad(d["sfA"], np.full((2, 2), 0x48, np.uint8))
    sB2 = pad(d["sfB"], np.full((3, 2), 0x48, np.uint8))
    D2, _ = oracle_lib.nv_gemm(A2, sA2, 1.0, B2, sB2, 1.0)
    assert np.array_equal(D, D2)


@pytest.mark.parametrize("kind", ["mx", "nv"])
def test_transpose_identity(oracle_lib, kind):
    rng = np.random.default_rng(41)
    gen = random_mx if kind == "mx" else random_nv
    d = gen(5, 7, 128, rng)
    D, S = oracle_lib.run(kind, d)
    sw = dict(d, A=d["B"], sfA=d["sfB"], B=d["A"], sfB=d["sfA"])
    Dt, St = oracle_lib.run(kind, sw)
    assert np.array_equal(D, Dt.T) and np.array_equal(S, St.T)


# ---- scale indexing: the counts the pages state, and the block boundary --------------------

def _influencing_scales(oracle_lib, case):
    """Perturb each scale of one row and count those that change the result."""
    K, k0, kl = case["K"], case["slice_start"], case["slice_k"]
    rng = np.random.default_rng(5)
    op = case["op"]
    if op in ("mx", "nv"):
        V = case["V"]
        gen = random_mx if op == "mx" else random_nv
        d = gen(1, 1, K, rng)
        a = unpack_nibbles(d["A"])
        b = unpack_nibbles(d["B"])
        a[:, :k0] = 0
        a[:, k0 + kl:] = 0
        a[:, k0:k0 + kl] = 2      # 1.0: every element of the slice contributes
        b[:, k0:k0 + kl] = 2
        d["A"], d["B"] = pack_nibbles(a), pack_nibbles(b)
        D0, _ = oracle_lib.run(op, d)
        count = 0
        for j in range(K // V):
            sf = d["sfA"].copy()
            sf[0, j] = sf[0, j] + (1 if op == "mx" else 8)
            D1, _ = oracle_lib.run(op, dict(d, sfA=sf))
            count += int(D1[0, 0] != D0[0, 0])
        return count
    d = random_w4a8(1, 1, K, rng)
    q = unpack_nibbles(d["B"])
    q[:, :k0] = 0
    q[:, k0 + kl:] = 0
    q[:, k0:k0 + kl] = 1
    d["B"] = pack_nibbles(q)
    d["A"][:] = 0x38
    D0, _ = oracle_lib.run("w4a8", d)
    count = 0
    for g in range(K // case["G"]):
        sB = d["sB"].copy()
        sB[0, g] += 0x80
        D1, _ = oracle_lib.run("w4a8", dict(d, sB=sB))
        count += int(D1[0, 0] != D0[0, 0])
    return count


with open(GOLDEN) as _f:
    _CASES = json.load(_f)["cases"]


@pytest.mark.parametrize("case", _CASES, ids=[f"{c['op']}-k{c['slice_k']}" for c in _CASES])
def test_scale_blocks_per_k_slice_match_pages(oracle_lib, case):
    assert _influencing_scales(oracle_lib, case) == case["scales"], case["cite"]


@pytest.mark.parametrize("kind,V", [("mx", 32), ("nv", 16)])
def test_block_boundary_straddle(oracle_lib, kind, V):
    """Nonzero codes only at k = jV-1 and k = jV: they must take scales j-1 and j."""
    K = 4 * V
    j = 2
    a = np.zeros((1, K), np.uint8)
    b = np.zeros((1, K), np.uint8)
    a[0, j * V - 1] = 2
    b[0, j * V - 1] = 2
    a[0, j * V] = 2
    b[0, j * V] = 2
    if kind == "mx":
        sfA = np.array([[127, 128, 130, 127]], np.uint8)   # 1, 2, 8, 1
        sfB = np.full((1, 4), 127, np.uint8)
        D, _ = oracle_lib.mx_gemm(pack_nibbles(a), sfA, pack_nibbles(b), sfB)
        assert D[0, 0] == 2.0 + 8.0
    else:
        sfA = np.array([[0x38, 0x40, 0x50, 0x38]], np.uint8)  # 1, 2, 8, 1
        sfB = np.full((1, 4), 0x38, np.uint8)
        D, _ = oracle_lib.nv_gemm(pack_nibbles(a), sfA, 1.0, pack_nibbles(b), sfB, 1.0)
        assert D[0, 0] == 2.0 + 8.0


def test_nibble_order_low_is_even_k(oracle_lib):
    """The byte 0x72 holds k=0 -> code 2 (1.0) and k=1 -> code 7 (6.0)."""
    A = np.array([[0x72] + [0] * 15], np.uint8)
    Bk0 = np.array([[0x02] + [0] * 15], np.uint8)   # 1.0 at k=0 only
    Bk1 = np.array([[0x20] + [0] * 15], np.uint8)   # 1.0 at k=1 only
    one = np.full((1, 1), 127, np.uint8)
    assert oracle_lib.mx_gemm(A, one, Bk0, one)[0][0, 0] == 1.0
    assert oracle_lib.mx_gemm(A, one, Bk1, one)[0][0, 0] == 6.0


@pytest.mark.parametrize("kind", ["mx", "nv", "w4a8"])
def test_sampled_outputs_equal_full_product(oracle_lib, kind):
    """The sampled entry point evaluates the same definition at chosen (m, n), also
    with negative scales (S must stay the sum of magnitudes)."""
    rng = np.random.default_rng(51)
    if kind == "mx":
        d = random_mx(9, 11, 256, rng)
    elif kind == "nv":
        d = random_nv(9, 11, 256, rng, gA=1.5, gB=-0.25)
        d["sfA"][::2] |= 0x80
    else:
        d = random_w4a8(9, 11, 256, rng)
        d["sa"][::3] *= -1
        d["sB"][1::2] |= 0x8000
    D, S = oracle_lib.run(kind, d)
    ms = rng.integers(0, 9, 40)
    ns = rng.integers(0, 11, 40)
    Ds, Ss = oracle_lib.sampled(kind, d, ms, ns)
    assert np.array_equal(Ds, D[ms, ns]) and np.array_equal(Ss, S[ms, ns])
    assert np.all(Ss >= np.abs(Ds)) and np.all(S >= np.abs(D))
