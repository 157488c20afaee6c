"""GPU parity of the NV quantizer (nv_fp4_quantize) against the CPU oracle.

The outputs are bytes (E2M1 codes and E4M3 scales), so the bar is bit-exact.  The rule
rounds exact real quotients (amax / 6g for the scale, x / (e4m3(s) g) for the codes);
the oracle decides them in fp64, the kernel in fp32 with an fp64 fallback near every
rounding boundary, so the boundary blocks below exercise that fallback.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen
import oracle
from tests.test_oracle_nvquant import _boundary_blocks

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def quantize_gpu(x_np, g, dtype=torch.float32):
    X = torch.from_numpy(x_np).to(DEV).to(dtype)
    c, s = fp4.nv_fp4_quantize(X, g)
    torch.cuda.synchronize(DEV)
    return c.cpu().numpy(), s.cpu().numpy()


def inputs(rows, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x *= np.ldexp(1.0, rng.integers(-8, 8, (rows, 1))).astype(np.float32)
    return x


def tensor_scale(x):
    """The global scale that puts the largest block scale near the top of E4M3."""
    return float(np.float32(np.abs(x).max() / (448.0 * 6.0)))


SHAPES = [(1, 16), (3, 48), (257, 1024), (1000, 4096), (64, 8208)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{k}" for r, k in SHAPES])
def test_fp32_matches_oracle(shape):
    rows, K = shape
    x = inputs(rows, K, rows + K)
    print(f"case nv quantize f32 {rows}x{K}", flush=True)
    for g in (tensor_scale(x), 1.0, 0.37, 1e-3):
        c, s = quantize_gpu(x, g)
        c_ref, s_ref = oracle.nv_quantize(x, g)
        assert np.array_equal(s, s_ref), f"scales differ at g={g}"
        assert np.array_equal(c, c_ref), f"codes differ at g={g}"


@pytest.mark.parametrize("shape", [(5, 64), (300, 2048), (1000, 4096)])
def test_bf16_matches_oracle(shape):
    """bf16 inputs: with g derived from them (or 0.37), a few percent of the blocks have
    quotients on or next to an E2M1 boundary, which the kernel settles exactly with a
    fused multiply-add against the boundary."""
    rows, K = shape
    x = inputs(rows, K, 11 * rows)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    xf = xb.float().numpy()                                   # bf16 -> fp32 is exact
    print(f"case nv quantize bf16 {rows}x{K}", flush=True)
    for g in (tensor_scale(xf), 0.37, 1.0, 1e-3):
        c, s = quantize_gpu(x, g, torch.bfloat16)
        c_ref, s_ref = oracle.nv_quantize(xf, g)
        assert np.array_equal(s, s_ref), f"scales differ at g={g}"
        assert np.array_equal(c, c_ref), f"codes differ at g={g}"


def test_special_values_and_boundaries():
    """Non-finite, zero and underflowing blocks; negative zeros; every E4M3 scale code
    and every midpoint between neighbouring codes (ties to even); every E2M1 tie;
    saturation of both the scale (past 448) and the elements (past 6)."""
    E4 = np.array([(c & 7) / 8 * 2.0 ** -6 if c < 8 else (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7)
                   for c in range(0x7F)])
    rows = []
    blk = np.zeros(16, np.float32); blk[3] = np.inf; rows.append(blk)
    blk = np.zeros(16, np.float32); blk[9] = np.nan; rows.append(blk)
    rows.append(np.zeros(16, np.float32))
    rows.append(np.full(16, -0.0, np.float32))
    rows.append(np.full(16, 1e-30, np.float32))                       # scale underflows: zero codes
    for c in range(1, 0x7F):                                           # sv = e4m3(c) exactly
        blk = np.zeros(16, np.float32); blk[5] = 6.0 * E4[c]; blk[6] = -3.0 * E4[c]; rows.append(blk)
    for c in range(0, 0x7E):                                           # sv on every scale midpoint
        blk = np.zeros(16, np.float32); blk[0] = 3.0 * (E4[c] + E4[c + 1]); rows.append(blk)
    blk = np.zeros(16, np.float32); blk[0] = 6.0
    blk[1:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]; blk[8:15] = -blk[1:8]; rows.append(blk)
    blk = np.zeros(16, np.float32); blk[0] = 6 * 500.0; blk[1] = -6 * 500.0; rows.append(blk)   # scale saturates
    blk = np.zeros(16, np.float32); blk[2] = np.float32(3e38); rows.append(blk)
    x = np.stack(rows).astype(np.float32)
    c, s = quantize_gpu(x, 1.0)
    c_ref, s_ref = oracle.nv_quantize(x, 1.0)
    assert np.array_equal(s, s_ref), f"scale rows differ: {np.nonzero((s != s_ref).any(axis=1))[0]}"
    bad = np.nonzero((c != c_ref).any(axis=1))[0]
    assert not len(bad), f"code rows differ: {bad}: gpu {c[bad[:3]]} oracle {c_ref[bad[:3]]} x {x[bad[:3]]}"
    assert s[0, 0] == 0x7F and s[1, 0] == 0x7F and s[2, 0] == 0 and not c[3].any()


@pytest.mark.parametrize("g", [1.0, 0.1, 0.37, 3.0e-3, 1.7e-39, 4.0e-43, 2.5e35, 1.0e38, 3.0e38])
def test_boundary_blocks_match_oracle(g):
    """Blocks on and one fp32 ulp around every rounding boundary of both grids (where
    fp32 arithmetic alone would decide some codes differently from the exact rule),
    for global scales from the fp32 subnormal range to past FLT_MAX / 6."""
    g = np.float32(g)
    print(f"case nv quantize boundary blocks g={g}", flush=True)
    rng = np.random.default_rng(int(g.view(np.uint32)))
    x = np.stack(_boundary_blocks(rng, g))
    for dt in (torch.float32,):
        c, s = quantize_gpu(x, float(g), dt)
        c_ref, s_ref = oracle.nv_quantize(x, g)
        assert np.array_equal(s, s_ref), f"scale rows differ: {np.nonzero(s != s_ref)[0][:5]}"
        bad = np.nonzero((c != c_ref).any(axis=1))[0]
        assert not len(bad), f"code rows differ: {bad[:5]}: gpu {c[bad[:2]]} oracle {c_ref[bad[:2]]}"


def test_random_blocks_wide_range_match_oracle():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((512, 256)) * np.ldexp(1.0, rng.integers(-20, 20, (512, 1)))).astype(np.float32)
    x[3, :16] = 0.0
    x[5, 16:32] *= np.float32(1e-35)
    print("case nv quantize wide-range random blocks", flush=True)
    for g in (tensor_scale(x), 0.01, 7.3e-40, 1.2e38):
        c, s = quantize_gpu(x, g)
        c_ref, s_ref = oracle.nv_quantize(x, g)
        assert np.array_equal(s, s_ref), f"scales differ at g={g}"
        assert np.array_equal(c, c_ref), f"codes differ at g={g}"


def test_workload_size_sampled_rows():
    rows, K = 8192, 8192
    print(f"case nv quantize f32 {rows}x{K} sampled rows", flush=True)
    rng = np.random.default_rng(12)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    g = tensor_scale(x)
    c, s = quantize_gpu(x, g)
    pick = np.concatenate([[0, rows - 1], rng.integers(0, rows, 30)])
    c_ref, s_ref = oracle.nv_quantize(x[pick], g)
    assert np.array_equal(s[pick], s_ref)
    assert np.array_equal(c[pick], c_ref)


def test_quantize_then_nvfp4_gemm():
    """The quantizer's output is the NVFP4 GEMM's operand: quantize activations and
    weights with their tensor scales, multiply with nv_fp4_gemm, and compare with the
    oracle's GEMM of the oracle's quantization (same bytes, so the usual bar)."""
    M, N, K = 96, 160, 512
    rng = np.random.default_rng(21)
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    ga, gb = tensor_scale(a), tensor_scale(b)
    ca, sa = fp4.nv_fp4_quantize(torch.from_numpy(a).to(DEV), ga)
    cb, sb = fp4.nv_fp4_quantize(torch.from_numpy(b).to(DEV), gb)
    D = fp4.nv_fp4_gemm(ca, sa, ga, cb, sb, gb, out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    oa, osa = oracle.nv_quantize(a, ga)
    ob, osb = oracle.nv_quantize(b, gb)
    assert np.array_equal(ca.cpu().numpy(), oa) and np.array_equal(sa.cpu().numpy(), osa)
    d = {"A": oa, "sfA": osa, "B": ob, "sfB": osb, "gA": np.float32(ga), "gB": np.float32(gb), "M": M, "N": N, "K": K}
    ref, S = oracle.run("nv", d)
    assert oracle.parity_ratio(D.cpu().numpy(), ref, S, "f32", oracle.REL_TOL) <= 1.0
    # and the dequantized product tracks the fp64 product of the unquantized inputs
    exact = a.astype(np.float64) @ b.astype(np.float64).T
    rel = np.abs(ref - exact).max() / np.abs(exact).max()
    assert rel < 0.25


def test_rejects_bad_scale():
    x = torch.ones((2, 16), device=DEV)
    for g in (0.0, -1.0, float("inf")):
        with pytest.raises(fp4.Fp4GemmError):
            fp4.nv_fp4_quantize(x, g)
