"""Maximum sizes: outputs and inputs past 2^31 elements, where every offset must be
64-bit.  Inputs are generated on the device; the oracle sees only the rows that the
sampled outputs need, and is checked at points spread over the whole output,
including its last rows and columns (offsets above 2^31)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def rand_u8(shape, lo=0, hi=256, seed=0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randint(lo, hi, shape, dtype=torch.uint8, device=DEV, generator=g)


def sampled_check(A, sA, B, sB, D, ms, ns, out_dtype):
    """Oracle on the sampled pairs, from host copies of only the rows involved."""
    ur, ir = np.unique(ms, return_inverse=True)
    uc, ic = np.unique(ns, return_inverse=True)
    rows = torch.from_numpy(ur).to(DEV)
    cols = torch.from_numpy(uc).to(DEV)
    d = {"A": A[rows].cpu().numpy(), "sfA": sA[rows].cpu().numpy(),
         "B": B[cols].cpu().numpy(), "sfB": sB[cols].cpu().numpy()}
    ref, S = oracle.sampled("mx", d, ir, ic)
    got = D[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    r = oracle.parity_ratio(got, ref, S, out_dtype)
    assert r <= 1.0, f"max |err|/tol = {r}"


def spread(M, N, count, rng):
    ms = np.concatenate([rng.integers(0, M, count), [M - 1, M - 1, 0, M // 2], np.full(64, M - 1)])
    ns = np.concatenate([rng.integers(0, N, count), [N - 1, 0, N - 1, N - 1], np.arange(N - 64, N)])
    return ms.astype(np.int64), ns.astype(np.int64)


def test_gemm_output_past_2_to_31_elements():
    M = N = 46400                                 # M * N = 2.15e9 > 2^31
    K = 128
    print(f"case large mx_fp4_gemm {M}x{N}x{K}", flush=True)
    A, B = rand_u8((M, K // 2), seed=1), rand_u8((N, K // 2), seed=2)
    sA, sB = rand_u8((M, K // 32), 124, 131, seed=3), rand_u8((N, K // 32), 124, 131, seed=4)
    D = fp4.mx_fp4_gemm(A, sA, B, sB, out_dtype=torch.bfloat16)
    torch.cuda.synchronize(DEV)
    rng = np.random.default_rng(5)
    ms, ns = spread(M, N, 3000, rng)
    assert int(ms[-1]) * N + int(ns[-1]) > 2 ** 31
    sampled_check(A, sA, B, sB, D, ms, ns, "bf16")
    del D
    torch.cuda.empty_cache()


def test_gemv_weights_past_2_to_31_bytes():
    M, N, K = 4, (1 << 27) + 37, 128              # 8.6 GB of weights, M * N > 2^29
    print(f"case large fp4_gemv {M}x{N}x{K}", flush=True)
    A, sA = rand_u8((M, K // 2), seed=6), rand_u8((M, K // 32), 124, 131, seed=7)
    B, sB = rand_u8((N, K // 2), seed=8), rand_u8((N, K // 32), 124, 131, seed=9)
    D = fp4.fp4_gemv(A, sA, B, sB, out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    rng = np.random.default_rng(10)
    ms, ns = spread(M, N, 3000, rng)
    sampled_check(A, sA, B, sB, D, ms, ns, "f32")
    del B, sB, D
    torch.cuda.empty_cache()


def test_quantizer_input_past_2_to_31_elements():
    rows, K = 1 << 16, 1 << 16                    # 2^32 fp32 inputs (16 GiB)
    print(f"case large mx_fp4_quantize {rows}x{K}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    X = torch.randn((rows, K), generator=g, device=DEV, dtype=torch.float32)
    codes, scales = fp4.mx_fp4_quantize(X)
    torch.cuda.synchronize(DEV)
    sel = np.array([0, 1, rows // 2, rows - 2, rows - 1])
    idx = torch.from_numpy(sel).to(DEV)
    c_ref, s_ref = oracle.mx_quantize(X[idx].cpu().numpy())
    assert np.array_equal(scales[idx].cpu().numpy(), s_ref)
    assert np.array_equal(codes[idx].cpu().numpy(), c_ref)
    del X, codes, scales
    torch.cuda.empty_cache()


def test_nv_quantizer_input_past_2_to_31_elements():
    rows, K = 1 << 16, 1 << 16                    # 2^32 fp32 inputs (16 GiB)
    print(f"case large nv_fp4_quantize {rows}x{K}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(13)
    X = torch.randn((rows, K), generator=g, device=DEV, dtype=torch.float32)
    gs = float(X.abs().max()) / (448.0 * 6.0)
    codes, scales = fp4.nv_fp4_quantize(X, gs)
    torch.cuda.synchronize(DEV)
    sel = np.array([0, 1, rows // 2, rows - 2, rows - 1])
    idx = torch.from_numpy(sel).to(DEV)
    c_ref, s_ref = oracle.nv_quantize(X[idx].cpu().numpy(), gs)
    assert np.array_equal(scales[idx].cpu().numpy(), s_ref)
    assert np.array_equal(codes[idx].cpu().numpy(), c_ref)
    del X, codes, scales
    torch.cuda.empty_cache()


def far_points(M, N, rng):
    ms, ns = spread(M, N, 2000, rng)
    assert int(ms[-1]) * N + int(ns[-1]) > 2 ** 31
    return ms, ns


def sample_rows(t, ms, ns, a_keys, b_keys):
    ur, ir = np.unique(ms, return_inverse=True)
    uc, ic = np.unique(ns, return_inverse=True)
    rows, cols = torch.from_numpy(ur).to(DEV), torch.from_numpy(uc).to(DEV)
    d = {k: t[k][rows].cpu().numpy() for k in a_keys}
    d.update({k: t[k][cols].cpu().numpy() for k in b_keys})
    return d, ir, ic


def check_points(D, d, kind, ir, ic, ms, ns, extra=None):
    ref, S = oracle.sampled(kind, d, ir, ic)
    got = D[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    r = oracle.parity_ratio(got, ref, S, "bf16", extra=extra)
    assert r <= 1.0, f"max |err|/tol = {r}"


def test_nvfp4_output_past_2_to_31_elements():
    M = N = 46400
    K = 128
    print(f"case large nv_fp4_gemm {M}x{N}x{K}", flush=True)
    t = {"A": rand_u8((M, K // 2), seed=21), "B": rand_u8((N, K // 2), seed=22),
         "sfA": rand_u8((M, K // 16), 0x28, 0x49, seed=23), "sfB": rand_u8((N, K // 16), 0x28, 0x49, seed=24)}
    D = fp4.nv_fp4_gemm(t["A"], t["sfA"], 1.0, t["B"], t["sfB"], 1.0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize(DEV)
    ms, ns = far_points(M, N, np.random.default_rng(25))
    d, ir, ic = sample_rows(t, ms, ns, ("A", "sfA"), ("B", "sfB"))
    check_points(D, d, "nv", ir, ic, ms, ns)
    del D
    torch.cuda.empty_cache()


def w4a8_inputs(M, N, K, seed):
    """The W4A8 workload's distributions, generated on the device: activations N(0,1)
    scaled per row so the row maximum maps to 448, then E4M3 (the codes are the
    inputs, whatever the rounding); INT4 uniform; group scales uniform in [0.005, 0.05).
    (Codes spread evenly over every E4M3 binade are a different regime: there the FP8
    instruction's inexact internal summation exceeds 1e-5 * S.)"""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, device=DEV)
    amax = x.abs().amax(dim=1, keepdim=True)
    A = (x * (448.0 / amax)).to(torch.float8_e4m3fn).view(torch.uint8)
    sa = (amax[:, 0] / 448.0).float()
    B = rand_u8((N, K // 2), seed=seed + 3)
    sB = (torch.rand((N, K // 128), generator=g, device=DEV) * 0.045 + 0.005).to(torch.bfloat16)
    return {"A": A, "sa": sa, "B": B, "sB": sB}


def w4a8_host(t, ms, ns):
    d, ir, ic = sample_rows(t, ms, ns, ("A", "sa"), ("B",))
    cols = torch.from_numpy(np.unique(ns)).to(DEV)
    d["sB"] = t["sB"][cols].view(torch.int16).cpu().numpy().view(np.uint16)
    return d, ir, ic


@pytest.mark.parametrize("packed,K", [(False, 128), (False, 256), (True, 128)],
                         ids=["unpacked-k128", "unpacked-k256", "prepacked"])
def test_w4a8_output_past_2_to_31_elements(packed, K):
    M = N = 46400
    print(f"case large w4a8 {M}x{N}x{K} packed={packed}", flush=True)
    t = w4a8_inputs(M, N, K, 30)
    if packed:
        Bp, Sp = fp4.w4a8_prepack(t["B"], t["sB"])
        D = fp4.w4a8_gemm_prepacked(t["A"], t["sa"], Bp, Sp, N, out_dtype=torch.bfloat16)
    else:
        D = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize(DEV)
    ms, ns = far_points(M, N, np.random.default_rng(31))
    d, ir, ic = w4a8_host(t, ms, ns)
    check_points(D, d, "w4a8", ir, ic, ms, ns)
    del D
    torch.cuda.empty_cache()


def test_fp8_blockwise_output_past_2_to_31_elements():
    M = N = 46400
    K = 128
    print(f"case large fp8_blockwise_gemm {M}x{N}x{K}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(40)
    t = {"A": rand_u8((M, K), 0, 0x77, seed=41), "B": rand_u8((N, K), 0, 0x77, seed=42),
         "sA": torch.rand((M, 1), generator=g, device=DEV) + 0.5,
         "sB": torch.rand((N, 1), generator=g, device=DEV) + 0.5}
    D = fp4.fp8_blockwise_gemm(t["A"], t["sA"], t["B"], t["sB"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize(DEV)
    ms, ns = far_points(M, N, np.random.default_rng(43))
    d, ir, ic = sample_rows(t, ms, ns, ("A", "sA"), ("B", "sB"))
    # codes uniform over 0..0x77 (all binades): the FP8 instruction's truncation bound applies
    check_points(D, d, "fp8b", ir, ic, ms, ns, extra=oracle.fp8_truncation_bound("fp8b", d, ir, ic))
    del D
    torch.cuda.empty_cache()
