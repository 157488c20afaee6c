"""GPU parity of the pre-packed W4A8 path: the re-pack (w4a8_prepack) is a nibble
permutation plus an exact bf16 -> fp32 widening, so it must equal the oracle's layout
bit for bit; the GEMM over it (w4a8_gemm_prepacked) must meet the W4A8 bar against the
oracle's product on the original operands (fp32 |D - D_exact| <= 1e-5 * S, bf16 adds
one bf16 ulp)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def up(d):
    return {"A": torch.from_numpy(d["A"]).to(DEV), "sa": torch.from_numpy(d["sa"]).to(DEV),
            "B": torch.from_numpy(d["B"]).to(DEV),
            "sB": torch.from_numpy(d["sB"].view(np.int16)).to(DEV).view(torch.bfloat16)}


@pytest.mark.parametrize("NK", [(16, 128), (20, 384), (100, 640), (8192, 8192), (777, 2048)])
def test_prepack_matches_oracle(NK):
    N, K = NK
    print(f"case w4a8 prepack {N}x{K}", flush=True)
    d = datagen.make_shape("w4a8", 4, N, K, seed=N + K)
    t = up(d)
    Bp, Sp = fp4.w4a8_prepack(t["B"], t["sB"])
    torch.cuda.synchronize(DEV)
    Bo, So = oracle.w4a8_prepack(d["B"], d["sB"])
    assert np.array_equal(Bp.cpu().numpy(), Bo)
    assert np.array_equal(Sp.cpu().numpy().view(np.uint32), So.view(np.uint32))


def run(d, out_dtype, t=None):
    t = t or up(d)
    Bp, Sp = fp4.w4a8_prepack(t["B"], t["sB"])
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    D = fp4.w4a8_gemm_prepacked(t["A"], t["sa"], Bp, Sp, d["N"], out_dtype=od)
    torch.cuda.synchronize(DEV)
    return D


SHAPES = [(1, 16, 128), (7, 33, 256), (64, 64, 128), (100, 300, 384), (257, 129, 512), (128, 128, 1024),
          (300, 1000, 256), (200, 70, 640), (33, 2000, 1152), (256, 8192, 256)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_prepacked_gemm_matches_oracle(shape, out):
    M, N, K = shape
    print(f"case w4a8 prepacked {M}x{N}x{K} {out}", flush=True)
    d = datagen.make_shape("w4a8", M, N, K, seed=M + 3 * N + K)
    D = run(d, out).float().cpu().numpy().astype(np.float64)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    r = oracle.parity_ratio(D, ref, S, out)
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


def test_int4_extremes():
    """All -8 and all 7 weights, and alternating signs, through both conversion halves."""
    M, N, K = 40, 48, 512
    d = datagen.make_shape("w4a8", M, N, K, seed=9)
    q = np.full((N, K), -8, np.int8)
    q[16:32] = 7
    q[32:] = np.where(np.arange(K) % 2, 7, -8)
    d["B"] = datagen.pack_nibbles(q.view(np.uint8) & np.uint8(15))
    D = run(d, "f32").cpu().numpy().astype(np.float64)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    assert oracle.parity_ratio(D, ref, S, "f32") <= 1.0


def test_workload_size_sampled():
    """256 x 8192 x 8192 (the W4A8 workload) in the launch configuration the benchmark
    times, on sampled outputs: random pairs plus whole rows and columns at tile edges."""
    d = datagen.make("w4a8_256x8192x8192")
    print("case w4a8 prepacked 256x8192x8192 seed 0", flush=True)
    D = run(d, "bf16")
    M, N = 256, 8192
    rng = np.random.default_rng(4)
    ms = np.concatenate([rng.integers(0, M, 20000), np.full(N, 127), np.full(N, 128),
                         np.arange(M), np.arange(M)])
    ns = np.concatenate([rng.integers(0, N, 20000), np.arange(N), np.arange(N),
                         np.full(M, 63), np.full(M, 8191)])
    Dn = D[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    ref, S = oracle.sampled("w4a8", d, ms, ns)
    r = oracle.parity_ratio(Dn, ref, S, "bf16")
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


def test_matches_unpacked_kernel_within_bar():
    d = datagen.make_shape("w4a8", 96, 320, 1024, seed=12)
    t = up(d)
    D1 = run(d, "f32", t).cpu().numpy().astype(np.float64)
    D2 = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    assert oracle.parity_ratio(D1, ref, S, "f32") <= 1.0
    assert oracle.parity_ratio(D2.cpu().numpy().astype(np.float64), ref, S, "f32") <= 1.0


def test_edge_cases():
    A = torch.zeros((0, 128), dtype=torch.uint8, device=DEV)
    sa = torch.zeros(0, dtype=torch.float32, device=DEV)
    Bp, Sp = fp4.w4a8_prepack(torch.zeros((20, 64), dtype=torch.uint8, device=DEV),
                              torch.zeros((20, 1), dtype=torch.bfloat16, device=DEV))
    assert fp4.w4a8_gemm_prepacked(A, sa, Bp, Sp, 20).shape == (0, 20)


# ---- E4M3 group scales (w4a8_prepack_e4m3) ------------------------------------------------
# Every E4M3 value is exactly a bf16 value, so the oracle's W4A8 product with the scales
# written as bf16 bit patterns is the product with E4M3 scales.

def e4m3_as_bf16_bits(codes):
    v = np.array([oracle.e4m3fn(int(c)) for c in codes.ravel()], np.float32).reshape(codes.shape)
    bits = v.view(np.uint32)
    assert not np.any(bits[np.isfinite(v)] & 0xFFFF), "an E4M3 value that bf16 does not hold"
    return (bits >> 16).astype(np.uint16)


def e4m3_scales(N, G, rng):
    """Codes of the workload's scale range (about 0.005 .. 0.05): 0x0A (2^-7 * 1.25) .. 0x1D."""
    return rng.integers(0x0A, 0x1E, (N, G)).astype(np.uint8)


@pytest.mark.parametrize("stride", [1, 8])
@pytest.mark.parametrize("NK", [(16, 128), (100, 640), (777, 2048)])
def test_prepack_e4m3_matches_definition(NK, stride):
    N, K = NK
    G = K // 128
    print(f"case w4a8 prepack e4m3 {N}x{K} stride {stride}", flush=True)
    rng = np.random.default_rng(N + K + stride)
    d = datagen.make_shape("w4a8", 4, N, K, seed=N + K)
    s8 = rng.integers(0, 256, (N, G)).astype(np.uint8)               # every code, NaN and negative included
    packed = np.repeat(s8[:, :, None], 8, axis=2) if stride == 8 else s8
    if stride == 8:
        packed[:, :, 1:] = rng.integers(0, 256, (N, G, 7))             # only the first byte counts
    t = up(d)
    Bp, Sp = fp4.w4a8_prepack_e4m3(t["B"], torch.from_numpy(np.ascontiguousarray(packed)).to(DEV), stride)
    torch.cuda.synchronize(DEV)
    Bo, _ = oracle.w4a8_prepack(d["B"], d["sB"])
    assert np.array_equal(Bp.cpu().numpy(), Bo)
    G16 = -(-N // 16)
    want = np.zeros((G, 16 * G16), np.float32)
    want[:, :N] = np.array([[oracle.e4m3fn(int(c)) for c in row] for row in s8], np.float32).T
    got = Sp.cpu().numpy().reshape(G, 16 * G16)
    nan = np.isnan(want)                                               # codes 0x7F and 0xFF
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))   # -0 included


@pytest.mark.parametrize("stride", [1, 8])
@pytest.mark.parametrize("shape", [(7, 33, 256), (100, 300, 384), (256, 1024, 2048)])
def test_prepacked_gemm_e4m3_scales_matches_oracle(shape, stride):
    M, N, K = shape
    G = K // 128
    print(f"case w4a8 prepacked e4m3 {M}x{N}x{K} stride {stride}", flush=True)
    rng = np.random.default_rng(M + N + K)
    d = datagen.make_shape("w4a8", M, N, K, seed=M + 5 * N + K)
    s8 = e4m3_scales(N, G, rng)
    d["sB"] = e4m3_as_bf16_bits(s8)
    packed = np.ascontiguousarray(np.repeat(s8[:, :, None], 8, axis=2) if stride == 8 else s8)
    t = up(d)
    Bp, Sp = fp4.w4a8_prepack_e4m3(t["B"], torch.from_numpy(packed).to(DEV), stride)
    D = fp4.w4a8_gemm_prepacked(t["A"], t["sa"], Bp, Sp, N, out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    r = oracle.parity_ratio(D.cpu().numpy().astype(np.float64), ref, S, "f32")
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0
