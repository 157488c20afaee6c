"""GPU parity of the FP6 re-encoded W4A8 path: the re-pack (w4a8_prepack_fp6) is an
exact re-encoding and re-ordering, so it must equal the oracle's layout bit for bit; the
GEMM over it (w4a8_gemm_prepacked_fp6) must meet the W4A8 bar against the oracle's
product on the original operands: fp32 |D - D_exact| <= 1e-5 * S (bf16 adds one bf16
ulp), plus H, the FP8 instruction's truncation bound for the one-value weight form
(split=False), where the activations span every binade.

Shapes cover token tails (M % 64), weight tails inside a 16-row half, a 32-row block and
a 128-row tile, one and many K groups (odd and even counts), and the 256 x 8192 x 8192
workload in the configuration the benchmark times (sampled outputs)."""
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


@pytest.mark.parametrize("NK", [(16, 128), (32, 256), (40, 384), (100, 640), (777, 2048), (8192, 8192)])
def test_prepack_fp6_matches_oracle(NK):
    N, K = NK
    print(f"case w4a8 prepack fp6 {N}x{K}", flush=True)
    d = datagen.make_shape("w4a8", 4, N, K, seed=N + K)
    t = up(d)
    Bp6, Sp = fp4.w4a8_prepack_fp6(t["B"], t["sB"])
    torch.cuda.synchronize(DEV)
    Bo, So = oracle.w4a8_prepack_fp6(d["B"], d["sB"])
    assert np.array_equal(Bp6.cpu().numpy(), Bo)
    assert np.array_equal(Sp.cpu().numpy().view(np.uint32), So.view(np.uint32))


def run(d, out_dtype, t=None):
    t = t or up(d)
    Bp6, Sp = fp4.w4a8_prepack_fp6(t["B"], t["sB"])
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    D = fp4.w4a8_gemm_prepacked_fp6(t["A"], t["sa"], Bp6, Sp, d["N"], out_dtype=od)
    torch.cuda.synchronize(DEV)
    return D


SHAPES = [(1, 16, 128), (7, 33, 256), (64, 128, 128), (65, 129, 384), (100, 300, 384), (257, 129, 512),
          (128, 128, 1024), (300, 1000, 256), (200, 70, 640), (33, 2000, 1152), (256, 8192, 256),
          (64, 96, 4096), (17, 48, 2176)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_fp6_gemm_matches_oracle(shape, out):
    M, N, K = shape
    print(f"case w4a8 fp6 {M}x{N}x{K} {out}", flush=True)
    d = datagen.make_shape("w4a8", M, N, K, seed=M + 3 * N + K)
    D = run(d, out).float().cpu().numpy().astype(np.float64)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    r = oracle.parity_ratio(D, ref, S, out)
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


def test_int4_extremes():
    """All -8 and all 7 weights, and alternating signs, with negative group scales."""
    M, N, K = 40, 48, 512
    d = datagen.make_shape("w4a8", M, N, K, seed=9)
    q = np.full((N, K), -8, np.int8)
    q[16:32] = 7
    q[32:] = np.where(np.arange(K) % 2, 7, -8)
    d["B"] = datagen.pack_nibbles(q.view(np.uint8) & np.uint8(15))
    d["sB"][::3] |= np.uint16(0x8000)
    D = run(d, "f32").cpu().numpy().astype(np.float64)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    assert oracle.parity_ratio(D, ref, S, "f32") <= 1.0


def test_activations_over_every_binade():
    """E4M3 activations drawn from every finite code: within 1e-5 * S + H, H the
    instruction's truncation for the one-value weight form."""
    M, N, K = 96, 160, 1024
    rng = np.random.default_rng(3)
    d = datagen.make_shape("w4a8", M, N, K, seed=3)
    d["A"] = rng.choice(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8), (M, K))
    H = oracle.fp8_truncation_bound("w4a8", d, split=False)
    D = run(d, "f32").cpu().numpy().astype(np.float64)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    r = oracle.parity_ratio(D, ref, S, "f32", extra=H)
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


def test_workload_size_sampled():
    """256 x 8192 x 8192 (the W4A8 workload) on sampled outputs: random pairs plus whole
    rows and columns at tile edges."""
    d = datagen.make("w4a8_256x8192x8192")
    print("case w4a8 fp6 256x8192x8192 seed 0", flush=True)
    D = run(d, "bf16")
    M, N = 256, 8192
    rng = np.random.default_rng(4)
    ms = np.concatenate([rng.integers(0, M, 20000), np.full(N, 63), np.full(N, 64),
                         np.arange(M), np.arange(M)])
    ns = np.concatenate([rng.integers(0, N, 20000), np.arange(N), np.arange(N),
                         np.full(M, 127), np.full(M, 8191)])
    Dn = D[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    ref, S = oracle.sampled("w4a8", d, ms, ns)
    r = oracle.parity_ratio(Dn, ref, S, "bf16")
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


def test_repeatable():
    d = datagen.make_shape("w4a8", 128, 256, 1152, seed=21)
    t = up(d)
    D1 = run(d, "f32", t)
    D2 = run(d, "f32", t)
    assert torch.equal(D1, D2)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    assert oracle.parity_ratio(D1.cpu().numpy().astype(np.float64), ref, S, "f32") <= 1.0


def test_edge_cases():
    A = torch.zeros((0, 128), dtype=torch.uint8, device=DEV)
    sa = torch.zeros(0, dtype=torch.float32, device=DEV)
    Bp6, Sp = fp4.w4a8_prepack_fp6(torch.zeros((20, 64), dtype=torch.uint8, device=DEV),
                                   torch.zeros((20, 1), dtype=torch.bfloat16, device=DEV))
    assert fp4.w4a8_gemm_prepacked_fp6(A, sa, Bp6, Sp, 20).shape == (0, 20)


# ---- 128 x 128 tiles: the unsplit wide path (tiles fill the GPU) and the K split ----

WIDE = [(2048, 2048, 256), (2100, 2000, 384)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", WIDE, ids=[f"{m}x{n}x{k}" for m, n, k in WIDE])
def test_wide_tiles_full(shape, out):
    """Problems with at least one 128 x 128 tile per CU run the wide kernel unsplit."""
    M, N, K = shape
    print(f"case w4a8 fp6 wide {M}x{N}x{K} {out}", flush=True)
    d = datagen.make_shape("w4a8", M, N, K, seed=M + N + K)
    D = run(d, out).float().cpu().numpy().astype(np.float64)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    r = oracle.parity_ratio(D, ref, S, out)
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


SPLITS = [(64, 200, 2048, 0), (100, 300, 1024, 2), (130, 129, 1536, 3), (256, 512, 4096, 5), (17, 64, 8192, 16),
          (256, 1000, 640, 0)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("case", SPLITS, ids=[f"{m}x{n}x{k}_s{s}" for m, n, k, s in SPLITS])
def test_split(case, out):
    M, N, K, splits = case
    print(f"case w4a8 fp6 split {M}x{N}x{K} splits={splits} {out}", flush=True)
    d = datagen.make_shape("w4a8", M, N, K, seed=M + 5 * N + K)
    t = up(d)
    Bp6, Sp = fp4.w4a8_prepack_fp6(t["B"], t["sB"])
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = fp4.w4a8_gemm_prepacked_fp6_split(t["A"], t["sa"], Bp6, Sp, N, out_dtype=od, splits=splits)
    torch.cuda.synchronize(DEV)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    r = oracle.parity_ratio(D.float().cpu().numpy().astype(np.float64), ref, S, out)
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


def test_split_workload_sampled_and_repeatable():
    """256 x 8192 x 8192 split in two (the library itself does not split it: its 64 x 128
    tiles already give every CU one), sampled; repeated calls agree bit for bit."""
    d = datagen.make("w4a8_256x8192x8192")
    M, N, K = 256, 8192, 8192
    assert fp4.w4a8_fp6_workspace_size(M, N, K) == 0
    assert fp4.w4a8_fp6_workspace_size(M, N, K, 2) == 2 * M * N * 4
    t = up(d)
    Bp6, Sp = fp4.w4a8_prepack_fp6(t["B"], t["sB"])
    D1 = fp4.w4a8_gemm_prepacked_fp6_split(t["A"], t["sa"], Bp6, Sp, N, out_dtype=torch.bfloat16, splits=2)
    D2 = fp4.w4a8_gemm_prepacked_fp6_split(t["A"], t["sa"], Bp6, Sp, N, out_dtype=torch.bfloat16, splits=2)
    torch.cuda.synchronize(DEV)
    assert torch.equal(D1, D2)
    rng = np.random.default_rng(6)
    ms = np.concatenate([rng.integers(0, M, 20000), np.full(N, 127), np.full(N, 128), np.arange(M)])
    ns = np.concatenate([rng.integers(0, N, 20000), np.arange(N), np.arange(N), np.full(M, 8191)])
    Dn = D1[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    ref, S = oracle.sampled("w4a8", d, ms, ns)
    r = oracle.parity_ratio(Dn, ref, S, "bf16")
    print(f"  max |err|/tol = {r:.3f}", flush=True)
    assert r <= 1.0


def test_split_small_workspace_and_wide_activations():
    """A workspace for two slices caps a request for eight; activations over every binade
    stay within 1e-5 * S + H through the split."""
    M, N, K = 96, 160, 2048
    rng = np.random.default_rng(8)
    d = datagen.make_shape("w4a8", M, N, K, seed=8)
    d["A"] = rng.choice(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8), (M, K))
    H = oracle.fp8_truncation_bound("w4a8", d, split=False)
    t = up(d)
    Bp6, Sp = fp4.w4a8_prepack_fp6(t["B"], t["sB"])
    ws = torch.empty(2 * M * N * 4, dtype=torch.uint8, device=DEV)
    D = fp4.w4a8_gemm_prepacked_fp6_split(t["A"], t["sa"], Bp6, Sp, N, out_dtype=torch.float32, splits=8,
                                          workspace=ws)
    torch.cuda.synchronize(DEV)
    ref, S = oracle.w4a8_gemm(d["A"], d["sa"], d["B"], d["sB"])
    assert oracle.parity_ratio(D.cpu().numpy().astype(np.float64), ref, S, "f32", extra=H) <= 1.0
