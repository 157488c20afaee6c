"""GPU parity of the pre-packed decode weights: the re-pack (fp4_gemv_prepack) is a
byte permutation, so it must equal the oracle's layout bit for bit; the GEMV over the
packed weights (fp4_gemv_prepacked) must meet the MXFP4 bar against the oracle's
product on the original weights (fp32 |D - D_exact| <= 1e-5 * S; bf16 adds one bf16
ulp)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev(d):
    return {k: torch.from_numpy(d[k]).to(DEV) for k in ("A", "sfA", "B", "sfB")}


@pytest.mark.parametrize("NK", [(16, 512), (37, 384), (1, 128), (100, 640), (14336, 4096), (777, 16512)])
def test_prepack_bytes_match_oracle(NK):
    N, K = NK
    print(f"case prepack {N}x{K}", flush=True)
    rng = np.random.default_rng(N * 7 + K)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sfB = rng.integers(0, 256, (N, K // 32), dtype=np.uint8)
    Bp, Sp = fp4.fp4_gemv_prepack(torch.from_numpy(B).to(DEV), torch.from_numpy(sfB).to(DEV))
    torch.cuda.synchronize(DEV)
    Bo, So = oracle.gemv_prepack(B, sfB)
    assert np.array_equal(Bp.cpu().numpy(), Bo)
    assert np.array_equal(Sp.cpu().numpy(), So)


def run_prepacked(d, out_dtype):
    t = to_dev(d)
    Bp, Sp = fp4.fp4_gemv_prepack(t["B"], t["sfB"])
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    D = fp4.fp4_gemv_prepacked(t["A"], t["sfA"], Bp, Sp, d["N"], out_dtype=od)
    torch.cuda.synchronize(DEV)
    return D.float().cpu().numpy().astype(np.float64)


def check(d, out_dtype):
    D = run_prepacked(d, out_dtype)
    ref, S = oracle.run("mx", d)
    r = oracle.parity_ratio(D, ref, S, out_dtype)
    assert r <= 1.0, f"prepacked gemv {d['M']}x{d['N']}x{d['K']} {out_dtype}: max |err|/tol = {r}"


def test_prepacked_decode_workload_full():
    d = datagen.make("mxfp4_gemv_8x14336x4096")
    print("case prepacked gemv 8x14336x4096 seed 0", flush=True)
    check(d, "bf16")


SHAPES = [(1, 16, 128), (3, 37, 384), (5, 200, 640), (8, 1000, 1024), (13, 64, 4096), (16, 130, 2048),
          (8, 48, 8192), (2, 33, 16512), (16, 500, 512), (7, 4000, 1152)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("MNK", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_prepacked_shapes(MNK, out):
    M, N, K = MNK
    print(f"case prepacked gemv {M}x{N}x{K} {out}", flush=True)
    d = datagen.make_shape("gemv", M, N, K, seed=M * 13 + N + K)
    check(d, out)


def test_prepacked_unaligned_token_scales():
    """Token scale rows that are not 16-byte multiples (K % 512 != 0) and a token-scale
    base that is only 4-byte aligned take the per-step scale loads."""
    M, N, K = 6, 96, 1536
    d = datagen.make_shape("gemv", M, N, K, seed=5)
    t = to_dev(d)
    Bp, Sp = fp4.fp4_gemv_prepack(t["B"], t["sfB"])
    big = torch.zeros(M * (K // 32) + 4, dtype=torch.uint8, device=DEV)
    sfA = big[4:].view(M, K // 32)
    sfA.copy_(t["sfA"])
    D = fp4.fp4_gemv_prepacked(t["A"], sfA, Bp, Sp, N, out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    ref, S = oracle.run("mx", d)
    assert oracle.parity_ratio(D.cpu().numpy().astype(np.float64), ref, S, "f32") <= 1.0


def test_prepacked_edge_cases():
    A = torch.zeros((0, 64), dtype=torch.uint8, device=DEV)
    sA = torch.zeros((0, 4), dtype=torch.uint8, device=DEV)
    Bp, Sp = fp4.fp4_gemv_prepack(torch.zeros((20, 64), dtype=torch.uint8, device=DEV),
                                  torch.zeros((20, 4), dtype=torch.uint8, device=DEV))
    assert fp4.fp4_gemv_prepacked(A, sA, Bp, Sp, 20).shape == (0, 20)
    with pytest.raises(fp4.Fp4GemmError):
        fp4.fp4_gemv_prepacked(torch.zeros((17, 64), dtype=torch.uint8, device=DEV),
                               torch.zeros((17, 4), dtype=torch.uint8, device=DEV), Bp, Sp, 20)
