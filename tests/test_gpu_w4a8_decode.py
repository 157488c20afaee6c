"""GPU parity of the W4A8 decode path: with 1 <= M <= 16 tokens and K <= 16384, and with
17 <= M <= 32 tokens, K <= 8192 and K/128 even, w4a8_gemm, w4a8_gemm_batched and
w4a8_gemm_prepacked run the decode kernel (weights in the 16-row slot of the FP8
instruction, tokens padded to one or two 16-token tiles).

Bar: the oracle module's parity rule, fp32 |D - D_exact| <= 1e-5 * S (bf16: plus one
bf16 ulp) on the workload's activation distribution, and 1e-5 * S + H, H the FP8
instruction's truncation bound for the decode kernel's two exact weight parts (split=2:
the subnormal code v * 2^-9 and the sign part), on activations spread over every
binade.  Shapes cover each segment configuration of the kernel
(K <= 4096, <= 8192, <= 16384), ragged K (groups past K inside a wave's segment),
ragged N (row groups past N), both token tiles (every M from 1 to 32), and the
boundaries to the 64-token kernel (M = 33; M = 17 with K = 8320 or K/128 odd;
K = 16512).
"""
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


def as_np(D):
    return D.float().cpu().numpy().astype(np.float64)


def both(d, out, t=None):
    """w4a8_gemm and w4a8_gemm_prepacked on the same inputs."""
    t = t or up(d)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D1 = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=od)
    Bp, Sp = fp4.w4a8_prepack(t["B"], t["sB"])
    D2 = fp4.w4a8_gemm_prepacked(t["A"], t["sa"], Bp, Sp, d["N"], out_dtype=od)
    torch.cuda.synchronize(DEV)
    return as_np(D1), as_np(D2)


def check(d, out, extra=None):
    D1, D2 = both(d, out)
    ref, S = oracle.run("w4a8", d)
    r1 = oracle.parity_ratio(D1, ref, S, out, extra=extra)
    r2 = oracle.parity_ratio(D2, ref, S, out, extra=extra)
    print(f"  max |err|/tol plain {r1:.3f} pre-packed {r2:.3f}", flush=True)
    assert r1 <= 1.0 and r2 <= 1.0, (r1, r2)


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M", [1, 8, 16, 17, 32])
def test_decode_workload_full(M, out):
    """The W4A8 workload's weights (N = K = 8192) with M decode tokens, every output."""
    print(f"case w4a8 decode {M}x8192x8192 {out} seed {M}", flush=True)
    d = datagen.make_shape("w4a8", M, 8192, 8192, seed=M)
    check(d, out)


SHAPES = [(1, 1, 128), (2, 17, 256), (3, 40, 384), (16, 64, 1024), (5, 100, 4096), (9, 33, 4224),
          (16, 300, 6016), (4, 48, 8192), (12, 250, 8320), (16, 129, 12288), (6, 31, 16384),
          (11, 14336, 4096), (17, 40, 256), (20, 100, 4096), (32, 64, 1024), (25, 129, 6144),
          (31, 33, 8192), (18, 300, 2304)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_decode_shapes(shape, out):
    M, N, K = shape
    print(f"case w4a8 decode {M}x{N}x{K} {out}", flush=True)
    d = datagen.make_shape("w4a8", M, N, K, seed=M + 5 * N + K)
    check(d, out)


@pytest.mark.parametrize("M", list(range(1, 33)))
def test_every_token_count(M):
    """Each M from 1 to 32: lanes whose token is past M read token 0 and are not stored
    (from M = 17 in the second token tile)."""
    print(f"case w4a8 decode M={M} 70x1280", flush=True)
    d = datagen.make_shape("w4a8", M, 70, 1280, seed=100 + M)
    check(d, "f32")


@pytest.mark.parametrize("MK", [(32, 1024), (33, 1024), (17, 8192), (17, 8448), (17, 1152), (16, 16512)])
def test_boundaries_to_the_gemm_kernel(MK):
    """M = 33, M = 17 with K = 8448 (66 groups) or K = 1152 (an odd group count) and
    K = 16512 leave the decode kernel; both sides of each boundary meet the bar."""
    M, K = MK
    print(f"case w4a8 decode boundary {M}x96x{K}", flush=True)
    d = datagen.make_shape("w4a8", M, 96, K, seed=M + K)
    check(d, "f32")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("MK", [(16, 1024), (16, 6016), (32, 2048)])
def test_decode_activations_over_every_binade(MK, out):
    """Activation codes spread over all binades inside every run of 8: the instruction
    truncates, and the decode kernel (two exact weight parts, v as a subnormal code)
    stays within 1e-5 S + H."""
    M, K = MK
    N = 96
    rng = np.random.default_rng(K + (out == "bf16"))
    d = datagen.make_shape("w4a8", M, N, K, seed=K + 1)
    d["A"] = rng.choice(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8), (M, K))
    print(f"case w4a8 decode wide activations {M}x{N}x{K} {out}", flush=True)
    ref, S = oracle.run("w4a8", d)
    H = oracle.fp8_truncation_bound("w4a8", d, split=2)
    assert (H > 1e-5 * S).any()               # the regime where the bound matters
    check(d, out, extra=H)


@pytest.mark.parametrize("M", [8, 24])
def test_decode_int4_extremes_and_signed_scales(M):
    """All -8 / 7 weights (both ends of the conversion), negative group and token scales."""
    N, K = 80, 2048
    rng = np.random.default_rng(21)
    d = datagen.make_shape("w4a8", M, N, K, seed=21)
    q = np.where(rng.integers(0, 2, (N, K)) > 0, 7, 8).astype(np.uint8)
    d["B"] = datagen.pack_nibbles(q)
    sB = d["sB"].view(np.uint16).copy()
    sB[::3] ^= 0x8000                         # negative bf16 group scales on every third row
    d["sB"] = sB
    d["sa"] = d["sa"] * np.where(np.arange(M) % 2 == 0, 1.0, -1.0).astype(np.float32)
    check(d, "f32")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("MK", [(8, 4224), (20, 4352)])
def test_decode_batched(MK, out):
    """w4a8_gemm_batched with M <= 32: problem b on grid row b."""
    L, N = 3, 200
    M, K = MK
    print(f"case w4a8 decode batched L={L} {M}x{N}x{K} {out}", flush=True)
    ds = [datagen.make_shape("w4a8", M, N, K, seed=40 + b) for b in range(L)]
    ts = [up(d) for d in ds]
    t = {k: torch.stack([x[k] for x in ts]) for k in ts[0]}
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = as_np(fp4.w4a8_gemm_batched(t["A"], t["sa"], t["B"], t["sB"], out_dtype=od))
    for b, d in enumerate(ds):
        ref, S = oracle.run("w4a8", d)
        assert oracle.parity_ratio(D[b], ref, S, out) <= 1.0


def test_scales_without_vector_alignment():
    """Group scales at an address that is only 4-byte aligned, and a row pitch that is not
    a 16-byte multiple: the kernel's element-wise scale loads."""
    for M, N, K in ((4, 50, 1152), (16, 33, 8192)):
        d = datagen.make_shape("w4a8", M, N, K, seed=N)
        t = up(d)
        G = K // 128
        buf = torch.zeros(N * G + 2, dtype=torch.bfloat16, device=DEV)
        buf[2:] = t["sB"].reshape(-1)
        sB = buf[2:].view(N, G)
        assert sB.data_ptr() % 16 == 4
        D = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], sB, out_dtype=torch.float32)
        ref, S = oracle.run("w4a8", d)
        assert oracle.parity_ratio(as_np(D), ref, S, "f32") <= 1.0


@pytest.mark.parametrize("M", [16, 32])
def test_decode_is_run_to_run_identical(M):
    d = datagen.make_shape("w4a8", M, 1000, 8192, seed=9)
    t = up(d)
    D1 = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32)
    D2 = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    assert torch.equal(D1, D2)

