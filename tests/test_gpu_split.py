"""GPU parity of the K-split NVFP4 and W4A8 GEMMs (nv_fp4_gemm_split, w4a8_gemm_split,
w4a8_gemm_prepacked_split): every split count, the automatic choice, batches, a
workspace too small for the requested split, and the unsplit fallbacks (the decode
kernels for M <= 16, plain W4A8 weights with K % 256 != 0) against the oracle.

Bar: the oracle module's parity rule, |D - D_exact| <= 1e-5 * S (bf16: plus one ulp);
W4A8 on activations over every binade adds H, the FP8 instruction's truncation bound
for the ring kernel's weight parts (split=True)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def as_np(D):
    torch.cuda.synchronize(DEV)
    return D.float().cpu().numpy().astype(np.float64)


def w4_dev(ds):
    return {"A": torch.stack([dev(d["A"]) for d in ds]), "sa": torch.stack([dev(d["sa"]) for d in ds]),
            "B": torch.stack([dev(d["B"]) for d in ds]),
            "sB": torch.stack([dev(d["sB"].view(np.int16)).view(torch.bfloat16) for d in ds])}


def nv_dev(ds):
    return {k: torch.stack([dev(d[k]) for d in ds]) for k in ("A", "sfA", "B", "sfB")}


def check(D, d, kind, out, extra=None):
    ref, S = oracle.run(kind, d)
    r = oracle.parity_ratio(D, ref, S, out, extra=extra)
    assert r <= 1.0, r
    return r


W4_CASES = [(1, 64, 200, 2048, 0), (1, 40, 130, 1024, 2), (1, 64, 96, 3072, 3), (2, 24, 64, 2048, 5),
            (1, 100, 70, 4096, 16), (1, 17, 512, 8192, 0), (3, 33, 64, 1536, 4)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("case", W4_CASES, ids=[f"L{l}_{m}x{n}x{k}_s{s}" for l, m, n, k, s in W4_CASES])
def test_w4a8_split(case, out):
    L, M, N, K, splits = case
    print(f"case w4a8 split L={L} {M}x{N}x{K} splits={splits} {out}", flush=True)
    ds = [datagen.make_shape("w4a8", M, N, K, seed=7 * b + M + K) for b in range(L)]
    t = w4_dev(ds)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = as_np(fp4.w4a8_gemm_split(t["A"], t["sa"], t["B"], t["sB"], out_dtype=od, splits=splits))
    for b, d in enumerate(ds):
        check(D[b], d, "w4a8", out)
    if L == 1:   # the pre-packed weights through the same split
        Bp, Sp = fp4.w4a8_prepack(t["B"][0], t["sB"][0])
        Dp = as_np(fp4.w4a8_gemm_prepacked_split(t["A"][0], t["sa"][0], Bp, Sp, N, out_dtype=od, splits=splits))
        check(Dp, ds[0], "w4a8", out)


def test_w4a8_split_wide_activations():
    """Activations over every binade: the split ring kernel stays within 1e-5 S + H."""
    M, N, K = 48, 96, 2048
    rng = np.random.default_rng(3)
    d = datagen.make_shape("w4a8", M, N, K, seed=3)
    d["A"] = rng.choice(np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8), (M, K))
    H = oracle.fp8_truncation_bound("w4a8", d, split=True)
    t = w4_dev([d])
    D = as_np(fp4.w4a8_gemm_split(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32, splits=4))
    check(D[0], d, "w4a8", "f32", extra=H)


def test_w4a8_split_small_workspace_and_fallbacks():
    """A workspace that holds two slices caps a request for eight; plain weights with
    K % 256 != 0 and M <= 16 run unsplit (no workspace needed)."""
    M, N, K = 64, 128, 4096
    d = datagen.make_shape("w4a8", M, N, K, seed=11)
    t = w4_dev([d])
    ws = torch.empty(2 * M * N * 4, dtype=torch.uint8, device=DEV)
    D = as_np(fp4.w4a8_gemm_split(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32, splits=8,
                                  workspace=ws))
    check(D[0], d, "w4a8", "f32")
    for (M2, K2) in ((40, 1152), (12, 2048)):
        d2 = datagen.make_shape("w4a8", M2, 96, K2, seed=M2)
        assert (fp4.w4a8_gemm_workspace_size(1, M2, 96, K2, 4) == 0) == (M2 <= 16)
        t2 = w4_dev([d2])
        D2 = as_np(fp4.w4a8_gemm_split(t2["A"], t2["sa"], t2["B"], t2["sB"], out_dtype=torch.float32, splits=4))
        check(D2[0], d2, "w4a8", "f32")


NV_CASES = [(1, 64, 200, 2048, 0), (1, 40, 130, 1024, 2), (1, 64, 96, 3072, 3), (2, 24, 64, 2048, 5),
            (1, 100, 70, 4096, 16), (1, 17, 512, 8192, 0), (1, 300, 260, 1024, 4)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("case", NV_CASES, ids=[f"L{l}_{m}x{n}x{k}_s{s}" for l, m, n, k, s in NV_CASES])
def test_nvfp4_split(case, out):
    L, M, N, K, splits = case
    print(f"case nv split L={L} {M}x{N}x{K} splits={splits} {out}", flush=True)
    rng = np.random.default_rng(M + K)
    ds = []
    for b in range(L):
        d = datagen.random_nv(M, N, K, rng, gA=2.0, gB=-0.375)
        d.update({"M": M, "N": N, "K": K})
        ds.append(d)
    t = nv_dev(ds)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = as_np(fp4.nv_fp4_gemm_split(t["A"], t["sfA"], 2.0, t["B"], t["sfB"], -0.375, out_dtype=od, splits=splits))
    for b, d in enumerate(ds):
        check(D[b], d, "nv", out)


def test_nvfp4_split_global_scales_leaving_fp32():
    """The reduce applies the global pair as the unsplit epilogue does: an fp32
    significand product and a power of two."""
    rng = np.random.default_rng(43)
    M, N, K = 64, 80, 2048
    d = datagen.random_nv(M, N, K, rng)
    d["gA"], d["gB"] = np.float32(1.37e-21), np.float32(-2.91e-21)
    d["sfA"] = rng.integers(0x60, 0x7F, d["sfA"].shape, dtype=np.uint8)
    d["sfB"] = rng.integers(0x60, 0x7F, d["sfB"].shape, dtype=np.uint8)
    d.update({"M": M, "N": N, "K": K})
    t = nv_dev([d])
    D = as_np(fp4.nv_fp4_gemm_split(t["A"], t["sfA"], float(d["gA"]), t["B"], t["sfB"], float(d["gB"]),
                                    out_dtype=torch.float32, splits=4))
    check(D[0], d, "nv", "f32")


def test_split_equals_unsplit_within_the_bar_and_is_repeatable():
    M, N, K = 64, 256, 8192
    d = datagen.make_shape("w4a8", M, N, K, seed=5)
    t = w4_dev([d])
    D1 = fp4.w4a8_gemm_split(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32, splits=4)
    D2 = fp4.w4a8_gemm_split(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32, splits=4)
    D0 = fp4.w4a8_gemm_batched(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    assert torch.equal(D1, D2)
    check(as_np(D0)[0], d, "w4a8", "f32")
    check(as_np(D1)[0], d, "w4a8", "f32")
