"""GPU parity of the NVFP4 decode path: with 1 <= M <= 16 tokens and K <= 16384, and
with 17 <= M <= 32 tokens and K <= 8192, nv_fp4_gemm and nv_fp4_gemm_batched run the
decode kernel (weights in the 16-row slot, tokens in one or two 16-token tiles, both
operands folded exactly to fp16, fp32 accumulation).

Bar: the oracle module's parity rule, fp32 |D - D_exact| <= 1e-5 * S (bf16: plus one
bf16 ulp).  Shapes cover each segment configuration of the kernel (K <= 4096, <= 8192,
<= 16384), ragged K (groups past K inside a wave's segment), ragged N (row groups past
N), every M from 1 to 32, and the boundaries to the GEMM kernel (M = 33; M = 17 with
K = 8320; K = 16512);
scales cover every finite E4M3 code (subnormals and negative codes), NaN codes, and
global scales whose product leaves fp32.
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
    return {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(DEV) for k in ("A", "sfA", "B", "sfB")}


def run(d, out):
    t = up(d)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = fp4.nv_fp4_gemm(t["A"], t["sfA"], float(d["gA"]), t["B"], t["sfB"], float(d["gB"]), out_dtype=od)
    torch.cuda.synchronize(DEV)
    return D.float().cpu().numpy().astype(np.float64)


def check(d, out):
    D = run(d, out)
    ref, S = oracle.run("nv", d)
    r = oracle.parity_ratio(D, ref, S, out)
    print(f"  max |err|/tol {r:.3f}", flush=True)
    assert r <= 1.0, r
    return D


def make(M, N, K, seed, gA=1.0, gB=1.0):
    d = datagen.random_nv(M, N, K, np.random.default_rng(seed), gA=gA, gB=gB)
    d.update({"M": M, "N": N, "K": K})
    return d


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M", [1, 8, 16, 17, 32])
def test_decode_8192_full(M, out):
    """M decode tokens against an 8192 x 8192 NVFP4 weight, every output."""
    print(f"case nv decode {M}x8192x8192 {out} seed {M}", flush=True)
    check(make(M, 8192, 8192, M), out)


SHAPES = [(1, 1, 128), (2, 17, 256), (3, 40, 384), (16, 64, 1024), (5, 100, 4096), (9, 33, 4224),
          (16, 300, 6016), (4, 48, 8192), (12, 250, 8320), (16, 129, 12288), (6, 31, 16384),
          (8, 14336, 4096), (17, 40, 256), (20, 100, 4096), (32, 64, 1024), (25, 129, 6144),
          (31, 33, 8192), (18, 300, 2432)]


@pytest.mark.parametrize("g", [(1.0, 1.0), (2.0, -0.375)])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_decode_shapes(shape, g):
    M, N, K = shape
    print(f"case nv decode {M}x{N}x{K} g={g}", flush=True)
    check(make(M, N, K, M + 3 * N + K, *g), "f32")


@pytest.mark.parametrize("M", list(range(1, 33)))
def test_every_token_count(M):
    print(f"case nv decode M={M} 70x1152", flush=True)
    check(make(M, 70, 1152, 200 + M), "bf16")


@pytest.mark.parametrize("MK", [(32, 1024), (33, 1024), (17, 8192), (17, 8320), (16, 16512)])
def test_boundaries_to_the_gemm_kernel(MK):
    M, K = MK
    print(f"case nv decode boundary {M}x96x{K}", flush=True)
    check(make(M, 96, K, M + K), "f32")


@pytest.mark.parametrize("M", [12, 28])
def test_decode_full_scale_range_including_subnormals(M):
    rng = np.random.default_rng(31)
    d = make(M, 80, 2048, 31)
    d["sfA"] = rng.integers(0, 0x7F, d["sfA"].shape, dtype=np.uint8)
    d["sfB"] = (rng.integers(0, 0x7F, d["sfB"].shape, dtype=np.uint8) |
                (rng.integers(0, 2, d["sfB"].shape, dtype=np.uint8) << 7))
    check(d, "f32")


@pytest.mark.parametrize("case", ["underflow", "overflow"])
def test_decode_global_scales_whose_product_leaves_fp32(case):
    rng = np.random.default_rng(37)
    M, N, K = 8, 80, 1024
    d = make(M, N, K, 37)
    if case == "underflow":
        d["gA"], d["gB"] = np.float32(1.37e-21), np.float32(-2.91e-21)
        d["sfA"] = rng.integers(0x60, 0x7F, d["sfA"].shape, dtype=np.uint8)
        d["sfB"] = rng.integers(0x60, 0x7F, d["sfB"].shape, dtype=np.uint8)
    else:
        d["gA"], d["gB"] = np.float32(3.1e25), np.float32(1.6e14)
        d["sfA"] = rng.integers(0x01, 0x05, d["sfA"].shape, dtype=np.uint8)
        d["sfB"] = rng.integers(0x01, 0x05, d["sfB"].shape, dtype=np.uint8)
        small = np.array([0, 1, 2, 8, 9, 10], np.uint8)
        d["A"] = datagen.pack_nibbles(rng.choice(small, (M, K)))
        d["B"] = datagen.pack_nibbles(rng.choice(small, (N, K)))
    ref, _ = oracle.run("nv", d)
    assert np.all(np.abs(ref) < 3.0e38) and np.max(np.abs(ref)) > 1.2e-38
    for out in ("f32", "bf16"):
        check(d, out)


@pytest.mark.parametrize("M", [8, 24])
def test_decode_nan_scale_codes(M):
    """A NaN scale code makes every product of its block NaN: the token rows and weight
    columns that meet it come out NaN, the rest stay finite."""
    d = make(M, 40, 4224, 41)
    d["sfA"][3, 2] = 0x7F
    d["sfB"][7, 5] = 0xFF
    d["sfB"][9, 4223 // 16] = 0x7F       # in the last group: the one a ragged segment re-reads
    D = run(d, "f32")
    assert np.isnan(D[3]).all() and np.isnan(D[:, 7]).all() and np.isnan(D[:, 9]).all()
    keep = np.delete(np.delete(D, 3, axis=0), [7, 9], axis=1)
    assert np.isfinite(keep).all()
    check(d, "f32")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M", [8, 20])
def test_decode_batched(M, out):
    L, N, K = 3, 200, 4224
    print(f"case nv decode batched L={L} {M}x{N}x{K} {out}", flush=True)
    ds = [make(M, N, K, 50 + b, 2.0, 0.5) for b in range(L)]
    t = {k: torch.stack([up(d)[k] for d in ds]) for k in ("A", "sfA", "B", "sfB")}
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = fp4.nv_fp4_gemm_batched(t["A"], t["sfA"], 2.0, t["B"], t["sfB"], 0.5, out_dtype=od)
    D = D.float().cpu().numpy().astype(np.float64)
    for b, d in enumerate(ds):
        ref, S = oracle.run("nv", d)
        assert oracle.parity_ratio(D[b], ref, S, out) <= 1.0


@pytest.mark.parametrize("M", [16, 32])
def test_decode_is_run_to_run_identical(M):
    d = make(M, 1000, 8192, 9)
    t = up(d)
    D1 = fp4.nv_fp4_gemm(t["A"], t["sfA"], 1.0, t["B"], t["sfB"], 1.0, out_dtype=torch.float32)
    D2 = fp4.nv_fp4_gemm(t["A"], t["sfA"], 1.0, t["B"], t["sfB"], 1.0, out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    assert torch.equal(D1, D2)
