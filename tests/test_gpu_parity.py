"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (the oracle module's parity rule): fp32 output |D - D_exact| <= 1e-5 * S,
bf16 output <= 1e-5 * S + one bf16 ulp of D_exact, with S = sum_k |a_hat b_hat|.
Full products at sizes the oracle finishes in seconds (several tiles plus ragged
tails); at the workloads' full sizes, in the launch configuration the benchmark
times, sampled outputs (random pairs plus whole rows and columns at the tile
edges) evaluated one by one by the oracle.
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
    t = {}
    for k, v in d.items():
        if not isinstance(v, np.ndarray) or v.ndim == 0:
            continue
        if k == "sB" and v.dtype == np.uint16:       # W4A8 group scales: raw bf16 bits
            t[k] = torch.from_numpy(v.view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            t[k] = torch.from_numpy(v).to(DEV)
    return t


def run(kind, d, out_dtype, t=None):
    t = t or up(d)
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    if kind == "mx":
        D = fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=od)
    elif kind == "gemv":
        D = fp4.fp4_gemv(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=od)
    elif kind == "nv":
        D = fp4.nv_fp4_gemm(t["A"], t["sfA"], float(d["gA"]), t["B"], t["sfB"], float(d["gB"]), out_dtype=od)
    elif kind == "w4a8":
        D = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=od)
    elif kind == "fp8b":
        D = fp4.fp8_blockwise_gemm(t["A"], t["sA"], t["B"], t["sB"], out_dtype=od)
    else:
        raise ValueError(kind)
    torch.cuda.synchronize(DEV)
    return D


def as_np(D):
    return D.float().cpu().numpy().astype(np.float64)


def okind(kind):
    return "mx" if kind == "gemv" else kind


# The FP8 matrix instruction truncates the products of each aligned run of 8 K elements
# below 2^-13 of the run's largest exponent (measured; oracle.fp8_truncation_bound holds
# the model).  The bar of the contractions that run on it is 1e-5 * S plus that bound H,
# computed exactly from the inputs.  The FP8 blockwise GEMM is checked against it
# everywhere; W4A8 on the workload's activation distribution meets 1e-5 * S alone and is
# checked against that, and against 1e-5 * S + H on activations spread over every binade.
def extra_bar(kind, d, ms=None, ns=None):
    if kind == "fp8b":
        return oracle.fp8_truncation_bound(kind, d, ms, ns)
    return None


def check_full(kind, d, out_dtype):
    D = as_np(run(kind, d, out_dtype))
    ref, S = oracle.run(okind(kind), d)
    r = oracle.parity_ratio(D, ref, S, out_dtype, extra=extra_bar(kind, d))
    assert r <= 1.0, f"{kind} {d['M']}x{d['N']}x{d['K']} {out_dtype}: max |err|/tol = {r}"
    return r


def sample_pairs(M, N, rng, count, edges=()):
    ms = list(rng.integers(0, M, count))
    ns = list(rng.integers(0, N, count))
    for m in edges:                       # whole rows at tile edges
        if 0 <= m < M:
            ms += [m] * N
            ns += list(range(N))
    return np.array(ms), np.array(ns)


def check_sampled(kind, d, out_dtype, ms, ns, D=None):
    if D is None:
        D = run(kind, d, out_dtype)
    Dn = as_np(D[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)])
    ref, S = oracle.sampled(okind(kind), d, ms, ns)
    r = oracle.parity_ratio(Dn, ref, S, out_dtype, extra=extra_bar(kind, d, ms, ns))
    assert r <= 1.0, f"{kind} sampled: max |err|/tol = {r}"
    return r


# ---- MXFP4 GEMM ---------------------------------------------------------------------------

def test_mxfp4_256_fp32_full():
    d = datagen.make("mxfp4_256")
    print("case mxfp4_256 seed 0", flush=True)
    check_full("mx", d, "f32")


MX_SHAPES = [(1, 1, 128), (7, 33, 256), (33, 7, 128), (64, 64, 128), (100, 300, 384),
             (255, 257, 256), (257, 129, 512), (128, 128, 1024), (300, 1000, 256), (513, 511, 128)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", MX_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in MX_SHAPES])
def test_mxfp4_shapes(shape, out):
    M, N, K = shape
    d = datagen.make_shape("mx", M, N, K, seed=M + N + K)
    check_full("mx", d, out)


@pytest.mark.parametrize("shape", [(2048, 2048, 256), (2176, 2100, 384)])
def test_mxfp4_mid_tile_config_full(shape):
    M, N, K = shape
    d = datagen.make_shape("mx", M, N, K, seed=5, dist="gaussian")
    check_full("mx", d, "bf16")


@pytest.mark.parametrize("shape", [(4096, 4096, 256), (4100, 4097, 384)])
def test_mxfp4_big_tile_config_sampled(shape):
    M, N, K = shape
    d = datagen.make_shape("mx", M, N, K, seed=7, dist="gaussian")
    rng = np.random.default_rng(1)
    ms, ns = sample_pairs(M, N, rng, 20000, edges=(0, 255, 256, M - 1))
    check_sampled("mx", d, "bf16", ms, ns)
    mt, nt = sample_pairs(N, M, rng, 0, edges=(0, 511, N - 1))   # whole columns
    check_sampled("mx", d, "bf16", nt, mt)


# 256 x 256 tiles with several tiles per workgroup (the next tile's copies go out before
# the epilogue), fp32 panels of 32 columns, and a ragged last column of tiles.
@pytest.mark.parametrize("shape,out", [((4096, 4096, 256), "f32"), ((4352, 8192, 256), "f32"),
                                       ((4352, 8200, 512), "bf16")])
def test_mxfp4_big_tile_multi_item_sampled(shape, out):
    M, N, K = shape
    print(f"case mx {M}x{N}x{K} {out} seed 11", flush=True)
    d = datagen.make_shape("mx", M, N, K, seed=11, dist="gaussian")
    D = run("mx", d, out)
    rng = np.random.default_rng(4)
    ms, ns = sample_pairs(M, N, rng, 20000, edges=(0, 255, 256, M - 1))
    check_sampled("mx", d, out, ms, ns, D=D)
    nt, mt = sample_pairs(N, M, rng, 0, edges=(0, 4095, N - 1))    # whole columns
    check_sampled("mx", d, out, mt, nt, D=D)


def test_mxfp4_headline_config_full_output():
    """The configuration the benchmark times (256 x 256 tiles, 256-element K stages,
    a persistent grid with 4 tiles per workgroup and the per-XCD tile order) compared
    element by element with the oracle over the whole 8192 x 8192 output, fp32 and
    bf16, on workload-distributed inputs (K = 256 keeps the oracle to about 20 s)."""
    M, N, K = 8192, 8192, 256
    print(f"case mx {M}x{N}x{K} full output, seed 31", flush=True)
    d = datagen.make_shape("mx", M, N, K, seed=31, dist="gaussian")
    t = up(d)
    D32 = as_np(run("mx", d, "f32", t))
    D16 = as_np(run("mx", d, "bf16", t))
    ref, S = oracle.run("mx", d)
    for D, out in ((D32, "f32"), (D16, "bf16")):
        r = oracle.parity_ratio(D, ref, S, out)
        print(f"  {out}: max |err|/tol = {r:.3g}", flush=True)
        assert r <= 1.0, f"mx {M}x{N}x{K} {out}: max |err|/tol = {r}"


def test_w4a8_workload_full_output_all_paths():
    """The W4A8 workload (256 x 8192 x 8192) compared element by element with the oracle
    over the whole output for the three W4A8 paths the benchmark times: plain INT4
    weights (the ring kernel), INT4 weights pre-packed by w4a8_prepack, and weights
    re-encoded as FP6 E3M2 by w4a8_prepack_fp6 (64 x 128 tiles, one per CU), fp32 and bf16
    outputs.  One oracle pass (about 20 s on 16 threads) serves all six comparisons."""
    d = datagen.make("w4a8_256x8192x8192")
    M, N, K = d["M"], d["N"], d["K"]
    print(f"case w4a8 {M}x{N}x{K} full output, three paths", flush=True)
    t = up(d)
    Bp, Sp = fp4.w4a8_prepack(t["B"], t["sB"])
    B6, S6 = fp4.w4a8_prepack_fp6(t["B"], t["sB"])
    outs = {}
    for od, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        outs[("plain", name)] = as_np(fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=od))
        outs[("prepacked", name)] = as_np(fp4.w4a8_gemm_prepacked(t["A"], t["sa"], Bp, Sp, N, out_dtype=od))
        outs[("fp6", name)] = as_np(fp4.w4a8_gemm_prepacked_fp6(t["A"], t["sa"], B6, S6, N, out_dtype=od))
    torch.cuda.synchronize(DEV)
    ref, S = oracle.run("w4a8", d)
    for (path, name), D in outs.items():
        r = oracle.parity_ratio(D, ref, S, name)
        print(f"  {path} {name}: max |err|/tol = {r:.3g}", flush=True)
        assert r <= 1.0, f"w4a8 {path} {M}x{N}x{K} {name}: max |err|/tol = {r}"


def test_mxfp4_8192_sampled_and_repeatable():
    d = datagen.make("mxfp4_8192")
    print("case mxfp4_8192 seed 0", flush=True)
    t = up(d)
    D1 = run("mx", d, "bf16", t)
    D2 = run("mx", d, "bf16", t)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16)), "not bitwise repeatable"
    rng = np.random.default_rng(2)
    ms, ns = sample_pairs(8192, 8192, rng, 8192, edges=(0, 4095, 8191))
    check_sampled("mx", d, "bf16", ms, ns, D=D1)
    cols = np.array([0, 300, 8191])
    ms2 = np.repeat(np.arange(8192), len(cols))
    ns2 = np.tile(cols, 8192)
    check_sampled("mx", d, "bf16", ms2, ns2, D=D1)


def test_mxfp4_transpose_identity():
    d = datagen.make_shape("mx", 200, 130, 256, seed=9)
    sw = dict(d, A=d["B"], sfA=d["sfB"], B=d["A"], sfB=d["sfA"], M=130, N=200)
    D = as_np(run("mx", d, "f32"))
    Dt = as_np(run("mx", sw, "f32"))
    ref, S = oracle.run("mx", d)
    assert oracle.parity_ratio(Dt.T, ref, S, "f32") <= 1.0
    assert oracle.parity_ratio(D, ref, S, "f32") <= 1.0


def test_mxfp4_output_guard_rows_untouched():
    M, N, K = 70, 90, 256
    d = datagen.make_shape("mx", M, N, K, seed=10)
    t = up(d)
    buf = torch.full((M + 3, N), float("nan"), dtype=torch.float32, device=DEV)
    out = buf[:M]
    fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out=out)
    torch.cuda.synchronize(DEV)
    assert torch.isfinite(out).all()
    assert torch.isnan(buf[M:]).all()
    ref, S = oracle.run("mx", d)
    assert oracle.parity_ratio(as_np(out), ref, S, "f32") <= 1.0


def test_mxfp4_nan_scale_propagates():
    d = datagen.make_shape("mx", 40, 50, 256, seed=11)
    d["sfA"][3, 2] = 0xFF
    D = as_np(run("mx", d, "f32"))
    ref, S = oracle.run("mx", d)
    assert np.isnan(ref[3]).all()
    assert oracle.parity_ratio(D, ref, S, "f32") <= 1.0


def test_nan_scale_on_every_mxfp4_path():
    """E8M0 0xFF (NaN) in a weight row's block and in a token row's block: the GEMV, the
    GEMV over pre-packed weights and the split-K batched GEMM put NaN exactly where the
    oracle does (the whole token row, the whole weight column) and stay finite elsewhere."""
    M, N, K = 8, 96, 1024
    d = datagen.make_shape("gemv", M, N, K, seed=23)
    d["sfA"][2, 5] = 0xFF
    d["sfB"][17, 30] = 0xFF
    ref, S = oracle.run("mx", d)
    assert np.isnan(ref[2]).all() and np.isnan(ref[:, 17]).all()
    t = up(d)
    outs = {"gemv": fp4.fp4_gemv(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=torch.float32)}
    Bp, Sp = fp4.fp4_gemv_prepack(t["B"], t["sfB"])
    outs["gemv_prepacked"] = fp4.fp4_gemv_prepacked(t["A"], t["sfA"], Bp, Sp, N, out_dtype=torch.float32)
    outs["batched_split"] = fp4.mx_fp4_gemm_batched(*(t[k][None] for k in ("A", "sfA", "B", "sfB")),
                                                    out_dtype=torch.float32, splits=4)[0]
    torch.cuda.synchronize(DEV)
    for name, D in outs.items():
        r = oracle.parity_ratio(as_np(D), ref, S, "f32")
        assert r <= 1.0, f"{name}: {r}"


def test_nan_activation_code_on_fp8_paths():
    """An E4M3 NaN code (0x7F) in one activation row: W4A8 (plain and pre-packed weights)
    and the FP8 blockwise GEMM make that output row NaN, as the oracle does."""
    M, N, K = 40, 72, 512
    d = datagen.make_shape("w4a8", M, N, K, seed=29)
    d["A"][6, 300] = 0x7F
    ref, S = oracle.run("w4a8", d)
    assert np.isnan(ref[6]).all() and np.isfinite(np.delete(ref, 6, axis=0)).all()
    t = up(d)
    Bp, Sp = fp4.w4a8_prepack(t["B"], t["sB"])
    for name, D in (("w4a8", fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=torch.float32)),
                    ("w4a8_prepacked", fp4.w4a8_gemm_prepacked(t["A"], t["sa"], Bp, Sp, N, out_dtype=torch.float32))):
        torch.cuda.synchronize(DEV)
        assert oracle.parity_ratio(as_np(D), ref, S, "f32") <= 1.0, name
    f = datagen.make_shape("fp8b", M, N, K, seed=31)
    f["B"][9, 17] = 0xFF                         # negative NaN code, in a weight row this time
    ref, S = oracle.run("fp8b", f)
    assert np.isnan(ref[:, 9]).all()
    D = as_np(run("fp8b", f, "f32"))
    assert oracle.parity_ratio(D, ref, S, "f32", extra=oracle.fp8_truncation_bound("fp8b", f)) <= 1.0


# ---- GEMV --------------------------------------------------------------------------------

def test_gemv_decode_workload_full():
    d = datagen.make("mxfp4_gemv_8x14336x4096")
    print("case gemv 8x14336x4096 seed 0", flush=True)
    check_full("gemv", d, "bf16")


@pytest.mark.parametrize("M", [17, 32])
def test_gemv_two_token_tiles_workload_weights(M):
    """The decode workload's weight shape (N = 14336, K = 4096) with 17 and 32 tokens:
    the second token tile, every output."""
    d = datagen.make_shape("gemv", M, 14336, 4096, seed=M, dist="gaussian")
    print(f"case gemv {M}x14336x4096", flush=True)
    check_full("gemv", d, "bf16")


def test_gemv_every_token_count_to_32():
    """Each M from 1 to 32 on one shape (lanes whose token is past M are not stored)."""
    for M in range(1, 33):
        d = datagen.make_shape("gemv", M, 70, 1152, seed=300 + M)
        check_full("gemv", d, "f32")


@pytest.mark.parametrize("M", [1, 3, 8, 13, 16, 17, 24, 32])
@pytest.mark.parametrize("NK", [(1, 128), (17, 384), (1000, 256), (4101, 1152)])
def test_gemv_shapes(M, NK):
    N, K = NK
    d = datagen.make_shape("gemv", M, N, K, seed=M * 31 + N)
    check_full("gemv", d, "f32")


@pytest.mark.parametrize("MNK", [(8, 300, 5120), (16, 257, 8192), (5, 130, 14336), (3, 70, 16384),
                                 (8, 40, 16512), (16, 1000, 4096), (1, 33, 12800), (20, 300, 5120),
                                 (32, 257, 8192), (17, 130, 14336), (29, 70, 16384), (32, 1000, 4096),
                                 (16, 8192, 8192), (32, 8192, 6144), (9, 8224, 8192), (16, 8224, 8192),
                                 (1, 8192, 8192), (8, 300, 7296), (24, 1000, 7680), (16, 16416, 8192),
                                 (32, 4100, 8192), (12, 8224, 6144)])
def test_gemv_long_k(MNK):
    # K past one 4096-element pass: segments of 8 and 16 steps per wave, a ragged last
    # segment, K beyond 16384 (the streaming kernel), and the second token tile.  At 4096
    # < K <= 7168, 8 waves, with 32 rows per workgroup for more than 8 tokens while
    # ceil(N / 32) workgroups fit the CUs (N = 8192 of K = 6144) and 16 rows beyond (N = 8224
    # on 256 CUs); at 7168 < K <= 8192, 4 waves of 16 steps, 32 rows for more than 8 tokens
    # while ceil(N / 32) is at most twice the CUs (N = 8192, 4100) and 16 rows beyond
    # (N = 16416 on 256 CUs), with a ragged last segment at K = 7296 and 7680.
    M, N, K = MNK
    d = datagen.make_shape("gemv", M, N, K, seed=M + N + K)
    print(f"case gemv {M}x{N}x{K}", flush=True)
    check_full("gemv", d, "bf16" if N % 2 == 0 else "f32")


def test_gemv_scale_rows_not_16_byte_aligned():
    # Scale pointers need only 4-byte alignment: a view 4 bytes into a buffer takes the
    # per-wave scale loads instead of the whole-line cooperative copy.
    M, N, K = 8, 200, 4096
    d = datagen.make_shape("gemv", M, N, K, seed=77)
    t = up(d)
    buf = torch.zeros(d["sfB"].size + 16, dtype=torch.uint8, device=DEV)
    sfB = buf[4:4 + d["sfB"].size].view(N, K // 32)
    sfB.copy_(t["sfB"])
    assert sfB.data_ptr() % 16 == 4
    D = as_np(fp4.fp4_gemv(t["A"], t["sfA"], t["B"], sfB, out_dtype=torch.float32))
    ref, S = oracle.run("mx", d)
    assert oracle.parity_ratio(D, ref, S, "f32") <= 1.0


@pytest.mark.parametrize("M", [1, 8, 17, 32])
def test_mxfp4_few_tokens_run_the_gemv(M):
    """mx_fp4_gemm with 1 to 32 tokens and K >= 4096 runs the decode GEMV: the result is
    fp4_gemv's bit for bit and meets the bar, and mx_fp4_gemm_batched with L = 1 and the
    automatic split takes the same path without a workspace."""
    N, K = 300, 4096
    d = datagen.make_shape("mx", M, N, K, seed=M, dist="gaussian")
    t = up(d)
    D1 = fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=torch.float32)
    D2 = fp4.fp4_gemv(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=torch.float32)
    D3 = fp4.mx_fp4_gemm_batched(*(t[k][None] for k in ("A", "sfA", "B", "sfB")), out_dtype=torch.float32)[0]
    torch.cuda.synchronize(DEV)
    assert fp4.mx_fp4_gemm_workspace_size(1, M, N, K) == 0
    assert torch.equal(D1, D2) and torch.equal(D1, D3)
    ref, S = oracle.run("mx", d)
    assert oracle.parity_ratio(as_np(D1), ref, S, "f32") <= 1.0


def test_gemv_matches_gemm():
    d = datagen.make_shape("mx", 16, 700, 512, seed=12, dist="gaussian")
    a = as_np(run("gemv", d, "f32"))
    b = as_np(run("mx", d, "f32"))
    ref, S = oracle.run("mx", d)
    assert np.all(np.abs(a - b) <= 2e-5 * S + 1e-30)


# ---- NVFP4 -------------------------------------------------------------------------------

def test_nvfp4_1024_full():
    d = datagen.make("nvfp4_1024")
    print("case nvfp4_1024 seed 0", flush=True)
    check_full("nv", d, "bf16")


NV_SHAPES = [(1, 1, 128), (17, 33, 256), (64, 64, 128), (130, 70, 384), (300, 257, 512), (1100, 1030, 256)]


@pytest.mark.parametrize("g", [(1.0, 1.0), (2.0, 0.375), (3.0, -0.5)])
@pytest.mark.parametrize("shape", NV_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in NV_SHAPES])
def test_nvfp4_shapes(shape, g):
    M, N, K = shape
    rng = np.random.default_rng(M + N)
    d = datagen.random_nv(M, N, K, rng, gA=g[0], gB=g[1])
    d.update({"M": M, "N": N, "K": K})
    check_full("nv", d, "f32")


def test_nvfp4_big_tile_config_full():
    """At least 256 tiles of 128 x 128 select the 4-wave 128 x 128 kernel; K = 384 is an
    odd number of 128-element steps (the register prefetch ends on its second buffer)."""
    M, N, K = 2048, 2112, 384
    print(f"case nv {M}x{N}x{K} seed 21", flush=True)
    d = datagen.random_nv(M, N, K, np.random.default_rng(21), gA=2.0, gB=0.375)
    check_full("nv", d, "bf16")


def test_nvfp4_full_scale_range_including_subnormals():
    rng = np.random.default_rng(13)
    d = datagen.random_nv(96, 80, 256, rng)
    d["sfA"] = rng.integers(0, 0x7F, d["sfA"].shape, dtype=np.uint8)   # every finite positive code
    d["sfB"] = (rng.integers(0, 0x7F, d["sfB"].shape, dtype=np.uint8) | (rng.integers(0, 2, d["sfB"].shape, dtype=np.uint8) << 7))
    d.update({"M": 96, "N": 80, "K": 256})
    check_full("nv", d, "f32")


@pytest.mark.parametrize("case", ["underflow", "overflow"])
def test_nvfp4_global_scales_whose_product_leaves_fp32(case):
    """global_a * global_b below the fp32 normal range (precision lost in a subnormal)
    or past FLT_MAX, while D itself is an ordinary fp32 value: the epilogue applies the
    pair as an fp32 significand product and a power of two, so D keeps the bar."""
    rng = np.random.default_rng(29)
    M, N, K = 64, 80, 256
    d = datagen.random_nv(M, N, K, rng)
    if case == "underflow":
        d["gA"], d["gB"] = np.float32(1.37e-21), np.float32(-2.91e-21)      # product ~ -4e-42
        d["sfA"] = rng.integers(0x60, 0x7F, d["sfA"].shape, dtype=np.uint8)
        d["sfB"] = rng.integers(0x60, 0x7F, d["sfB"].shape, dtype=np.uint8)
    else:
        d["gA"], d["gB"] = np.float32(3.1e25), np.float32(1.6e14)           # product ~ 5e39
        d["sfA"] = rng.integers(0x01, 0x05, d["sfA"].shape, dtype=np.uint8)
        d["sfB"] = rng.integers(0x01, 0x05, d["sfB"].shape, dtype=np.uint8)
        small = np.array([0, 1, 2, 8, 9, 10], np.uint8)                     # |e2m1| <= 1
        d["A"] = datagen.pack_nibbles(rng.choice(small, (M, K)))
        d["B"] = datagen.pack_nibbles(rng.choice(small, (N, K)))
    d.update({"M": M, "N": N, "K": K})
    ref, _ = oracle.run("nv", d)
    assert np.all(np.abs(ref) < 3.0e38) and np.max(np.abs(ref)) > 1.2e-38
    print(f"case nv global scales {case}", flush=True)
    for out in ("f32", "bf16"):
        check_full("nv", d, out)


def test_nvfp4_nan_scale_codes():
    """A NaN scale code (0x7F or 0xFF) makes every product of its block NaN: the
    rows and columns that meet it come out NaN, the rest stay finite."""
    rng = np.random.default_rng(17)
    d = datagen.random_nv(48, 40, 256, rng)
    d["sfA"][3, 2] = 0x7F
    d["sfB"][7, 5] = 0xFF
    d.update({"M": 48, "N": 40, "K": 256})
    D = as_np(run("nv", d, "f32"))
    assert np.isnan(D[3]).all() and np.isnan(D[:, 7]).all()
    assert np.isfinite(np.delete(np.delete(D, 3, axis=0), 7, axis=1)).all()
    check_full("nv", d, "f32")


# ---- W4A8 --------------------------------------------------------------------------------

W4_SHAPES = [(1, 1, 128), (5, 70, 256), (64, 64, 128), (130, 65, 384), (256, 300, 1024), (300, 1000, 512),
             (64, 128, 256), (70, 130, 768), (100, 300, 2048), (256, 512, 4096)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", W4_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in W4_SHAPES])
def test_w4a8_shapes(shape, out):
    M, N, K = shape
    d = datagen.make_shape("w4a8", M, N, K, seed=M + 2 * N + K)
    check_full("w4a8", d, out)


def test_w4a8_workload_sampled():
    d = datagen.make("w4a8_256x8192x8192")
    print("case w4a8 256x8192x8192 seed 0", flush=True)
    rng = np.random.default_rng(3)
    ms, ns = sample_pairs(256, 8192, rng, 4096, edges=(0, 127, 255))
    check_sampled("w4a8", d, "bf16", ms, ns)


def test_w4a8_int4_extremes():
    """All-(-8) and all-7 weights exercise both conversion tables' ends."""
    rng = np.random.default_rng(14)
    d = datagen.make_shape("w4a8", 64, 64, 256, seed=14)
    q = np.where(rng.integers(0, 2, (64, 256)) > 0, 7, 8).astype(np.uint8)
    d["B"] = datagen.pack_nibbles(q)
    check_full("w4a8", d, "f32")


# ---- FP8 blockwise ----------------------------------------------------------------------

F8_SHAPES = [(1, 1, 128), (5, 70, 256), (64, 128, 128), (130, 200, 384), (256, 256, 1024), (300, 257, 512)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", F8_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in F8_SHAPES])
def test_fp8b_shapes(shape, out):
    M, N, K = shape
    d = datagen.make_shape("fp8b", M, N, K, seed=M + 3 * N + K)
    print(f"case fp8b {M}x{N}x{K} {out}", flush=True)
    check_full("fp8b", d, out)


# Shapes with at least one 256 x 128 tile per CU, which take the large-tile kernel:
# ragged in M and N with an odd number of K groups (289 tiles: no per-XCD regrouping),
# a single K group, and 9 tile rows x 32 (288 tiles: the last group of 4 tile rows
# holds one).
F8_BIG = [(4300, 2100, 384, "bf16"), (4096, 2048, 128, "f32"), (2304, 4096, 128, "bf16")]


@pytest.mark.parametrize("shape", F8_BIG, ids=[f"{m}x{n}x{k}-{o}" for m, n, k, o in F8_BIG])
def test_fp8b_big_tile_config_full(shape):
    M, N, K, out = shape
    d = datagen.make_shape("fp8b", M, N, K, seed=M + N + K)
    if out == "f32":                              # scales over many octaves, one negative
        rng = np.random.default_rng(K)
        d["sA"] = (d["sA"] * np.ldexp(1.0, rng.integers(-20, 20, d["sA"].shape))).astype(np.float32)
        d["sB"][1000, 0] = -d["sB"][1000, 0]
    print(f"case fp8b big tiles {M}x{N}x{K} {out}", flush=True)
    check_full("fp8b", d, out)


def test_fp8b_workload_sampled():
    d = datagen.make("fp8_block_4096")
    print("case fp8b 4096^3 seed 0", flush=True)
    rng = np.random.default_rng(5)
    ms, ns = sample_pairs(4096, 4096, rng, 4096, edges=(0, 127, 4095))
    check_sampled("fp8b", d, "bf16", ms, ns)


def test_fp8b_scale_extremes():
    # Scales spanning many octaves and a negative scale: the per-group fp32 multiply
    # must keep each group's weight.
    d = datagen.make_shape("fp8b", 64, 96, 512, seed=9)
    rng = np.random.default_rng(9)
    d["sA"] = (d["sA"] * np.ldexp(1.0, rng.integers(-20, 20, d["sA"].shape))).astype(np.float32)
    d["sB"][3, 1] = -d["sB"][3, 1]
    check_full("fp8b", d, "f32")


# ---- edge cases ----------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["mx", "gemv", "nv", "w4a8"])
def test_empty_k_gives_zeros(kind):
    M, N = 5, 37
    if kind == "w4a8":
        d = {"A": np.zeros((M, 0), np.uint8), "sa": np.ones(M, np.float32),
             "B": np.zeros((N, 0), np.uint8), "sB": np.zeros((N, 0), np.uint16)}
    else:
        V = 16 if kind == "nv" else 32
        d = {"A": np.zeros((M, 0), np.uint8), "sfA": np.zeros((M, 0), np.uint8),
             "B": np.zeros((N, 0), np.uint8), "sfB": np.zeros((N, 0), np.uint8), "gA": 1.0, "gB": 1.0}
    for out in ("f32", "bf16"):
        D = run(kind, d, out)
        assert D.shape == (M, N) and not as_np(D).any()


@pytest.mark.parametrize("kind", ["mx", "nv", "w4a8"])
def test_empty_m(kind):
    d = datagen.make_shape(kind if kind != "w4a8" else "w4a8", 3, 20, 256, seed=1)
    for k in ("A", "sfA", "sa"):
        if k in d:
            d[k] = d[k][:0]
    D = run(kind, d, "bf16")
    assert D.shape == (0, 20)


def test_invalid_calls_raise():
    d = datagen.make_shape("mx", 4, 4, 256, seed=1)
    t = up(d)
    with pytest.raises(fp4.Fp4GemmError):
        fp4.fp4_gemv(torch.zeros((33, 128), dtype=torch.uint8, device=DEV),
                     torch.zeros((33, 8), dtype=torch.uint8, device=DEV), t["B"], t["sfB"])
    with pytest.raises(TypeError):
        fp4.mx_fp4_gemm(t["A"].to(torch.int8), t["sfA"], t["B"], t["sfB"])
    with pytest.raises(ValueError):
        fp4.mx_fp4_gemm(t["A"], t["sfA"][:, :4], t["B"], t["sfB"])
    K = 192
    A = torch.zeros((4, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.zeros((4, K // 32), dtype=torch.uint8, device=DEV)
    with pytest.raises(fp4.Fp4GemmError, match="status 2"):
        fp4.mx_fp4_gemm(A, s, A, s)


# ---- FP8 instruction truncation: activations over every binade --------------------------

FINITE_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def wide_codes(rng, rows, K):
    """E4M3 codes uniform over every finite code: each run of 8 spans many binades."""
    return rng.choice(FINITE_E4M3, (rows, K))


def narrow_codes(rng, rows, K, spread):
    """E4M3 codes whose exponent fields differ by at most `spread` inside each aligned run
    of 8 K elements, while the runs themselves sit anywhere from 2^-6 to 2^8."""
    lo = rng.integers(1, 15 - spread, (rows, K // 8))
    E = np.repeat(lo, 8, axis=1) + rng.integers(0, spread + 1, (rows, K))
    return ((E << 3) | rng.integers(0, 8, (rows, K)) | (rng.integers(0, 2, (rows, K)) << 7)).astype(np.uint8)


def w4a8_both(d, out_dtype):
    """w4a8_gemm and w4a8_gemm_prepacked on the same inputs."""
    t = up(d)
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    D1 = fp4.w4a8_gemm(t["A"], t["sa"], t["B"], t["sB"], out_dtype=od)
    Bp, Sp = fp4.w4a8_prepack(t["B"], t["sB"])
    D2 = fp4.w4a8_gemm_prepacked(t["A"], t["sa"], Bp, Sp, d["N"], out_dtype=od)
    torch.cuda.synchronize(DEV)
    return as_np(D1), as_np(D2)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("K", [256, 384])
def test_w4a8_activations_over_every_binade(K, out):
    """Activation codes spread over all 17 binades inside every run of 8: the FP8
    instruction truncates, and both kernels stay within 1e-5 S + H (K = 256 runs the
    pipelined kernel on the two exact weight parts, K = 384 the kernel that converts each
    weight to one E4M3 value; pre-packed weights always take the pipelined kernel)."""
    M, N = 96, 160
    rng = np.random.default_rng(K + (out == "bf16"))
    d = datagen.make_shape("w4a8", M, N, K, seed=K)
    d["A"] = wide_codes(rng, M, K)
    print(f"case w4a8 wide activations {M}x{N}x{K} {out}", flush=True)
    D1, D2 = w4a8_both(d, out)
    ref, S = oracle.run("w4a8", d)
    H_direct = oracle.fp8_truncation_bound("w4a8", d, split=False)
    H_split = oracle.fp8_truncation_bound("w4a8", d, split=True)
    assert (H_split > 1e-5 * S).any()          # the regime where the bound matters
    r1 = oracle.parity_ratio(D1, ref, S, out, extra=H_split if K % 256 == 0 else H_direct)
    r2 = oracle.parity_ratio(D2, ref, S, out, extra=H_split)
    assert r1 <= 1.0 and r2 <= 1.0, (r1, r2)


@pytest.mark.parametrize("K", [256, 384])
def test_w4a8_narrow_runs_meet_the_plain_bar(K):
    """Activation exponents within 6 binades inside every run of 8 (and anywhere from
    2^-6 to 2^8 across runs): H is zero, so both kernels meet 1e-5 S alone."""
    M, N = 96, 160
    rng = np.random.default_rng(K + 5)
    d = datagen.make_shape("w4a8", M, N, K, seed=K + 5)
    d["A"] = narrow_codes(rng, M, K, 6)
    assert not oracle.fp8_truncation_bound("w4a8", d, split=True).any()
    assert not oracle.fp8_truncation_bound("w4a8", d, split=False).any()
    D1, D2 = w4a8_both(d, "f32")
    ref, S = oracle.run("w4a8", d)
    for D in (D1, D2):
        assert oracle.parity_ratio(D, ref, S, "f32") <= 1.0


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fp8b_operands_over_every_binade(out):
    M, N, K = 200, 130, 384
    rng = np.random.default_rng(77)
    d = datagen.make_shape("fp8b", M, N, K, seed=77)
    d["A"] = wide_codes(rng, M, K)
    d["B"] = wide_codes(rng, N, K)
    ref, S = oracle.run("fp8b", d)
    assert (oracle.fp8_truncation_bound("fp8b", d) > 1e-5 * S).any()
    print(f"case fp8b wide operands {M}x{N}x{K} {out}", flush=True)
    check_full("fp8b", d, out)


def test_fp8b_narrow_runs_meet_the_plain_bar():
    M, N, K = 200, 130, 384
    rng = np.random.default_rng(78)
    d = datagen.make_shape("fp8b", M, N, K, seed=78)
    d["A"] = narrow_codes(rng, M, K, 3)
    d["B"] = narrow_codes(rng, N, K, 3)
    assert not oracle.fp8_truncation_bound("fp8b", d).any()
    D = as_np(run("fp8b", d, "f32"))
    ref, S = oracle.run("fp8b", d)
    assert oracle.parity_ratio(D, ref, S, "f32") <= 1.0
