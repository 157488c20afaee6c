"""GPU parity of the batched GEMMs: MXFP4 with its split of K (mx_fp4_gemm_batched),
NVFP4 (nv_fp4_gemm_batched) and W4A8 (w4a8_gemm_batched).

Each of the L problems is an independent product, so the oracle is the plain
oracle of that format applied batch by batch; the bar is the format's bar (fp32 output
|D - D_exact| <= 1e-5 * S, bf16 adds one bf16 ulp).  A split of K only changes the
order in which fp32 partial sums are added, so every split must meet the same bar,
and one split run twice must give the same bits.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
KEYS = ("A", "sfA", "B", "sfB")


def batch(L, M, N, K, seed, dist="uniform"):
    ds = [datagen.make_shape("mx", M, N, K, seed=seed + 101 * b, dist=dist) for b in range(L)]
    t = {k: torch.from_numpy(np.stack([d[k] for d in ds])).to(DEV) for k in KEYS}
    return ds, t


def run(t, out_dtype, splits, workspace=None):
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    D = fp4.mx_fp4_gemm_batched(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=od, splits=splits,
                                workspace=workspace)
    torch.cuda.synchronize(DEV)
    return D.float().cpu().numpy().astype(np.float64)


def check(ds, D, out_dtype):
    worst = 0.0
    for b, d in enumerate(ds):
        ref, S = oracle.run("mx", d)
        worst = max(worst, oracle.parity_ratio(D[b], ref, S, out_dtype))
    assert worst <= 1.0, f"max |err|/tol = {worst}"


SHAPES = [(3, 100, 200, 1024), (2, 257, 129, 2048), (4, 64, 64, 512), (1, 33, 300, 640), (5, 1, 7, 256)]


@pytest.mark.parametrize("splits", [1, 0, 2, 3, 8])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"L{l}_{m}x{n}x{k}" for l, m, n, k in SHAPES])
def test_batched_matches_oracle(shape, out, splits):
    L, M, N, K = shape
    print(f"case batched L={L} {M}x{N}x{K} {out} splits={splits}", flush=True)
    ds, t = batch(L, M, N, K, seed=L + M + N + K)
    check(ds, run(t, out, splits), out)


def test_split_is_reproducible_and_differs_only_by_rounding():
    L, M, N, K = 2, 192, 320, 4096
    ds, t = batch(L, M, N, K, seed=9, dist="gaussian")
    D1 = run(t, "f32", 5)
    D2 = run(t, "f32", 5)
    assert np.array_equal(D1, D2)
    D0 = run(t, "f32", 1)
    check(ds, D1, "f32")
    check(ds, D0, "f32")


def test_small_workspace_shrinks_the_split():
    L, M, N, K = 2, 96, 160, 2048
    ds, t = batch(L, M, N, K, seed=13)
    per_split = L * M * N * 4
    for nbytes in (0, per_split, 2 * per_split + 16, 3 * per_split):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        print(f"case batched workspace {nbytes} bytes", flush=True)
        check(ds, run(t, "bf16", 8, workspace=ws), "bf16")


def test_batch_of_one_equals_mx_fp4_gemm():
    M, N, K = 300, 500, 1024
    d = datagen.make_shape("mx", M, N, K, seed=17)
    t = {k: torch.from_numpy(d[k]).to(DEV) for k in KEYS}
    D_plain = fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=torch.float32)
    D_b = fp4.mx_fp4_gemm_batched(*(t[k][None] for k in KEYS), out_dtype=torch.float32, splits=1)
    torch.cuda.synchronize(DEV)
    assert torch.equal(D_plain, D_b[0])


def test_empty_batch_and_zero_k():
    z = torch.empty((0, 4, 64), dtype=torch.uint8, device=DEV)
    zs = torch.empty((0, 4, 4), dtype=torch.uint8, device=DEV)
    D = fp4.mx_fp4_gemm_batched(z, zs, z, zs)
    assert D.shape == (0, 4, 4)
    A = torch.empty((3, 5, 0), dtype=torch.uint8, device=DEV)
    D = fp4.mx_fp4_gemm_batched(A, A, A[:, :2], A[:, :2], out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    assert D.shape == (3, 5, 2) and not D.any()


@pytest.mark.parametrize("shape", [(1, 64, 8192, 8192), (1, 256, 8192, 8192), (4, 128, 2048, 4096)])
def test_skinny_automatic_split_sampled(shape):
    """Skinny problems at full size with the library's own split choice (the
    configuration the benchmark times), checked on sampled outputs of every batch."""
    L, M, N, K = shape
    print(f"case skinny L={L} {M}x{N}x{K} auto split", flush=True)
    ds, t = batch(L, M, N, K, seed=23, dist="gaussian")
    assert fp4.mx_fp4_gemm_workspace_size(L, M, N, K) > 0
    D = run(t, "bf16", 0)
    rng = np.random.default_rng(3)
    for b, d in enumerate(ds):
        ms = np.concatenate([rng.integers(0, M, 3000), np.full(N, M - 1)])
        ns = np.concatenate([rng.integers(0, N, 3000), np.arange(N)])
        ref, S = oracle.sampled("mx", d, ms, ns)
        r = oracle.parity_ratio(D[b][ms, ns], ref, S, "bf16")
        assert r <= 1.0, f"batch {b}: max |err|/tol = {r}"


# ---- batched NVFP4 and W4A8 -------------------------------------------------------------

def stack(ds, keys):
    t = {}
    for k in keys:
        v = np.stack([d[k] for d in ds])
        if v.dtype == np.uint16:                  # raw bf16 bits
            t[k] = torch.from_numpy(v.view(np.int16)).to(DEV).view(torch.bfloat16)
        else:
            t[k] = torch.from_numpy(v).to(DEV)
    return t


NV_SHAPES = [(3, 100, 200, 1024), (2, 257, 129, 128), (4, 1, 7, 256), (2, 300, 520, 2048)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", NV_SHAPES, ids=[f"L{l}_{m}x{n}x{k}" for l, m, n, k in NV_SHAPES])
def test_nv_batched_matches_oracle(shape, out):
    L, M, N, K = shape
    print(f"case nv batched L={L} {M}x{N}x{K} {out}", flush=True)
    gA, gB = 0.5, 3.0
    ds = [datagen.make_shape("nv", M, N, K, seed=7 + 31 * b) for b in range(L)]
    for d in ds:
        d["gA"], d["gB"] = np.float32(gA), np.float32(gB)
    t = stack(ds, KEYS)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = fp4.nv_fp4_gemm_batched(t["A"], t["sfA"], gA, t["B"], t["sfB"], gB, out_dtype=od)
    torch.cuda.synchronize(DEV)
    D = D.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for b, d in enumerate(ds):
        ref, S = oracle.run("nv", d)
        worst = max(worst, oracle.parity_ratio(D[b], ref, S, out))
    assert worst <= 1.0, f"max |err|/tol = {worst}"


W4_SHAPES = [(3, 100, 200, 1024), (2, 257, 129, 384), (4, 1, 7, 128), (2, 64, 520, 2048)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("shape", W4_SHAPES, ids=[f"L{l}_{m}x{n}x{k}" for l, m, n, k in W4_SHAPES])
def test_w4a8_batched_matches_oracle(shape, out):
    """K = 1024 and 2048 take the K-ring kernel, K = 384 and 128 the other one."""
    L, M, N, K = shape
    print(f"case w4a8 batched L={L} {M}x{N}x{K} {out}", flush=True)
    ds = [datagen.make_shape("w4a8", M, N, K, seed=11 + 17 * b) for b in range(L)]
    t = stack(ds, ("A", "sa", "B", "sB"))
    od = torch.bfloat16 if out == "bf16" else torch.float32
    D = fp4.w4a8_gemm_batched(t["A"], t["sa"], t["B"], t["sB"], out_dtype=od)
    torch.cuda.synchronize(DEV)
    D = D.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for b, d in enumerate(ds):
        ref, S = oracle.run("w4a8", d)
        worst = max(worst, oracle.parity_ratio(D[b], ref, S, out))
    assert worst <= 1.0, f"max |err|/tol = {worst}"


def test_nv_and_w4a8_batch_of_one_equals_plain_call():
    M, N, K = 130, 260, 1024
    nv = stack([datagen.make_shape("nv", M, N, K, seed=3)], KEYS)
    D1 = fp4.nv_fp4_gemm(nv["A"][0], nv["sfA"][0], 2.0, nv["B"][0], nv["sfB"][0], 0.25, out_dtype=torch.float32)
    Db = fp4.nv_fp4_gemm_batched(nv["A"], nv["sfA"], 2.0, nv["B"], nv["sfB"], 0.25, out_dtype=torch.float32)
    w = stack([datagen.make_shape("w4a8", M, N, K, seed=4)], ("A", "sa", "B", "sB"))
    W1 = fp4.w4a8_gemm(w["A"][0], w["sa"][0], w["B"][0], w["sB"][0], out_dtype=torch.float32)
    Wb = fp4.w4a8_gemm_batched(w["A"], w["sa"], w["B"], w["sB"], out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    assert torch.equal(D1, Db[0]) and torch.equal(W1, Wb[0])


def test_nv_and_w4a8_empty_batch_and_zero_k():
    z = torch.empty((0, 4, 64), dtype=torch.uint8, device=DEV)
    assert fp4.nv_fp4_gemm_batched(z, z[:, :, :8], 1.0, z, z[:, :, :8], 1.0).shape == (0, 4, 4)
    a = torch.empty((0, 4, 128), dtype=torch.uint8, device=DEV)
    sa = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    sb = torch.empty((0, 4, 1), dtype=torch.bfloat16, device=DEV)
    assert fp4.w4a8_gemm_batched(a, sa, a[:, :, :64], sb).shape == (0, 4, 4)
    e = torch.empty((3, 5, 0), dtype=torch.uint8, device=DEV)
    D = fp4.nv_fp4_gemm_batched(e, e, 1.0, e[:, :2], e[:, :2], 1.0, out_dtype=torch.float32)
    sa = torch.ones((3, 5), dtype=torch.float32, device=DEV)
    sb = torch.empty((3, 2, 0), dtype=torch.bfloat16, device=DEV)
    W = fp4.w4a8_gemm_batched(e, sa, e[:, :2], sb, out_dtype=torch.float32)
    torch.cuda.synchronize(DEV)
    assert D.shape == (3, 5, 2) and not D.any()
    assert W.shape == (3, 5, 2) and not W.any()
