"""The allocation-free split-K GEMM (mx_fp4_gemm_batched_noalloc) through the C ABI,
against the entry point it varies (mx_fp4_gemm_batched with a caller workspace) and
the oracle: two calls in a row, the second on a smaller problem, so the second reads
the library's scratch after the first has filled it with other partial sums."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def batched_inputs(L, M, N, K, seed):
    rng = np.random.default_rng(seed)
    parts = [datagen.random_mx_gaussian(M, N, K, rng) for _ in range(L)]
    return {k: np.stack([p[k] for p in parts]) for k in ("A", "sfA", "B", "sfB")}


def noalloc_call(t, out, splits):
    lib = fp4.load_library()
    L, M, K2 = t["A"].shape
    N = t["B"].shape[1]
    dt = fp4.OUT_BF16 if out.dtype == torch.bfloat16 else fp4.OUT_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    st = lib.mx_fp4_gemm_batched_noalloc(L, M, N, 2 * K2, t["A"].data_ptr(), t["sfA"].data_ptr(),
                                         t["B"].data_ptr(), t["sfB"].data_ptr(), out.data_ptr(), dt,
                                         splits, stream)
    assert st == 0, fp4.fp4g_status_string(st)


def reference_call(t, out_dtype, splits):
    """The existing entry point with a caller workspace of the size it asks for."""
    L, M, K2 = t["A"].shape
    N = t["B"].shape[1]
    nbytes = fp4.mx_fp4_gemm_workspace_size(L, M, N, 2 * K2, splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    return fp4.mx_fp4_gemm_batched(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=out_dtype, splits=splits,
                                   workspace=ws)


def check_oracle(d, D, b, pairs=None):
    one = {k: d[k][b] for k in ("A", "sfA", "B", "sfB")}
    out = "bf16" if D.dtype == torch.bfloat16 else "f32"
    Dn = D[b].float().cpu().numpy().astype(np.float64)
    if pairs is None:
        ref, S = oracle.run("mx", one)
        r = oracle.parity_ratio(Dn, ref, S, out)
    else:
        ms, ns = pairs
        ref, S = oracle.sampled("mx", one, ms, ns)
        r = oracle.parity_ratio(Dn[ms, ns], ref, S, out)
    assert r <= 1.0, f"max |err|/tol = {r}"


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry_point(out_dtype):
    # 1) the skinny workload shape, split 4 ways: 16 MiB of partial sums in the scratch
    print(f"case noalloc 1x128x8192x8192 splits=4 {out_dtype}", flush=True)
    d1 = batched_inputs(1, 128, 8192, 8192, seed=41)
    t1 = {k: torch.from_numpy(v).to(DEV) for k, v in d1.items()}
    D1 = torch.empty((1, 128, 8192), dtype=out_dtype, device=DEV)
    noalloc_call(t1, D1, 4)
    R1 = reference_call(t1, out_dtype, 4)
    torch.cuda.synchronize(DEV)
    assert torch.equal(D1.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                       R1.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
    rng = np.random.default_rng(3)
    check_oracle(d1, D1, 0, (rng.integers(0, 128, 1500), rng.integers(0, 8192, 1500)))
    # 2) right after, a smaller batched problem with the library's own split choice and
    #    with an explicit odd split; the scratch still holds the first call's partials
    for splits in (0, 3):
        print(f"case noalloc 2x64x1000x2048 splits={splits} {out_dtype}", flush=True)
        d2 = batched_inputs(2, 64, 1000, 2048, seed=42 + splits)
        t2 = {k: torch.from_numpy(v).to(DEV) for k, v in d2.items()}
        D2 = torch.full((2, 64, 1000), float("nan"), dtype=out_dtype, device=DEV)
        noalloc_call(t2, D2, splits)
        R2 = reference_call(t2, out_dtype, splits)
        torch.cuda.synchronize(DEV)
        assert torch.equal(D2.float(), R2.float())
        for b in range(2):
            check_oracle(d2, D2, b)


def test_noalloc_without_split_and_oversized_split():
    d = batched_inputs(1, 96, 256, 512, seed=43)
    t = {k: torch.from_numpy(v).to(DEV) for k, v in d.items()}
    D = torch.empty((1, 96, 256), dtype=torch.float32, device=DEV)
    print("case noalloc 1x96x256x512 splits=1", flush=True)
    noalloc_call(t, D, 1)
    torch.cuda.synchronize(DEV)
    check_oracle(d, D, 0)
    # a requested split that does not fit the scratch is refused, and launches nothing
    big = {"A": torch.zeros((1, 512, 4096), dtype=torch.uint8, device=DEV),
           "sfA": torch.zeros((1, 512, 256), dtype=torch.uint8, device=DEV),
           "B": torch.zeros((1, 4096, 4096), dtype=torch.uint8, device=DEV),
           "sfB": torch.zeros((1, 4096, 256), dtype=torch.uint8, device=DEV)}
    out = torch.empty((1, 512, 4096), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fp4.Fp4GemmError):
        fp4.mx_fp4_gemm_batched_noalloc(big["A"], big["sfA"], big["B"], big["sfB"], out, splits=8)
