"""The entry points under HIP graph capture.

Every entry point enqueues only kernels (the empty-K product is a fill kernel, never a
memset node), so a caller may capture it.  Captured calls are replayed several times,
with unrelated eager work and synchronisations between the replays, and every replay
must reproduce the eager result bit for bit: the kernels use a fixed summation order.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def up(d, keys):
    return {k: torch.from_numpy(d[k]).to(DEV) for k in keys}


def test_replays_match_eager():
    mx = up(datagen.make_shape("mx", 200, 300, 1024, seed=1), ("A", "sfA", "B", "sfB"))
    gv = up(datagen.make_shape("gemv", 8, 1000, 2048, seed=2), ("A", "sfA", "B", "sfB"))
    L, M, N, K = 2, 64, 256, 4096
    bd = [datagen.make_shape("mx", M, N, K, seed=3 + b) for b in range(L)]
    bt = {k: torch.from_numpy(np.stack([d[k] for d in bd])).to(DEV) for k in ("A", "sfA", "B", "sfB")}
    ws = torch.empty(fp4.mx_fp4_gemm_workspace_size(L, M, N, K, 4), dtype=torch.uint8, device=DEV)
    x = torch.randn((300, 512), device=DEV)
    za = torch.empty((5, 0), dtype=torch.uint8, device=DEV)             # K = 0 operands
    zb = torch.empty((7, 0), dtype=torch.uint8, device=DEV)

    outs = {
        "mx": torch.empty((200, 300), dtype=torch.bfloat16, device=DEV),
        "gemv": torch.empty((8, 1000), dtype=torch.float32, device=DEV),
        "batched": torch.empty((L, M, N), dtype=torch.bfloat16, device=DEV),
        "codes": torch.empty((300, 256), dtype=torch.uint8, device=DEV),
        "scales": torch.empty((300, 16), dtype=torch.uint8, device=DEV),
        "zero": torch.empty((5, 7), dtype=torch.float32, device=DEV),
    }

    def calls():
        fp4.mx_fp4_gemm(mx["A"], mx["sfA"], mx["B"], mx["sfB"], out=outs["mx"])
        fp4.fp4_gemv(gv["A"], gv["sfA"], gv["B"], gv["sfB"], out=outs["gemv"])
        fp4.mx_fp4_gemm_batched(bt["A"], bt["sfA"], bt["B"], bt["sfB"], out=outs["batched"], splits=4,
                                workspace=ws)
        fp4.mx_fp4_quantize(x, outs["codes"], outs["scales"])
        fp4.nv_fp4_gemm(za, za, 1.0, zb, zb, 1.0, out=outs["zero"])       # empty sum: a fill kernel

    calls()
    torch.cuda.synchronize(DEV)
    eager = {k: v.clone() for k, v in outs.items()}
    assert not eager["zero"].any()

    stream = torch.cuda.Stream(device=DEV)
    stream.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(stream):
        calls()                                   # warm the side stream before capture
    torch.cuda.current_stream(DEV).wait_stream(stream)
    torch.cuda.synchronize(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for v in outs.values():
            v.fill_(1)                            # the replay must overwrite everything
        g.replay()
        torch.cuda.synchronize(DEV)
        for k, v in outs.items():
            assert torch.equal(v, eager[k]), f"replay {rep}: {k} differs from the eager result"
        # unrelated eager work between replays
        fp4.mx_fp4_gemm(gv["A"], gv["sfA"], gv["B"], gv["sfB"], out_dtype=torch.float32)
        (x * 2).sum()
        torch.cuda.synchronize(DEV)
