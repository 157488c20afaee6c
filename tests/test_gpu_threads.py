"""The C ABI from several host threads at once, each on its own stream: results equal
those of the same calls made one at a time (the library keeps no per-call state)."""
import threading

import numpy as np
import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4
import datagen

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_concurrent_calls_match_serial():
    jobs = []
    for j in range(6):
        d = datagen.make_shape("mx", 96 + 32 * j, 200, 512, seed=50 + j)
        t = {k: torch.from_numpy(d[k]).to(DEV) for k in ("A", "sfA", "B", "sfB")}
        jobs.append(t)
    serial = [fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=torch.float32) for t in jobs]
    gv = [fp4.fp4_gemv(t["A"][:8], t["sfA"][:8], t["B"], t["sfB"], out_dtype=torch.float32) for t in jobs]
    torch.cuda.synchronize(DEV)
    results = [None] * len(jobs)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(s):
                t = jobs[i]
                outs = []
                for _ in range(5):
                    outs.append(fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out_dtype=torch.float32))
                    outs.append(fp4.fp4_gemv(t["A"][:8], t["sfA"][:8], t["B"], t["sfB"], out_dtype=torch.float32))
            s.synchronize()
            results[i] = outs
        except Exception as e:          # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for i, outs in enumerate(results):
        for k, o in enumerate(outs):
            ref = serial[i] if k % 2 == 0 else gv[i]
            assert torch.equal(o, ref), f"thread {i} call {k}"
