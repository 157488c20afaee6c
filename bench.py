"""Benchmark of the block-scaled FP4 GEMM path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME ...] [--no-cpu]

A step is one call of the hot path on one batch of resident synthetic input:
the headline is the MXFP4 GEMM M = N = K = 8192 (E2M1 operands quantized from
N(0,1) with max-abs E8M0 block scales, fp32 accumulation, bf16 output).  The
decode GEMV (M=8, N=14336, K=4096, cache-cold through rotating weight copies),
the W4A8 GEMM (256x8192x8192), the NVFP4 GEMM (1024^3) and the MXFP4 256^3 case
are timed after it and reported in "also".  Every duration is the average over
`steps` launches captured in one HIP graph and replayed between a HIP event pair
on the stream the kernels run on (torch's current stream, which the binding
passes to the library); the GEMV is also timed with eager launches.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_scaled_precision_e2m1_amd as fp4  # noqa: E402
import datagen  # noqa: E402

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "bf16": 2500.0}
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_scaled_precision_e2m1_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fp4_device_cus(dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def to_dev(d, dev):
    out = {}
    for k, v in d.items():
        if isinstance(v, np.ndarray) and v.ndim > 0:
            if k == "sB" and v.dtype == np.uint16:      # W4A8 group scales: raw bf16 bits
                out[k] = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
            else:
                out[k] = torch.from_numpy(v).to(dev)
    return out


USE_GRAPH = True


def time_launches(fn, steps, warmup, dev, arg_sets=None, graph=None):
    """Average duration (ms) of one launch.  `steps` launches (rotating through
    `arg_sets`) are captured into one HIP graph, which is replayed once untimed and
    once between a HIP event pair on the current stream, so the host's per-call cost
    (Python, ctypes) does not leave the GPU idle between short kernels.  With
    graph=False the launches are enqueued eagerly between the event pair instead.
    Returns (ms per launch, host wall seconds of the timed region)."""
    arg_sets = arg_sets or [()]
    graph = USE_GRAPH if graph is None else graph
    for i in range(warmup):
        fn(*arg_sets[i % len(arg_sets)])
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(*arg_sets[i % len(arg_sets)])
        g.replay()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        e0.record(stream)
        g.replay()
        e1.record(stream)
    else:
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            fn(*arg_sets[i % len(arg_sets)])
        e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    return float(e0.elapsed_time(e1) / steps), wall


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Counter summaries: (profile name, kernel-name prefix in the trace, sources of the kernel).
_NS = "fp4g::(anonymous namespace)::"
COUNTED = [("mxfp4_gemm_8192", _NS + "mxfp4_gemm_kernel<256, 256, 128, 128, 256, 2, true, false>",
            ["mxfp4_gemm.hip", "common.hpp"]),
           ("fp4_gemv_8x14336x4096", _NS + "fp4_gemv_kernel<1, 2, 1,", ["fp4_gemv.hip", "common.hpp"]),
           ("fp4_gemv_prepacked_8x14336x4096", _NS + "fp4_gemv_prepacked_kernel<",
            ["fp4_gemv_prepacked.hip", "common.hpp"]),
           ("mxfp4_split_k_128x8192x8192", _NS + "mxfp4_gemm_kernel<128, 128, 64, 64, 256, 2, false, true>",
            ["mxfp4_gemm.hip", "common.hpp"]),
           ("mxfp4_split_k_reduce_128x8192x8192", _NS + "splitk_reduce_kernel<", ["mxfp4_gemm.hip", "common.hpp"]),
           ("w4a8_256x8192x8192", _NS + "w4a8p_gemm_kernel<64, false, false",
            ["w4a8_gemm.hip", "w4a8_prepacked.hip", "common.hpp"]),
           ("w4a8_prepacked_256x8192x8192", _NS + "w4a8p_gemm_kernel<64, true, false",
            ["w4a8_prepacked.hip", "common.hpp"]),
           ("nvfp4_gemm_1024", _NS + "nvfp4_gemm_kernel<64, 64, 16, 32, false",
            ["nvfp4_gemm.hip", "nv_fold.hpp", "common.hpp"]),
           ("fp8_blockwise_4096", _NS + "fp8b_gemm_big_kernel<", ["fp8b_gemm.hip", "common.hpp"]),
           ("mx_quantize_8192x8192_f32", _NS + "mx_quantize_kernel<", ["mx_quantize.hip", "common.hpp"]),
           ("nv_quantize_8192x8192_f32", _NS + "nv_quantize_kernel<", ["mx_quantize.hip", "common.hpp"]),
           # decode (M = 8, K = 8192: two 4-group segments per wave, two row groups; M = 32:
           # the same with two token tiles) and the K-split GEMMs at M = 64 (64-row tiles,
           # split kernel + scaled reduction)
           ("w4a8_decode_8x8192x8192", _NS + "w4a8_gemv_kernel<2, 2, 2, 1, 1,", ["w4a8_gemv.hip", "common.hpp"]),
           ("w4a8_decode_prepacked_8x8192x8192", _NS + "w4a8_gemv_kernel<2, 2, 2, 0, 1,",
            ["w4a8_gemv.hip", "common.hpp"]),
           ("nvfp4_decode_8x8192x8192", _NS + "nvfp4_gemv_kernel<2, 2, 1,",
            ["nvfp4_gemv.hip", "nv_fold.hpp", "common.hpp"]),
           ("w4a8_decode_32x8192x8192", _NS + "w4a8_gemv_kernel<2, 2, 2, 1, 2,", ["w4a8_gemv.hip", "common.hpp"]),
           ("w4a8_decode_prepacked_32x8192x8192", _NS + "w4a8_gemv_kernel<2, 2, 2, 0, 2,",
            ["w4a8_gemv.hip", "common.hpp"]),
           ("nvfp4_decode_32x8192x8192", _NS + "nvfp4_gemv_kernel<2, 2, 2,",
            ["nvfp4_gemv.hip", "nv_fold.hpp", "common.hpp"]),
           ("w4a8_split_64x8192x8192", _NS + "w4a8p_gemm_kernel<64, false, true",
            ["w4a8_gemm.hip", "w4a8_prepacked.hip", "common.hpp"]),
           ("w4a8_prepacked_split_64x8192x8192", _NS + "w4a8p_gemm_kernel<64, true, true",
            ["w4a8_prepacked.hip", "common.hpp"]),
           ("nvfp4_split_64x8192x8192", _NS + "nvfp4_gemm_kernel<64, 64, 16, 32, true",
            ["nvfp4_gemm.hip", "nv_fold.hpp", "common.hpp"]),
           ("split_reduce_64x8192x8192", _NS + "scaled_reduce_kernel<", ["splitk_reduce.hip", "common.hpp"]),
           ("w4a8_fp6_256x8192x8192", _NS + "w4a8f6_gemm_kernel<", ["w4a8_fp6.hip", "common.hpp"])]
# The kernels that the counter runs cover: `bench.py --only` + this list.
COUNTED_ONLY = "mx8192 gemv gemvp w4a8 w4a8p w4a8f6 nv1024 fp8b quant nvquant skinny decode copy"


def traffic_of(name):
    """traffic_from_profile for a COUNTED entry."""
    src = next(src for n, _, src in COUNTED if n == name)
    return traffic_from_profile(name, src, None)
COPY_KERNEL = "__amd_rocclr_copyBuffer"
TRAFFIC_SOURCE = ("committed rocprofv3 counter summary (profiles/<kernel>_counters.txt: FETCH_SIZE and WRITE_SIZE "
                  "scaled by a 512 MiB device copy), used only while the kernel's source hash matches; null otherwise")


def traffic_from_profile(name, kernel_src, launches_bytes):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{name}_counters.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_src_sha") != src_digest(*kernel_src):
        return None
    return float(c["fetch_bytes_scaled"] + c["write_bytes_scaled"])


def summarize_counters(fetch_dir, write_dir, command):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
    `bench.py --only <COUNTED_ONLY> --no-graph` into profiles/<name>_counters.txt.
    The counters are scaled by what they read for the 512 MiB device copy (which
    reads and writes exactly 512 MiB): bytes = counter * (copy bytes / copy counter)."""
    import csv
    import glob

    def load(d, counter):
        per = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return per

    os.makedirs(PROFILES, exist_ok=True)
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")

    def pick(per, prefix):
        vals = [v for k, vs in per.items() if prefix in k for v in vs]
        if not vals:
            raise SystemExit(f"no dispatches of {prefix} in the counter runs")
        return float(np.median(vals)), len(vals)

    def pick_copy(per):
        # The 512 MiB copy is the largest blit in the run (input uploads and the GEMV's
        # weight clones are blits too): take the dispatches within 1% of the largest.
        vals = [v for k, vs in per.items() if COPY_KERNEL in k for v in vs]
        if not vals:
            raise SystemExit("no copy dispatches in the counter runs")
        top = max(vals)
        return float(np.median([v for v in vals if v >= 0.99 * top]))

    copy_bytes = 512 * (1 << 20)
    cf, cw = pick_copy(fetch), pick_copy(write)
    f_scale, w_scale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    for name, prefix, src in COUNTED:
        fk, nf = pick(fetch, prefix)
        wk, nw = pick(write, prefix)
        out = {"kernel": prefix, "kernel_src_sha": src_digest(*src), "dispatches": [nf, nw],
               "fetch_kib_median": fk, "write_kib_median": wk,
               "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes_each_way": copy_bytes,
               "fetch_scale": f_scale, "write_scale": w_scale,
               "fetch_bytes_scaled": fk * 1024 * f_scale, "write_bytes_scaled": wk * 1024 * w_scale,
               "command": command}
        with open(os.path.join(PROFILES, f"{name}_counters.txt"), "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        log(f"{name}: fetch {out['fetch_bytes_scaled'] / 1e6:.1f} MB, write {out['write_bytes_scaled'] / 1e6:.1f} MB "
            f"per launch (scales {f_scale:.3f} / {w_scale:.3f})")


# Utilisation counters: (workload key, kernel-name prefix, sources of the kernel).
UTIL_KERNELS = [("mxfp4_gemm_8192x8192x8192", "mxfp4_gemm_kernel<256, 256, 128, 128, 256, 2, true, false>",
                 ["mxfp4_gemm.hip", "common.hpp"]),
                ("mxfp4_gemv_8x14336x4096", "fp4_gemv_kernel<1, 2, 1, true, true, true, 8>", ["fp4_gemv.hip", "common.hpp"]),
                ("w4a8_256x8192x8192", "w4a8p_gemm_kernel<64, false, false",
                 ["w4a8_gemm.hip", "w4a8_prepacked.hip", "common.hpp"]),
                ("w4a8_256x8192x8192_prepacked", "w4a8p_gemm_kernel<64, true, false",
                 ["w4a8_prepacked.hip", "common.hpp"]),
                ("fp8_blockwise_4096", "fp8b_gemm_big_kernel<", ["fp8b_gemm.hip", "common.hpp"]),
                ("nvfp4_1024", "nvfp4_gemm_kernel<64, 64, 16, 32, false", ["nvfp4_gemm.hip", "nv_fold.hpp", "common.hpp"]),
                ("w4a8_256x8192x8192_fp6", "w4a8f6_gemm_kernel<", ["w4a8_fp6.hip", "common.hpp"]),
                ("decode_8x8192x8192_w4a8", "w4a8_gemv_kernel<2, 2, 2, 1, 1,", ["w4a8_gemv.hip", "common.hpp"]),
                ("decode_8x8192x8192_nvfp4", "nvfp4_gemv_kernel<2, 2, 1,", ["nvfp4_gemv.hip", "nv_fold.hpp", "common.hpp"]),
                ("mx_quantize_8192x8192_f32", "mx_quantize_kernel<", ["mx_quantize.hip", "common.hpp"])]
UTIL_METRICS = ("MfmaUtil", "LdsUtil", "VALUBusy", "LdsBankConflict")
UTIL_FILE = os.path.join(PROFILES, "utilisation_counters.txt")


def summarize_util(util_dir, command):
    """Turn one rocprofv3 --pmc run of the derived metrics MfmaUtil, LdsUtil, VALUBusy and
    LdsBankConflict (percent of the busy GPU's cycles; conflicts per LDS cycle) over
    `bench.py --no-graph` into profiles/utilisation_counters.txt."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(util_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
            per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {"command": command, "kernels": {}}
    for key, prefix, src in UTIL_KERNELS:
        hits = [c for n, c in per.items() if prefix in n]
        if not hits:
            continue
        vals = {m: float(np.median([v for c in hits for v in c.get(m, [])])) for m in UTIL_METRICS
                if any(m in c for c in hits)}
        out["kernels"][key] = {"kernel": prefix, "kernel_src_sha": src_digest(*src), **vals}
        log(f"{key}: " + ", ".join(f"{m} {v:.1f}" for m, v in vals.items()))
    os.makedirs(PROFILES, exist_ok=True)
    with open(UTIL_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def util_from_profile(key):
    """MFMA/LDS/VALU utilisation of a workload's kernel from the committed counter
    summary, if it was taken on the current kernel source; otherwise None."""
    if not os.path.exists(UTIL_FILE):
        return None
    k = json.load(open(UTIL_FILE)).get("kernels", {}).get(key)
    if k is None:
        return None
    src = next(src for kk, _, src in UTIL_KERNELS if kk == key)
    if k["kernel_src_sha"] != src_digest(*src):
        return None
    return {"mfma_util_pct": k.get("MfmaUtil"), "lds_util_pct": k.get("LdsUtil"),
            "valu_busy_pct": k.get("VALUBusy")}


# ---- workloads ------------------------------------------------------------------------

def bench_mx8192(steps, warmup, dev):
    d = datagen.make("mxfp4_8192")
    t = to_dev(d, dev)
    M = N = K = 8192
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out=D)
    mean_ms, wall = time_launches(fn, steps, warmup, dev)
    flops = 2.0 * M * N * K
    tf = flops / (mean_ms * 1e-3) / 1e12
    bytes_alg = d["A"].nbytes + d["sfA"].nbytes + d["B"].nbytes + d["sfB"].nbytes + M * N * 2
    # The shader clock the GEMM runs at, averaged over 200 back-to-back launches (outside
    # the timed region).
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(50):
            fn()
    g.replay()
    torch.cuda.synchronize(dev)
    ghz = shader_clock_over(lambda: [g.replay() for _ in range(4)], dev)
    return d, {"ms": mean_ms, "wall_s": wall, "tflops": tf, "flops": flops,
               "bytes": bytes_alg, "D": D, "ghz": ghz}


def bench_gemv(steps, warmup, dev):
    d = datagen.make("mxfp4_gemv_8x14336x4096")
    M, N, K = 8, 14336, 4096
    base = to_dev(d, dev)
    wbytes = d["B"].nbytes + d["sfB"].nbytes
    copies = int(np.ceil(320e6 / wbytes))          # > 256 MB infinity cache: cold reads
    sets = []
    for c in range(copies):
        B = base["B"].clone() if c else base["B"]
        sB = base["sfB"].clone() if c else base["sfB"]
        sets.append((B, sB))
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda B, sB: fp4.fp4_gemv(base["A"], base["sfA"], B, sB, out=D)
    mean_ms, wall = time_launches(fn, steps, warmup, dev, sets)
    replayed = D.clone()                           # output of the graph's last launch
    fn(*sets[(steps - 1) % copies])
    torch.cuda.synchronize(dev)
    if not torch.equal(replayed, D):
        raise RuntimeError("GEMV: graph replay and eager launch disagree")
    eager_ms, _ = time_launches(fn, steps, 0, dev, sets, graph=False)
    bytes_alg = d["A"].nbytes + d["sfA"].nbytes + wbytes + M * N * 2
    gbs = bytes_alg / (mean_ms * 1e-3) / 1e9
    return {"ms": mean_ms, "eager_ms": eager_ms, "gbs": gbs, "bytes": bytes_alg, "copies": copies,
            "tflops": 2.0 * M * N * K / (mean_ms * 1e-3) / 1e12, "d": d, "D": D}


def bench_gemv_prepacked(steps, warmup, dev):
    """The decode GEMV over weights re-packed once at load time (fp4_gemv_prepack), with
    the same rotating cold copies as the plain GEMV."""
    d = datagen.make("mxfp4_gemv_8x14336x4096")
    M, N, K = 8, 14336, 4096
    base = to_dev(d, dev)
    Bp0, Sp0 = fp4.fp4_gemv_prepack(base["B"], base["sfB"])
    wbytes = Bp0.numel() + Sp0.numel()
    copies = int(np.ceil(320e6 / wbytes))
    sets = [((Bp0.clone(), Sp0.clone()) if c else (Bp0, Sp0)) for c in range(copies)]
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda Bp, Sp: fp4.fp4_gemv_prepacked(base["A"], base["sfA"], Bp, Sp, N, out=D)
    mean_ms, _ = time_launches(fn, steps, warmup, dev, sets)
    bytes_alg = d["A"].nbytes + d["sfA"].nbytes + d["B"].nbytes + d["sfB"].nbytes + M * N * 2
    return {"ms": mean_ms, "gbs": bytes_alg / (mean_ms * 1e-3) / 1e9, "bytes": bytes_alg, "copies": copies}


def bench_w4a8(steps, warmup, dev):
    d = datagen.make("w4a8_256x8192x8192")
    M, N, K = 256, 8192, 8192
    base = to_dev(d, dev)
    wbytes = d["B"].nbytes + d["sB"].nbytes
    copies = int(np.ceil(320e6 / wbytes))
    sets = [((base["B"].clone(), base["sB"].clone()) if c else (base["B"], base["sB"])) for c in range(copies)]
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda B, sB: fp4.w4a8_gemm(base["A"], base["sa"], B, sB, out=D)
    mean_ms, wall = time_launches(fn, steps, warmup, dev, sets)
    flops = 2.0 * M * N * K
    bytes_alg = d["A"].nbytes + d["sa"].nbytes + wbytes + M * N * 2
    return {"ms": mean_ms, "tflops": flops / (mean_ms * 1e-3) / 1e12,
            "gbs": bytes_alg / (mean_ms * 1e-3) / 1e9, "bytes": bytes_alg, "copies": copies, "d": d, "D": D}


def bench_w4a8_prepacked(steps, warmup, dev):
    """W4A8 over weights re-packed once at load time (w4a8_prepack), same rotating cold
    copies as the unpacked kernel."""
    d = datagen.make("w4a8_256x8192x8192")
    M, N, K = 256, 8192, 8192
    base = to_dev(d, dev)
    Bp0, Sp0 = fp4.w4a8_prepack(base["B"], base["sB"])
    wbytes = Bp0.numel() + Sp0.numel() * 4
    copies = int(np.ceil(320e6 / wbytes))
    sets = [((Bp0.clone(), Sp0.clone()) if c else (Bp0, Sp0)) for c in range(copies)]
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda Bp, Sp: fp4.w4a8_gemm_prepacked(base["A"], base["sa"], Bp, Sp, N, out=D)
    mean_ms, _ = time_launches(fn, steps, warmup, dev, sets)
    flops = 2.0 * M * N * K
    bytes_alg = d["A"].nbytes + d["sa"].nbytes + d["B"].nbytes + d["sB"].nbytes + M * N * 2
    return {"ms": mean_ms, "tflops": flops / (mean_ms * 1e-3) / 1e12,
            "gbs": bytes_alg / (mean_ms * 1e-3) / 1e9, "bytes": bytes_alg, "copies": copies}


def bench_w4a8_fp6(steps, warmup, dev):
    """W4A8 over weights re-encoded once at load time as FP6 (w4a8_prepack_fp6), rotating
    cold copies as for the other W4A8 kernels."""
    d = datagen.make("w4a8_256x8192x8192")
    M, N, K = 256, 8192, 8192
    base = to_dev(d, dev)
    Bp0, Sp0 = fp4.w4a8_prepack_fp6(base["B"], base["sB"])
    wbytes = Bp0.numel() + Sp0.numel() * 4
    copies = int(np.ceil(320e6 / wbytes))
    sets = [((Bp0.clone(), Sp0.clone()) if c else (Bp0, Sp0)) for c in range(copies)]
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda Bp6, Sp: fp4.w4a8_gemm_prepacked_fp6(base["A"], base["sa"], Bp6, Sp, N, out=D)
    mean_ms, _ = time_launches(fn, steps, warmup, dev, sets)
    flops = 2.0 * M * N * K
    bytes_alg = d["A"].nbytes + d["sa"].nbytes + d["B"].nbytes + d["sB"].nbytes + M * N * 2
    layout_bytes = d["A"].nbytes + d["sa"].nbytes + wbytes + M * N * 2
    return {"ms": mean_ms, "tflops": flops / (mean_ms * 1e-3) / 1e12,
            "gbs": bytes_alg / (mean_ms * 1e-3) / 1e9, "bytes": bytes_alg, "layout_bytes": layout_bytes,
            "copies": copies}


def bench_nv1024(steps, warmup, dev):
    d = datagen.make("nvfp4_1024")
    t = to_dev(d, dev)
    M = N = K = 1024
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp4.nv_fp4_gemm(t["A"], t["sfA"], 1.0, t["B"], t["sfB"], 1.0, out=D)
    mean_ms, _ = time_launches(fn, steps, warmup, dev)
    return {"ms": mean_ms, "tflops": 2.0 * M * N * K / (mean_ms * 1e-3) / 1e12, "d": d, "D": D}


def bench_mx256(steps, warmup, dev):
    d = datagen.make("mxfp4_256")
    t = to_dev(d, dev)
    D = torch.empty((256, 256), dtype=torch.float32, device=dev)
    fn = lambda: fp4.mx_fp4_gemm(t["A"], t["sfA"], t["B"], t["sfB"], out=D)
    mean_ms, _ = time_launches(fn, steps, warmup, dev)
    return {"ms": mean_ms, "tflops": 2.0 * 256 ** 3 / (mean_ms * 1e-3) / 1e12, "d": d, "D": D}


def bench_fp8b(steps, warmup, dev):
    d = datagen.make("fp8_block_4096")
    M = N = K = 4096
    t = to_dev(d, dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda: fp4.fp8_blockwise_gemm(t["A"], t["sA"], t["B"], t["sB"], out=D)
    mean_ms, _ = time_launches(fn, steps, warmup, dev)
    bytes_alg = d["A"].nbytes + d["sA"].nbytes + d["B"].nbytes + d["sB"].nbytes + M * N * 2
    return {"ms": mean_ms, "tflops": 2.0 * M * N * K / (mean_ms * 1e-3) / 1e12, "bytes": bytes_alg, "d": d, "D": D}


def bench_skinny(steps, warmup, dev, L=1, M=128, N=8192, K=8192):
    """Batched MXFP4 GEMM on a skinny problem whose 128 x 128 tiles cannot fill the
    CUs, timed with the library's own K split and without one.  Weight copies rotate
    (past the 256 MB last-level cache) as in a decode/prefill step."""
    rng = np.random.default_rng(0)
    d = datagen.random_mx_gaussian(L * M, N, K, rng)
    A = torch.from_numpy(d["A"]).to(dev).view(L, M, K // 2)
    sA = torch.from_numpy(d["sfA"]).to(dev).view(L, M, K // 32)
    B0 = torch.from_numpy(d["B"]).to(dev)[None].expand(L, N, K // 2).contiguous()
    sB0 = torch.from_numpy(d["sfB"]).to(dev)[None].expand(L, N, K // 32).contiguous()
    wbytes = B0.numel() + sB0.numel()
    copies = int(np.ceil(320e6 / wbytes))
    sets = [((B0.clone(), sB0.clone()) if c else (B0, sB0)) for c in range(copies)]
    D = torch.empty((L, M, N), dtype=torch.bfloat16, device=dev)
    out = {"copies": copies}
    for label, splits in (("auto", 0), ("none", 1)):
        nbytes = fp4.mx_fp4_gemm_workspace_size(L, M, N, K, splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        fn = lambda B, sB: fp4.mx_fp4_gemm_batched(A, sA, B, sB, out=D, splits=splits, workspace=ws)
        ms, _ = time_launches(fn, steps, warmup, dev, sets)
        out[label] = {"ms": ms, "tflops": 2.0 * L * M * N * K / (ms * 1e-3) / 1e12,
                      "splits": nbytes // (L * M * N * 4) if nbytes else 1}
    return out


def bench_decode(steps, warmup, dev, N=8192, K=8192):
    """Few-token calls on an N x K = 8192 x 8192 weight, cold rotating weight copies: the
    decode kernels (W4A8 plain and pre-packed, NVFP4) at M = 8 (one 16-token tile) and
    M = 32 (two), and the K-split W4A8 and NVFP4 GEMMs at M = 64 with the library's own
    split."""
    w = datagen.make_shape("w4a8", 64, N, K, seed=0)
    n = datagen.random_nv(64, N, K, np.random.default_rng(0))
    A8, sa = torch.from_numpy(w["A"]).to(dev), torch.from_numpy(w["sa"]).to(dev)
    B4 = torch.from_numpy(w["B"]).to(dev)
    sB = torch.from_numpy(w["sB"].view(np.int16)).to(dev).view(torch.bfloat16)
    A4, sfA = torch.from_numpy(n["A"]).to(dev), torch.from_numpy(n["sfA"]).to(dev)
    NB, sfB = torch.from_numpy(n["B"]).to(dev), torch.from_numpy(n["sfB"]).to(dev)
    copies = int(np.ceil(320e6 / (B4.numel() + sB.numel() * 2)))
    w_sets = [((B4.clone(), sB.clone()) if c else (B4, sB)) for c in range(copies)]
    p_sets = [fp4.w4a8_prepack(b, s) for b, s in w_sets]
    n_sets = [((NB.clone(), sfB.clone()) if c else (NB, sfB)) for c in range(copies)]
    out = {"copies": copies}
    wbytes = {"w4a8": B4.numel() + sB.numel() * 2, "w4a8_prepacked": B4.numel() + sB.numel() * 4,
              "nvfp4": NB.numel() + sfB.numel()}
    # per token: E4M3 codes + the fp32 row scale (W4A8); E2M1 codes + E4M3 scales (NVFP4)
    abytes = {"w4a8": K + 4, "w4a8_prepacked": K + 4, "nvfp4": K // 2 + K // 16}
    for M in (8, 32, 64):
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        a8, s8, a4, f4 = A8[:M].contiguous(), sa[:M].contiguous(), A4[:M].contiguous(), sfA[:M].contiguous()
        ws = torch.empty(max(fp4.w4a8_gemm_workspace_size(1, M, N, K), fp4.nv_fp4_gemm_workspace_size(1, M, N, K), 16),
                         dtype=torch.uint8, device=dev)
        fns = {"w4a8": (lambda B, s_: fp4.w4a8_gemm_split(a8[None], s8[None], B[None], s_[None], out=D[None],
                                                           workspace=ws), w_sets),
               "w4a8_prepacked": (lambda Bp, Sp: fp4.w4a8_gemm_prepacked_split(a8, s8, Bp, Sp, N, out=D,
                                                                               workspace=ws), p_sets),
               "nvfp4": (lambda B, s_: fp4.nv_fp4_gemm_split(a4[None], f4[None], 1.0, B[None], s_[None], 1.0,
                                                              out=D[None], workspace=ws), n_sets)}
        row = {"splits": {"w4a8": fp4.w4a8_gemm_workspace_size(1, M, N, K) // (M * N * 4) or 1,
                          "nvfp4": fp4.nv_fp4_gemm_workspace_size(1, M, N, K) // (M * N * 4) or 1}}
        for name, (fn, sets) in fns.items():
            ms, _ = time_launches(fn, steps, warmup, dev, sets)
            nbytes = wbytes[name] + abytes[name] * M + M * N * 2
            row[name] = {"us": ms * 1e3, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
                         "tflops": 2.0 * M * N * K / (ms * 1e-3) / 1e12}
        out[M] = row
    return out


def decode_traffic(name, M):
    """HBM bytes per call of a bench_decode row from the counter summaries: the decode
    kernel (M = 8 and 32), or the split kernel plus its scaled reduction (M = 64)."""
    if M <= 32:
        return traffic_of({"w4a8": f"w4a8_decode_{M}x8192x8192", "w4a8_prepacked": f"w4a8_decode_prepacked_{M}x8192x8192",
                           "nvfp4": f"nvfp4_decode_{M}x8192x8192"}[name])
    t = traffic_of({"w4a8": "w4a8_split_64x8192x8192", "w4a8_prepacked": "w4a8_prepacked_split_64x8192x8192",
                    "nvfp4": "nvfp4_split_64x8192x8192"}[name])
    r = traffic_of("split_reduce_64x8192x8192")
    return t + r if t is not None and r is not None else None


def bench_quant(steps, warmup, dev):
    """MX quantizer on an 8192 x 8192 fp32 activation (the GEMM's operand size): two
    input copies alternate (512 MB, past the 256 MB last-level cache)."""
    rows, K = 8192, 8192
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    xs = [torch.randn((rows, K), generator=g, device=dev, dtype=torch.float32) for _ in range(2)]
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=dev)
    fn = lambda X: fp4.mx_fp4_quantize(X, codes, scales)
    mean_ms, _ = time_launches(fn, steps, warmup, dev, [(x,) for x in xs])
    bytes_alg = rows * K * 4 + codes.numel() + scales.numel()
    return {"ms": mean_ms, "bytes": bytes_alg, "gbs": bytes_alg / (mean_ms * 1e-3) / 1e9}


def bench_nvquant(steps, warmup, dev):
    """NV quantizer on the same 8192 x 8192 fp32 activations (two alternating copies),
    with the tensor's global scale max|x| / (448 * 6) computed once, outside the timing."""
    rows, K = 8192, 8192
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    xs = [torch.randn((rows, K), generator=g, device=dev, dtype=torch.float32) for _ in range(2)]
    gs = [float(x.abs().max()) / (448.0 * 6.0) for x in xs]
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
    fn = lambda X, gsc: fp4.nv_fp4_quantize(X, gsc, codes, scales)
    mean_ms, _ = time_launches(fn, steps, warmup, dev, list(zip(xs, gs)))
    bytes_alg = rows * K * 4 + codes.numel() + scales.numel()
    return {"ms": mean_ms, "bytes": bytes_alg, "gbs": bytes_alg / (mean_ms * 1e-3) / 1e9}


def bench_copy(dev, mib=512):
    """A plain device copy of known size, the reference that scales the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) into bytes."""
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    ms, _ = time_launches(lambda: dst.copy_(src), 3, 1, dev, graph=False)   # eager: a blit kernel
    return {"bytes_each_way": n, "ms": ms, "gbs": 2 * n / (ms * 1e-3) / 1e9}


# ---- measured ceilings and the shader clock ------------------------------------------------

PROBE_LIB = os.path.join(ROOT, "block_scaled_precision_e2m1_amd", "libfp4probe.so")


def measure_peaks(dev, cus):
    """The FP4 matrix pipe's attainable rate (all CUs, one wave per SIMD, 12 independent
    32x32x64 chains on random operand bits) with the shader clock it held, and the HBM
    read rate of a 1 GiB stream (past the 256 MB last-level cache)."""
    import ctypes
    lib = _probe_lib()
    if lib is None:
        return None
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    grid, iters, chains = cus, 100000, 12
    sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(grid * 4, dtype=torch.int64, device=dev)
    run = lambda: lib.fp4p_mfma_probe(grid, iters, 12345, sink.data_ptr(), clocks.data_ptr(), stream)
    if run():
        return None
    ms, _ = time_launches(run, 3, 1, dev, graph=False)
    c = clocks.view(grid, 4).cpu().numpy().astype(np.float64)
    ghz = float(np.median((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6))) / 1e9
    flops = grid * 4 * iters * chains * 2.0 * 32 * 32 * 64
    n = 1 << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev).fill_(3)
    rgrid = cus * 8
    rsink = torch.empty(rgrid * 256, dtype=torch.int32, device=dev)
    rrun = lambda: lib.fp4p_read_probe(rgrid, buf.data_ptr(), n, rsink.data_ptr(), stream)
    if rrun():
        return None
    rms, _ = time_launches(rrun, 5, 1, dev, graph=False)
    del buf
    return {"fp4_mfma": {"tflops": flops / (ms * 1e-3) / 1e12, "peak": PEAK_TFLOPS["fp4"],
                         "frac_of_peak": flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["fp4"], "shader_ghz": ghz,
                         "probe": f"{cus} workgroups x 4 waves, {chains} independent scaled FP4 32x32x64 chains "
                                  f"per wave, random operand bits, {iters} rounds"},
            "hbm_read": {"gbs": n / (rms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "frac_of_peak": n / (rms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "probe": "1 GiB read once per launch with 16-byte non-temporal loads, 5 launches"}}


def _probe_lib():
    import ctypes
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    lib.fp4p_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.fp4p_read_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.fp4p_timestamp.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def shader_clock_over(run, dev):
    """Average shader clock (GHz) over `run()` (kernels enqueued on the current stream):
    kernels with one workgroup per CU before and after record each XCC's shader clock
    counter and the 100 MHz counter; the median over XCCs of their clocks."""
    import ctypes
    lib = _probe_lib()
    if lib is None:
        return None
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    grid = fp4_device_cus(dev)
    ts = torch.zeros((2, grid, 3), dtype=torch.int64, device=dev)
    if lib.fp4p_timestamp(grid, ts[0].data_ptr(), stream):
        return None
    run()
    if lib.fp4p_timestamp(grid, ts[1].data_ptr(), stream):
        return None
    torch.cuda.synchronize(dev)
    t = ts.cpu().numpy()
    clocks = []
    for x in np.unique(t[0, :, 0]):
        a, b = t[0][t[0, :, 0] == x], t[1][t[1, :, 0] == x]
        if len(a) and len(b):
            dt = float(np.median(b[:, 1]) - np.median(a[:, 1]))
            dr = float(np.median(b[:, 2]) - np.median(a[:, 2]))
            if dr > 0:
                clocks.append(dt / (dr / 100e6) / 1e9)
    return float(np.median(clocks)) if clocks else None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_threads():
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def parity_of_headline(d, D, rows):
    """Parity of the benched 8192^3 output on the oracle's baseline rows (computed again
    here, outside the baseline's timing, so the baseline times the oracle alone)."""
    import oracle
    rows = min(rows, 64)
    ref, S = oracle.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"], rows=(0, rows))
    Dg = D[:rows].float().cpu().numpy().astype(np.float64)
    return {"max_err_over_tol": oracle.parity_ratio(Dg, ref, S, "bf16"), "rows": rows, "out": "bf16"}


def cpu_baseline(d, budget_s=15.0):
    """The oracle, untuned, on whole rows of the 8192^3 workload: a short calibration
    run picks the row count that fills about `budget_s` seconds."""
    import oracle
    threads = cpu_threads()
    oracle.set_threads(threads)
    N, K = 8192, 8192
    t0 = time.perf_counter()
    oracle.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"], rows=(0, threads))
    per_row = (time.perf_counter() - t0) / threads
    rows = int(max(threads, min(8192, budget_s / max(per_row, 1e-6))))
    rows = (rows // threads) * threads
    t0 = time.perf_counter()
    oracle.mx_gemm(d["A"], d["sfA"], d["B"], d["sfB"], rows=(0, rows))
    secs = time.perf_counter() - t0
    return {"value": 2.0 * rows * N * K / secs / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "rows": rows,
            "sample": f"rows 0..{rows - 1} of the 8192^3 MXFP4 GEMM (all 8192 columns, full K), "
                      f"{secs:.1f} s on {threads} threads"}


def _median_time(fn, repeats=3):
    ts, out = [], None
    for _ in range(repeats):
        t0 = time.perf_counter()
        out = fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), out


def oracle_leg(results):
    """After all GPU timing: for each benchmarked workload, the oracle's time on a bounded
    sample of the same inputs (median of 3 runs; whole rows, all columns, full K) and the
    parity ratio max |D_gpu - D| / tol of the benched output on those rows (the bar of the
    oracle module: 1e-5 S, plus one bf16 ulp for bf16 output, plus the FP8 instruction's
    truncation bound for the FP8 blockwise GEMM)."""
    import oracle
    threads = cpu_threads()
    oracle.set_threads(threads)
    out = {}
    # name -> (kind, rows of the sample, output type, FLOPs per row)
    plan = {"mxfp4_256_f32": ("mx", 256, "f32", 2.0 * 256 * 256),
            "nvfp4_1024": ("nv", 1024, "bf16", 2.0 * 1024 * 1024),
            "mxfp4_gemv_8x14336x4096": ("mx", 8, "bf16", 2.0 * 14336 * 4096),
            "w4a8_256x8192x8192": ("w4a8", 8, "bf16", 2.0 * 8192 * 8192),
            "fp8_blockwise_4096": ("fp8b", 16, "bf16", 2.0 * 4096 * 4096)}
    for name, (kind, rows, od, flops_row) in plan.items():
        r = results.get(name)
        if r is None:
            continue
        d = r["d"]
        secs, (ref, S) = _median_time(lambda: oracle.run(kind, d, rows=(0, rows)))
        Dg = r["D"][:rows].float().cpu().numpy().astype(np.float64)
        extra = None
        if kind == "fp8b":
            sub = dict(d, A=d["A"][:rows], sA=d["sA"][:rows])
            extra = oracle.fp8_truncation_bound("fp8b", sub)
        out[name] = {"cpu_baseline": {"value": rows * flops_row / secs / 1e12, "unit": "TFLOP/s", "cores": threads,
                                      "kind": "oracle", "seconds": secs,
                                      "sample": f"rows 0..{rows - 1} (all columns, full K), median of 3 runs"},
                     "parity": {"max_err_over_tol": oracle.parity_ratio(Dg, ref, S, od, extra=extra),
                                "rows": rows, "out": od}}
        log(f"bench: oracle {name}: {secs:.2f} s for {rows} rows; parity {out[name]['parity']['max_err_over_tol']:.3g}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", nargs="*", default=None,
                    help="subset of: mx8192 gemv gemvp w4a8 w4a8p w4a8f6 nv1024 mx256 quant nvquant fp8b skinny "
                         "decode copy peaks")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-graph", action="store_true",
                    help="enqueue launches eagerly instead of replaying a HIP graph (for counter runs)")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/*_counters.txt from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                         f"of `bench.py --only {COUNTED_ONLY} --no-graph`, then exit")
    ap.add_argument("--counters-command", default="", help="the profiling command, recorded with --counters")
    ap.add_argument("--util", metavar="UTIL_DIR",
                    help="write profiles/utilisation_counters.txt from a rocprofv3 --pmc run of "
                         "MfmaUtil LdsUtil LdsBankConflict VALUBusy, then exit")
    args = ap.parse_args()
    if args.counters:
        if not args.counters_command:
            ap.error("--counters needs --counters-command: the profiling command the summary records")
        summarize_counters(args.counters[0], args.counters[1], args.counters_command)
        return
    if args.util:
        if not args.counters_command:
            ap.error("--util needs --counters-command: the profiling command the summary records")
        summarize_util(args.util, args.counters_command)
        return
    global USE_GRAPH
    USE_GRAPH = not args.no_graph
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    fp4.load_library()
    only = set(args.only) if args.only else {"mx8192", "gemv", "gemvp", "w4a8", "w4a8p", "w4a8f6", "nv1024", "mx256",
                                             "quant", "nvquant", "fp8b", "skinny", "decode", "peaks"}
    also = {}
    head = None
    d8192 = None
    kept = {}          # outputs and inputs of the benched workloads, for the oracle leg
    clock_ghz = None
    if "mx8192" in only:
        log("bench: mxfp4 8192^3 ...")
        d8192, head = bench_mx8192(args.steps, args.warmup, dev)
        clock_ghz = head["ghz"]
        log(f"bench: shader clock under the GEMM {clock_ghz} GHz")
        log(f"bench: mxfp4 8192^3 {head['ms'] * 1e3:.1f} us/launch, {head['tflops']:.0f} TFLOP/s")
    if "gemv" in only:
        log("bench: gemv 8x14336x4096 (cold) ...")
        g = bench_gemv(max(args.steps, 100), args.warmup, dev)
        kept["mxfp4_gemv_8x14336x4096"] = g
        log(f"bench: gemv {g['ms'] * 1e3:.2f} us/launch, {g['gbs']:.0f} GB/s "
            f"(eager launches: {g['eager_ms'] * 1e3:.2f} us)")
        traffic = traffic_from_profile("fp4_gemv_8x14336x4096", ["fp4_gemv.hip", "common.hpp"], g["bytes"])
        also["mxfp4_gemv_8x14336x4096"] = {
            "metric": "HBM GB/s", "value": g["gbs"], "ms_per_launch": g["ms"],
            "ms_per_launch_eager": g["eager_ms"],
            "cache": f"cold ({g['copies']} rotating weight copies)",
            "roofline": {"bound": "hbm", "achieved": g["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": g["gbs"] / PEAK_HBM_GBS, "traffic": traffic},
            "algorithmic_bytes": g["bytes"], "tflops": g["tflops"]}
    if "gemvp" in only:
        log("bench: prepacked gemv 8x14336x4096 (cold) ...")
        g = bench_gemv_prepacked(max(args.steps, 100), args.warmup, dev)
        log(f"bench: prepacked gemv {g['ms'] * 1e3:.2f} us/launch, {g['gbs']:.0f} GB/s")
        also["mxfp4_gemv_8x14336x4096_prepacked"] = {
            "metric": "HBM GB/s", "value": g["gbs"], "ms_per_launch": g["ms"],
            "cache": f"cold ({g['copies']} rotating weight copies)",
            "weights": "re-packed once at load time (fp4_gemv_prepack), not timed",
            "roofline": {"bound": "hbm", "achieved": g["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": g["gbs"] / PEAK_HBM_GBS, "traffic": traffic_of("fp4_gemv_prepacked_8x14336x4096")},
            "algorithmic_bytes": g["bytes"]}
    if "w4a8" in only:
        log("bench: w4a8 256x8192x8192 ...")
        w = bench_w4a8(args.steps, args.warmup, dev)
        kept["w4a8_256x8192x8192"] = w
        log(f"bench: w4a8 {w['ms'] * 1e3:.1f} us/launch, {w['tflops']:.0f} TFLOP/s, {w['gbs']:.0f} GB/s")
        also["w4a8_256x8192x8192"] = {
            "metric": "TFLOP/s", "value": w["tflops"], "ms_per_launch": w["ms"],
            "cache": f"cold ({w['copies']} rotating weight copies)",
            "roofline": {"bound": "mfma", "achieved": w["tflops"], "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                         "frac": w["tflops"] / PEAK_TFLOPS["fp8"], "traffic": traffic_of("w4a8_256x8192x8192")},
            "hbm": {"achieved": w["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": w["gbs"] / PEAK_HBM_GBS},
            "algorithmic_bytes": w["bytes"]}
    if "w4a8p" in only:
        log("bench: prepacked w4a8 256x8192x8192 ...")
        w = bench_w4a8_prepacked(args.steps, args.warmup, dev)
        log(f"bench: prepacked w4a8 {w['ms'] * 1e3:.1f} us/launch, {w['tflops']:.0f} TFLOP/s, {w['gbs']:.0f} GB/s")
        also["w4a8_256x8192x8192_prepacked"] = {
            "metric": "TFLOP/s", "value": w["tflops"], "ms_per_launch": w["ms"],
            "cache": f"cold ({w['copies']} rotating weight copies)",
            "weights": "re-packed once at load time (w4a8_prepack), not timed",
            "roofline": {"bound": "mfma", "achieved": w["tflops"], "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                         "frac": w["tflops"] / PEAK_TFLOPS["fp8"],
                         "traffic": traffic_of("w4a8_prepacked_256x8192x8192")},
            "hbm": {"achieved": w["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": w["gbs"] / PEAK_HBM_GBS},
            "algorithmic_bytes": w["bytes"]}
    if "w4a8f6" in only:
        log("bench: fp6 w4a8 256x8192x8192 ...")
        w = bench_w4a8_fp6(args.steps, args.warmup, dev)
        log(f"bench: fp6 w4a8 {w['ms'] * 1e3:.1f} us/launch, {w['tflops']:.0f} TFLOP/s")
        also["w4a8_256x8192x8192_fp6"] = {
            "metric": "TFLOP/s", "value": w["tflops"], "ms_per_launch": w["ms"],
            "cache": f"cold ({w['copies']} rotating weight copies)",
            "weights": "re-encoded once at load time as FP6 E3M2 (w4a8_prepack_fp6), not timed",
            "roofline": {"bound": "mfma", "achieved": w["tflops"], "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                         "frac": w["tflops"] / PEAK_TFLOPS["fp8"],
                         "traffic": traffic_of("w4a8_fp6_256x8192x8192")},
            "hbm": {"achieved": w["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": w["gbs"] / PEAK_HBM_GBS},
            "algorithmic_bytes": w["bytes"], "layout_bytes": w["layout_bytes"]}
    if "nv1024" in only:
        n = bench_nv1024(args.steps, args.warmup, dev)
        kept["nvfp4_1024"] = n
        log(f"bench: nvfp4 1024^3 {n['ms'] * 1e3:.1f} us/launch, {n['tflops']:.0f} TFLOP/s")
        also["nvfp4_1024"] = {"metric": "TFLOP/s", "value": n["tflops"], "ms_per_launch": n["ms"],
                              "roofline": {"bound": "mfma", "achieved": n["tflops"], "peak": PEAK_TFLOPS["bf16"],
                                           "unit": "TFLOP/s", "frac": n["tflops"] / PEAK_TFLOPS["bf16"],
                                           "traffic": traffic_of("nvfp4_gemm_1024")},
                              "algorithmic_bytes": 3276808}
    if "fp8b" in only:
        log("bench: fp8 blockwise 4096^3 ...")
        f = bench_fp8b(args.steps, args.warmup, dev)
        kept["fp8_blockwise_4096"] = f
        log(f"bench: fp8 blockwise 4096^3 {f['ms'] * 1e3:.1f} us/launch, {f['tflops']:.0f} TFLOP/s")
        also["fp8_blockwise_4096"] = {
            "metric": "TFLOP/s", "value": f["tflops"], "ms_per_launch": f["ms"],
            "roofline": {"bound": "mfma", "achieved": f["tflops"], "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                         "frac": f["tflops"] / PEAK_TFLOPS["fp8"], "traffic": traffic_of("fp8_blockwise_4096")},
            "algorithmic_bytes": f["bytes"]}
    if "quant" in only:
        log("bench: mx quantize 8192x8192 fp32 ...")
        q = bench_quant(args.steps, args.warmup, dev)
        log(f"bench: mx quantize {q['ms'] * 1e3:.1f} us/launch, {q['gbs']:.0f} GB/s")
        also["mx_quantize_8192x8192_f32"] = {
            "metric": "HBM GB/s", "value": q["gbs"], "ms_per_launch": q["ms"],
            "roofline": {"bound": "hbm", "achieved": q["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": q["gbs"] / PEAK_HBM_GBS, "traffic": traffic_of("mx_quantize_8192x8192_f32")},
            "algorithmic_bytes": q["bytes"]}
    if "nvquant" in only:
        log("bench: nv quantize 8192x8192 fp32 ...")
        q = bench_nvquant(args.steps, args.warmup, dev)
        log(f"bench: nv quantize {q['ms'] * 1e3:.1f} us/launch, {q['gbs']:.0f} GB/s")
        also["nv_quantize_8192x8192_f32"] = {
            "metric": "HBM GB/s", "value": q["gbs"], "ms_per_launch": q["ms"],
            "roofline": {"bound": "hbm", "achieved": q["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": q["gbs"] / PEAK_HBM_GBS, "traffic": traffic_of("nv_quantize_8192x8192_f32")},
            "algorithmic_bytes": q["bytes"]}
    if "skinny" in only:
        log("bench: mxfp4 batched/split-K 128x8192x8192 (cold weights) ...")
        k = bench_skinny(args.steps, args.warmup, dev)
        log(f"bench: mxfp4 128x8192x8192 split {k['auto']['splits']}: {k['auto']['ms'] * 1e3:.1f} us "
            f"({k['auto']['tflops']:.0f} TFLOP/s); unsplit {k['none']['ms'] * 1e3:.1f} us")
        # the split kernel and its reduction together, when both have current counters
        ts, tr = traffic_of("mxfp4_split_k_128x8192x8192"), traffic_of("mxfp4_split_k_reduce_128x8192x8192")
        split_traffic = ts + tr if ts is not None and tr is not None else None
        also["mxfp4_split_k_128x8192x8192"] = {
            "metric": "TFLOP/s", "value": k["auto"]["tflops"], "ms_per_launch": k["auto"]["ms"],
            "splits": k["auto"]["splits"], "unsplit_ms_per_launch": k["none"]["ms"],
            "cache": f"cold ({k['copies']} rotating weight copies)",
            "roofline": {"bound": "mfma", "achieved": k["auto"]["tflops"], "peak": PEAK_TFLOPS["fp4"],
                         "unit": "TFLOP/s", "frac": k["auto"]["tflops"] / PEAK_TFLOPS["fp4"],
                         "traffic": split_traffic}}
    if "decode" in only:
        log("bench: decode (M = 8, 32) and skinny (M = 64) W4A8 / NVFP4 on 8192x8192 weights (cold) ...")
        k = bench_decode(args.steps, args.warmup, dev)
        for M, label in ((8, "decode_8x8192x8192"), (32, "decode_32x8192x8192"), (64, "skinny_64x8192x8192")):
            r = k[M]
            log(f"bench: {label}: " + ", ".join(f"{n} {r[n]['us']:.1f} us" for n in ("w4a8", "w4a8_prepacked", "nvfp4")))
            entry = {"metric": "us per launch", "cache": f"cold ({k['copies']} rotating weight copies)",
                     "kernels": ("decode kernels, one 16-token tile" if M <= 16 else
                                 "decode kernels, two 16-token tiles" if M <= 32 else "K-split GEMMs (library's choice)"),
                     "splits": r["splits"]}
            for n in ("w4a8", "w4a8_prepacked", "nvfp4"):
                entry[n] = {"us": r[n]["us"], "tflops": r[n]["tflops"], "algorithmic_bytes": r[n]["bytes"],
                            "roofline": {"bound": "hbm", "achieved": r[n]["gbs"], "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": r[n]["gbs"] / PEAK_HBM_GBS,
                                         "traffic": decode_traffic(n, M), "traffic_source": TRAFFIC_SOURCE}}
                if M <= 16 and n != "w4a8_prepacked":
                    entry[n]["roofline"]["utilisation"] = util_from_profile(f"decode_8x8192x8192_{n}")
            also[label] = entry
    if "copy" in only:
        c = bench_copy(dev)
        log(f"bench: copy 512 MiB {c['ms'] * 1e3:.1f} us, {c['gbs']:.0f} GB/s (read+write)")
        also["copy_512MiB"] = c
    if "mx256" in only:
        s = bench_mx256(args.steps, args.warmup, dev)
        kept["mxfp4_256_f32"] = s
        also["mxfp4_256_f32"] = {"metric": "TFLOP/s", "value": s["tflops"], "ms_per_launch": s["ms"]}
    peaks = None
    if "peaks" in only:
        log("bench: measured ceilings (FP4 matrix pipe, HBM read) ...")
        peaks = measure_peaks(dev, fp4_device_cus(dev))
        if peaks:
            log(f"bench: FP4 MFMA-only {peaks['fp4_mfma']['tflops']:.0f} TFLOP/s at "
                f"{peaks['fp4_mfma']['shader_ghz']:.2f} GHz; HBM read {peaks['hbm_read']['gbs']:.0f} GB/s")

    line = {"metric": "TFLOP/s MXFP4 GEMM 8192^3 (% MFMA peak); FP4 GEMV HBM GB/s (% of 8 TB/s)",
            "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "fp4e2m1", "data": "synthetic",
            "config": {"workload": "mxfp4_gemm_8192x8192x8192", "M": 8192, "N": 8192, "K": 8192,
                       "scale": "e8m0 per 32", "out": "bf16", "inputs": "N(0,1) max-abs MX-quantized, seed 0"}}
    if head is not None:
        line["value"] = head["tflops"]
        line["ms_per_step"] = head["ms"]
        line["roofline"] = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_TFLOPS["fp4"],
                            "unit": "TFLOP/s", "frac": head["tflops"] / PEAK_TFLOPS["fp4"],
                            "traffic": traffic_from_profile("mxfp4_gemm_8192", ["mxfp4_gemm.hip", "common.hpp"],
                                                            head["bytes"]),
                            "traffic_source": TRAFFIC_SOURCE, "shader_ghz_during_run": clock_ghz}
        if peaks:
            line["roofline"]["measured_peak"] = peaks["fp4_mfma"]
        if not args.no_cpu:
            log("bench: cpu oracle baseline ...")
            line["cpu_baseline"] = cpu_baseline(d8192)
            line["cpu_baseline"]["cpu_model"] = cpu_model()
            line["parity"] = parity_of_headline(d8192, head["D"], line["cpu_baseline"]["rows"])
    if peaks:
        for key in ("mxfp4_gemv_8x14336x4096", "mxfp4_gemv_8x14336x4096_prepacked", "mx_quantize_8192x8192_f32",
                    "nv_quantize_8192x8192_f32"):
            if key in also:
                also[key]["roofline"]["measured_peak"] = peaks["hbm_read"]
        also["measured_peaks"] = peaks
    if not args.no_cpu and kept:
        for name, res in oracle_leg(kept).items():
            if name in also:
                also[name].update(res)
    for entry in also.values():
        if isinstance(entry, dict) and isinstance(entry.get("roofline"), dict):
            entry["roofline"]["traffic_source"] = TRAFFIC_SOURCE
    # MFMA / LDS / VALU utilisation of each kernel from the committed counter run
    # (null when the kernel changed since the counters were taken).
    if "roofline" in line:
        line["roofline"]["utilisation"] = util_from_profile("mxfp4_gemm_8192x8192x8192")
    for key, entry in also.items():
        if isinstance(entry, dict) and "roofline" in entry and any(key == k for k, _, _ in UTIL_KERNELS):
            entry["roofline"]["utilisation"] = util_from_profile(key)
    line["also"] = also
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
