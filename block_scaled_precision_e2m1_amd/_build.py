"""Build the gfx950 HIP library libfp4gemm.so in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only and linked into one shared
library next to this file.  Packed FP32 VALU instructions are disabled
(-packed-fp32-ops): the kernels use plain scalar float code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4gemm.so")
BUILD = os.path.join(HERE, "_build")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


# Per-file device flags.  w4a8_fp6.hip: the MFMA results are folded into fp32
# accumulators by VALU after every K group, so they are wanted in VGPRs (no AGPR reads).
DEVICE_FLAGS = {"w4a8_fp6.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc] + COMMON + DEVICE_FLAGS.get(os.path.basename(src), []) + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        if out.strip() and verbose:
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    build_probe(cc)
    return LIB


PROBE_SRC = os.path.join(HERE, "probe", "peak_probe.hip")
PROBE_LIB = os.path.join(HERE, "libfp4probe.so")


def build_probe(cc=None) -> str:
    """The benchmark's measurement kernels (matrix-pipe and HBM-read ceilings): a separate
    shared library, not part of the operations' ABI."""
    cc = cc or hipcc()
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([cc] + COMMON + ["-shared", "-x", "hip", PROBE_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
