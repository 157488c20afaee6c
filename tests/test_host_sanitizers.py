"""The library's host code (argument validation, kernel selection, launch set-up) under
AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled with the sanitizers on the host side only (device code is
built as usual and never runs here), linked into a separate library, and the C-ABI
validation tests run against it in a child Python with the sanitizer runtime
preloaded.  Those tests call every entry point with invalid or empty arguments, so
nothing reaches a GPU; a host memory or undefined-behaviour error aborts the child.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from block_scaled_precision_e2m1_amd import _build  # noqa: E402

HOST_SANITIZERS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()

RUNNER = """
import sys
sys.path.insert(0, {root!r})
import block_scaled_precision_e2m1_amd as fp4
fp4._LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {test!r}]))
"""


def test_abi_validation_under_host_asan_and_ubsan(tmp_path):
    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "llvm", "bin", "clang"),
                         "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True).stdout.strip()
    if not (os.path.isabs(rt) and os.path.exists(rt)):
        pytest.skip("clang's AddressSanitizer runtime not found")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={_build.ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fno-omit-frame-pointer"] + HOST_SANITIZERS

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        subprocess.run([cc] + flags + lang + ["-c", src, "-o", obj], check=True, capture_output=True)
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, _build.sources()))
    lib = str(tmp_path / "libfp4gemm_san.so")
    subprocess.run([cc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC"] + HOST_SANITIZERS + ["-o", lib] + objs,
                   check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, lib=lib, test=os.path.join(ROOT, "tests", "test_abi.py"))],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
