"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.c is built with -fsanitize=address,undefined (host code only; nothing here
touches a GPU), loaded into a child Python with the sanitizer runtimes preloaded, and
every quick pin (the same list the mutant tests use) runs against it.  Any
out-of-bounds access, use after free or undefined operation in the oracle aborts the
child and fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

RUNNER = """
import ctypes, sys
sys.path.insert(0, {root!r})
import oracle
from tests import test_oracle_mutants as mt
oracle._lib = oracle.bind(ctypes.CDLL({so!r}))
n = 0
for fn, kw in mt._quick_pins():
    fn(oracle_lib=oracle, **kw)
    n += 1
print("quick pins run:", n)
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_quick_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", so, SRC, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, so=so)], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "quick pins run:" in r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
