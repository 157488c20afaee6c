"""Host-side checks of the C ABI: the library loads, exports every entry point
that include/fp4gemm.h declares, and rejects invalid arguments with the
documented status codes before touching any device (no GPU needed: every call
here fails validation or has an empty output, so nothing is launched)."""
import ctypes
import os
import re

import pytest
import torch

import block_scaled_precision_e2m1_amd as fp4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4gemm.h")

OK, EINVAL, EUNSUP, EALIGN, EHIP = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return fp4.load_library()


def test_header_declares_the_operations():
    assert declared_functions() == sorted(["mx_fp4_gemm", "mx_fp4_gemm_batched", "mx_fp4_gemm_batched_noalloc",
                                            "mx_fp4_gemm_workspace_size",
                                            "nv_fp4_gemm", "w4a8_gemm", "fp4_gemv", "fp4_gemv_prepack_size",
                                            "fp4_gemv_prepack", "fp4_gemv_prepacked",
                                            "w4a8_prepack_size", "w4a8_prepack", "w4a8_prepack_e4m3",
                                            "w4a8_gemm_prepacked", "w4a8_prepack_fp6_size", "w4a8_prepack_fp6",
                                            "w4a8_gemm_prepacked_fp6", "w4a8_fp6_workspace_size",
                                            "w4a8_gemm_prepacked_fp6_split",
                                            "nv_fp4_gemm_batched", "w4a8_gemm_batched",
                                            "nv_fp4_gemm_workspace_size", "w4a8_gemm_workspace_size",
                                            "nv_fp4_gemm_split", "w4a8_gemm_split", "w4a8_gemm_prepacked_split",
                                            "mx_fp4_quantize", "nv_fp4_quantize", "fp8_blockwise_gemm",
                                            "fp4g_status_string"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(fp4.SYMBOLS) == set(declared_functions())


def test_library_is_gfx950_only():
    out = os.popen(f"/opt/rocm/bin/roc-obj-ls {fp4.library_path()} 2>/dev/null").read()
    if not out.strip():
        pytest.skip("roc-obj-ls unavailable")
    assert "gfx950" in out
    assert "gfx942" not in out and "gfx90a" not in out


def test_status_strings(lib):
    for s in range(5):
        assert fp4.fp4g_status_string(s)
    assert fp4.fp4g_status_string(99) == "unknown status"


# Fake, aligned, non-overlapping "device" addresses: validation never dereferences them.
A_, SA_, B_, SB_, D_ = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def mx(lib, M, N, K, A=A_, sA=SA_, B=B_, sB=SB_, D=D_, dt=0):
    return lib.mx_fp4_gemm(M, N, K, A, sA, B, sB, D, dt, None)


def test_invalid_sizes(lib):
    assert mx(lib, -1, 4, 128) == EINVAL
    assert mx(lib, 4, -1, 128) == EINVAL
    assert mx(lib, 4, 4, -128) == EINVAL
    assert mx(lib, 1 << 31, 4, 128) == EINVAL
    assert mx(lib, 4, 4, 64) == EUNSUP
    assert mx(lib, 4, 4, 100) == EUNSUP


def test_output_size_limit(lib):
    # 2^30 x 2^30 outputs would overflow the byte counts of the range checks: rejected
    assert mx(lib, 1 << 30, 1 << 30, 128) == EINVAL
    assert lib.mx_fp4_gemm_batched(4, 1 << 27, 1 << 27, 128, A_, SA_, B_, SB_, D_, 1, 0, None, 0, None) == EINVAL


def test_bad_output_type(lib):
    assert mx(lib, 4, 4, 128, dt=2) == EINVAL
    assert mx(lib, 4, 4, 128, dt=-1) == EINVAL


def test_null_pointers(lib):
    assert mx(lib, 4, 4, 128, A=None) == EINVAL
    assert mx(lib, 4, 4, 128, sA=None) == EINVAL
    assert mx(lib, 4, 4, 128, B=None) == EINVAL
    assert mx(lib, 4, 4, 128, sB=None) == EINVAL
    assert mx(lib, 4, 4, 128, D=None) == EINVAL


def test_alignment(lib):
    assert mx(lib, 4, 4, 128, A=A_ + 8) == EALIGN
    assert mx(lib, 4, 4, 128, B=B_ + 4) == EALIGN
    assert mx(lib, 4, 4, 128, D=D_ + 2) == EALIGN
    assert mx(lib, 4, 4, 128, sA=SA_ + 2) == EALIGN
    assert mx(lib, 4, 4, 128, sB=SB_ + 1) == EALIGN


def test_output_overlapping_an_input(lib):
    assert mx(lib, 4, 4, 128, D=A_) == EINVAL
    assert mx(lib, 4, 4, 1024, D=SB_ + 64) == EINVAL   # sfB spans 4 * 32 bytes
    assert mx(lib, 4, 4, 1024, D=B_ + 1024) == EINVAL  # B spans 4 * 512 bytes


def test_empty_outputs_are_noops(lib):
    assert mx(lib, 0, 4, 128, A=None, sA=None, B=None, sB=None, D=None) == OK
    assert mx(lib, 4, 0, 128, A=None, sA=None, B=None, sB=None, D=None) == OK
    assert lib.w4a8_gemm(0, 5, 256, None, None, None, None, None, 1, None) == OK
    assert lib.nv_fp4_gemm(3, 0, 256, None, None, 1.0, None, None, 1.0, None, 1, None) == OK


def test_gemv_token_limit(lib):
    # 1..16 tokens at any K, 17..32 tokens at K <= 16384 (the second token tile)
    assert lib.fp4_gemv(33, 64, 128, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP
    assert lib.fp4_gemv(17, 64, 16512, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP
    assert lib.fp4_gemv(4, 64, 96, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP


def test_nv_and_w4a8_validation(lib):
    assert lib.nv_fp4_gemm(4, 4, 128, None, SA_, 1.0, B_, SB_, 1.0, D_, 0, None) == EINVAL
    assert lib.nv_fp4_gemm(4, 4, 192, A_, SA_, 1.0, B_, SB_, 1.0, D_, 0, None) == EUNSUP
    assert lib.w4a8_gemm(4, 4, 128, A_, None, B_, SB_, D_, 0, None) == EINVAL
    assert lib.w4a8_gemm(4, 4, 128, A_, SA_ + 2, B_, SB_, D_, 0, None) == EALIGN
    assert lib.w4a8_gemm(4, 4, 128, A_, SA_, B_, SB_, A_ + 64, 0, None) == EINVAL


def test_fp8_blockwise_validation(lib):
    f = lib.fp8_blockwise_gemm
    assert f(0, 4, 128, None, None, None, None, None, 1, None) == OK
    assert f(4, 4, 192, A_, SA_, B_, SB_, D_, 0, None) == EUNSUP
    assert f(4, 4, 128, A_, None, B_, SB_, D_, 0, None) == EINVAL
    assert f(4, 4, 128, A_ + 8, SA_, B_, SB_, D_, 0, None) == EALIGN
    assert f(4, 4, 128, A_, SA_ + 2, B_, SB_, D_, 0, None) == EALIGN
    assert f(4, 4, 128, A_, SA_, B_, SB_, A_ + 256, 0, None) == EINVAL   # D inside A


def test_quantizer_validation(lib):
    q = lib.mx_fp4_quantize
    assert q(0, 64, None, 0, None, None, None) == OK                 # empty: nothing read
    assert q(4, 0, None, 1, None, None, None) == OK
    assert q(-1, 64, A_, 0, B_, SB_, None) == EINVAL
    assert q(4, 64, A_, 2, B_, SB_, None) == EINVAL                  # bad input type
    assert q(4, 48, A_, 0, B_, SB_, None) == EUNSUP                  # K % 32
    assert q(4, 64, None, 0, B_, SB_, None) == EINVAL
    assert q(4, 64, A_ + 4, 0, B_, SB_, None) == EALIGN
    assert q(4, 64, A_, 0, B_ + 2, SB_, None) == EALIGN
    assert q(4, 64, A_, 0, A_ + 512, SB_, None) == EINVAL            # codes inside X (1 KB of fp32)
    assert q(4, 64, A_, 1, B_, B_ + 64, None) == EINVAL              # scales inside codes
    assert q(1 << 30, 1 << 30, A_, 0, B_, SB_, None) == EINVAL       # rows*K above 2^50


def test_nv_quantizer_validation(lib):
    q = lib.nv_fp4_quantize
    assert q(0, 64, None, 0, 1.0, None, None, None) == OK             # empty: nothing read
    assert q(4, 0, None, 1, 1.0, None, None, None) == OK
    assert q(-1, 64, A_, 0, 1.0, B_, SB_, None) == EINVAL
    assert q(4, 64, A_, 2, 1.0, B_, SB_, None) == EINVAL              # bad input type
    for g in (0.0, -2.0, float("inf"), float("nan")):                 # global scale finite and > 0
        assert q(4, 64, A_, 0, g, B_, SB_, None) == EINVAL
    assert q(4, 40, A_, 0, 1.0, B_, SB_, None) == EUNSUP              # K % 16
    assert q(4, 64, None, 0, 1.0, B_, SB_, None) == EINVAL
    assert q(4, 64, A_ + 4, 0, 1.0, B_, SB_, None) == EALIGN
    assert q(4, 64, A_, 0, 1.0, B_ + 4, SB_, None) == EALIGN          # codes 8-byte aligned
    assert q(4, 64, A_, 0, 1.0, A_ + 512, SB_, None) == EINVAL        # codes inside X
    assert q(4, 64, A_, 1, 1.0, B_, B_ + 64, None) == EINVAL          # scales inside codes
    assert q(1 << 30, 1 << 30, A_, 0, 1.0, B_, SB_, None) == EINVAL   # rows*K above 2^50


def test_w4a8_prepack_e4m3_validation(lib):
    f = lib.w4a8_prepack_e4m3
    assert f(0, 128, None, None, 1, None, None, None) == OK           # empty: nothing touched
    assert f(4, 128, A_, SB_, 2, B_, D_, None) == EINVAL              # stride 1 or 8 only
    assert f(4, 192, A_, SB_, 1, B_, D_, None) == EUNSUP
    assert f(4, 128, A_, None, 8, B_, D_, None) == EINVAL
    assert f(4, 128, A_ + 8, SB_, 1, B_, D_, None) == EALIGN
    assert f(4, 128, A_, SB_, 1, B_, D_ + 2, None) == EALIGN          # Sp 4-byte aligned
    assert f(4, 128, A_, SB_, 8, A_ + 16, D_, None) == EINVAL          # Bp over B


W_ = 0x10000000     # fake workspace address, far from the operands


def mxb(lib, L, M, N, K, A=A_, sA=SA_, B=B_, sB=SB_, D=D_, dt=1, splits=0, ws=None, wsb=0):
    return lib.mx_fp4_gemm_batched(L, M, N, K, A, sA, B, sB, D, dt, splits, ws, wsb, None)


def test_batched_validation(lib):
    assert mxb(lib, -1, 4, 4, 128) == EINVAL
    assert mxb(lib, 2, 4, 4, 128, splits=-1) == EINVAL
    assert mxb(lib, 1 << 20, 1 << 11, 4, 128) == EINVAL               # L*M = 2^31
    assert mxb(lib, 2, 4, 4, 192) == EUNSUP
    assert mxb(lib, 2, 4, 4, 128, dt=3) == EINVAL
    assert mxb(lib, 0, 4, 4, 128, A=None, sA=None, B=None, sB=None, D=None) == OK
    assert mxb(lib, 2, 4, 4, 128, ws=None, wsb=64) == EINVAL          # bytes without memory
    assert mxb(lib, 2, 4, 4, 128, A=None) == EINVAL
    assert mxb(lib, 2, 4, 4, 128, sB=SB_ + 2) == EALIGN
    # D inside the second problem of A: A spans L*M*K/2 = 2*4*512 bytes
    assert mxb(lib, 2, 4, 4, 1024, D=A_ + 2048) == EINVAL
    # workspace checks apply only when a split may run (splits != 1, bytes > 0)
    assert mxb(lib, 2, 4, 4, 1024, splits=2, ws=W_ + 8, wsb=4096) == EALIGN
    assert mxb(lib, 2, 4, 4, 1024, splits=2, ws=D_, wsb=4096) == EINVAL   # overlaps D
    assert mxb(lib, 2, 4, 4, 1024, splits=2, ws=B_, wsb=4096) == EINVAL   # overlaps B


def test_noalloc_validation(lib):
    f = lib.mx_fp4_gemm_batched_noalloc

    def call(L, M, N, K, A=A_, sA=SA_, B=B_, sB=SB_, D=D_, dt=1, splits=0):
        return f(L, M, N, K, A, sA, B, sB, D, dt, splits, None)

    assert call(-1, 4, 4, 128) == EINVAL
    assert call(2, 4, 4, 128, splits=-1) == EINVAL
    assert call(2, 4, 4, 192) == EUNSUP
    assert call(2, 4, 4, 128, dt=3) == EINVAL
    assert call(0, 4, 4, 128, A=None, sA=None, B=None, sB=None, D=None) == OK
    assert call(2, 4, 4, 128, A=None) == EINVAL
    assert call(2, 4, 4, 128, sB=SB_ + 2) == EALIGN
    assert call(2, 4, 4, 1024, D=A_ + 2048) == EINVAL
    # an explicit split whose partial sums exceed the 32 MiB scratch is refused before
    # any device call: 1 x 512 x 4096 x 8192 at s = 5 needs 40 MiB (operands 1 GiB apart)
    far = dict(A=1 << 30, sA=2 << 30, B=3 << 30, sB=4 << 30, D=5 << 30)
    assert call(1, 512, 4096, 8192, splits=5, **far) == EUNSUP
    assert call(2, 1024, 1024, 8192, splits=16, **far) == EUNSUP


def test_nv_and_w4a8_batched_validation(lib):
    nb, wb = lib.nv_fp4_gemm_batched, lib.w4a8_gemm_batched
    assert nb(-1, 4, 4, 128, A_, SA_, 1.0, B_, SB_, 1.0, D_, 1, None) == EINVAL
    assert nb(0, 4, 4, 128, None, None, 1.0, None, None, 1.0, None, 1, None) == OK
    assert nb(65536, 4, 4, 128, A_, SA_, 1.0, B_, SB_, 1.0, D_, 1, None) == EUNSUP   # grid y
    assert nb(2, 4, 4, 192, A_, SA_, 1.0, B_, SB_, 1.0, D_, 1, None) == EUNSUP
    assert nb(2, 4, 4, 1024, A_, SA_, 1.0, B_, SB_, 1.0, A_ + 2048, 1, None) == EINVAL  # D in 2nd A
    assert wb(-1, 4, 4, 128, A_, SA_, B_, SB_, D_, 1, None) == EINVAL
    assert wb(0, 4, 4, 128, None, None, None, None, None, 1, None) == OK
    assert wb(65536, 4, 4, 128, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP
    assert wb(2, 4, 4, 128, A_, None, B_, SB_, D_, 1, None) == EINVAL
    assert wb(2, 4, 4, 128, A_, SA_ + 2, B_, SB_, D_, 1, None) == EALIGN
    assert wb(3, 4, 4, 128, A_, SA_, B_, SB_, SA_ + 32, 1, None) == EINVAL           # D in sa (48 B)


def test_workspace_size(lib):
    n = ctypes.c_size_t(123)
    f = lib.mx_fp4_gemm_workspace_size
    assert f(2, 4, 4, 128, 0, None) == EINVAL
    assert f(-1, 4, 4, 128, 0, ctypes.byref(n)) == EINVAL
    assert f(1, 4, 4, 96, 0, ctypes.byref(n)) == EUNSUP
    assert f(3, 128, 128, 4096, 1, ctypes.byref(n)) == OK and n.value == 0        # no split
    assert f(3, 128, 128, 0, 4, ctypes.byref(n)) == OK and n.value == 0          # empty sum
    assert f(3, 128, 128, 256, 4, ctypes.byref(n)) == OK and n.value == 0        # one K stage
    assert f(3, 128, 128, 4096, 4, ctypes.byref(n)) == OK and n.value == 3 * 4 * 128 * 128 * 4
    assert f(1, 64, 64, 8192, 100, ctypes.byref(n)) == OK and n.value == 16 * 64 * 64 * 4   # clamped
    assert f(1, 64, 64, 640, 100, ctypes.byref(n)) == OK and n.value == 5 * 64 * 64 * 4     # K/128 stages
    assert f(1, 8192, 8192, 8192, 0, ctypes.byref(n)) == OK and n.value == 0     # fills the GPU
    assert f(1, 32, 8192, 4096, 0, ctypes.byref(n)) == OK and n.value == 0       # the decode GEMV
    assert f(1, 32, 8192, 4096, 4, ctypes.byref(n)) == OK and n.value == 4 * 32 * 8192 * 4   # asked to split
    assert f(1, 64, 8192, 8192, 0, ctypes.byref(n)) == OK
    assert n.value > 0 and n.value % (64 * 8192 * 4) == 0 and n.value <= 16 * 64 * 8192 * 4


def test_prepack_validation(lib):
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    f = lib.fp4_gemv_prepack_size
    assert f(37, 640, ctypes.byref(wb), ctypes.byref(sb)) == OK
    assert wb.value == 3 * 5 * 1024 and sb.value == 3 * 2 * 256     # G = 3, KT = 5, KC = 2
    assert f(37, 640, None, ctypes.byref(sb)) == EINVAL
    assert f(-1, 640, ctypes.byref(wb), ctypes.byref(sb)) == EINVAL
    assert f(4, 96, ctypes.byref(wb), ctypes.byref(sb)) == EUNSUP
    p = lib.fp4_gemv_prepack
    assert p(0, 128, None, None, None, None, None) == OK
    assert p(4, 128, B_, SB_, None, D_, None) == EINVAL
    assert p(4, 128, B_ + 4, SB_, A_, D_, None) == EALIGN
    assert p(4, 128, B_, SB_, A_, D_ + 2, None) == EALIGN
    assert p(4, 128, B_, SB_, B_, D_, None) == EINVAL                  # packed weights over B
    assert p(4, 128, B_, SB_, A_, A_ + 512, None) == EINVAL            # Sp inside Bp (1 KB)
    g = lib.fp4_gemv_prepacked
    assert g(0, 16, 128, None, None, None, None, None, 1, None) == OK
    assert g(17, 16, 128, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP
    assert g(4, 16, 128, A_, SA_, None, SB_, D_, 1, None) == EINVAL
    assert g(4, 16, 128, A_, SA_, B_ + 8, SB_, D_, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_, SB_ + 2, D_, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_, SB_, B_ + 256, 1, None) == EINVAL   # D inside Bp


def test_w4a8_prepack_validation(lib):
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    f = lib.w4a8_prepack_size
    assert f(20, 384, ctypes.byref(wb), ctypes.byref(sb)) == OK
    assert wb.value == 2 * 3 * 1024 and sb.value == 3 * 32 * 4          # G16 = 2, KG = 3
    assert f(20, 384, ctypes.byref(wb), None) == EINVAL
    assert f(20, 200, ctypes.byref(wb), ctypes.byref(sb)) == EUNSUP
    p = lib.w4a8_prepack
    assert p(0, 128, None, None, None, None, None) == OK
    assert p(4, 128, B_, None, A_, D_, None) == EINVAL
    assert p(4, 128, B_, SB_ + 1, A_, D_, None) == EALIGN
    assert p(4, 128, B_, SB_, A_ + 8, D_, None) == EALIGN
    assert p(4, 128, B_, SB_, A_, B_, None) == EINVAL                   # Sp over B
    g = lib.w4a8_gemm_prepacked
    assert g(0, 16, 128, None, None, None, None, None, 1, None) == OK
    assert g(4, 16, 192, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP
    assert g(4, 16, 128, A_, None, B_, SB_, D_, 1, None) == EINVAL
    assert g(4, 16, 128, A_ + 4, SA_, B_, SB_, D_, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_, SB_ + 2, D_, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_, SB_, SB_ + 32, 1, None) == EINVAL   # D inside Sp (64 B)


def test_w4a8_prepack_fp6_validation(lib):
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    f = lib.w4a8_prepack_fp6_size
    assert f(40, 384, ctypes.byref(wb), ctypes.byref(sb)) == OK
    assert wb.value == 2 * 3 * 3072 and sb.value == 3 * 48 * 4          # G32 = 2, G16 = 3, KG = 3
    assert f(40, 384, None, ctypes.byref(sb)) == EINVAL
    assert f(40, 200, ctypes.byref(wb), ctypes.byref(sb)) == EUNSUP
    assert f(-1, 128, ctypes.byref(wb), ctypes.byref(sb)) == EINVAL
    p = lib.w4a8_prepack_fp6
    assert p(0, 128, None, None, None, None, None) == OK
    assert p(4, 192, B_, SB_, A_, D_, None) == EUNSUP
    assert p(4, 128, B_, None, A_, D_, None) == EINVAL
    assert p(4, 128, B_ + 8, SB_, A_, D_, None) == EALIGN
    assert p(4, 128, B_, SB_ + 1, A_, D_, None) == EALIGN
    assert p(4, 128, B_, SB_, A_ + 8, D_, None) == EALIGN
    assert p(4, 128, B_, SB_, A_, D_ + 2, None) == EALIGN
    assert p(4, 128, B_, SB_, A_, B_, None) == EINVAL                   # Sp over B
    assert p(4, 128, B_, SB_, B_, D_, None) == EINVAL                   # Bp6 over B
    g = lib.w4a8_gemm_prepacked_fp6
    assert g(0, 16, 128, None, None, None, None, None, 1, None) == OK
    assert g(4, 16, 128, None, None, None, None, None, 2, None) == EINVAL   # output type
    assert g(4, 16, 192, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP
    assert g(4, 16, 128, A_, None, B_, SB_, D_, 1, None) == EINVAL
    assert g(4, 16, 128, A_ + 4, SA_, B_, SB_, D_, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_ + 4, SB_, D_, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_, SB_ + 4, D_, 1, None) == EALIGN      # Sp needs 16 bytes here
    assert g(4, 16, 128, A_, SA_ + 2, B_, SB_, D_, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_, SB_, D_ + 8, 1, None) == EALIGN
    assert g(4, 16, 128, A_, SA_, B_, SB_, B_ + 1024, 1, None) == EINVAL   # D inside Bp6 (3072 B)
    assert g(4, 16, (1 << 23) + 128, A_, SA_, B_, SB_, D_, 1, None) == EUNSUP
    sp = lib.w4a8_gemm_prepacked_fp6_split
    assert sp(0, 16, 128, None, None, None, None, None, 1, 0, None, 0, None) == OK
    assert sp(4, 16, 128, A_, SA_, B_, SB_, D_, 1, -1, None, 0, None) == EINVAL      # negative split
    assert sp(4, 16, 128, A_, SA_, B_, SB_, D_, 1, 0, None, 64, None) == EINVAL      # bytes without a workspace
    assert sp(4, 16, 128, A_, SA_, B_, SB_ + 4, D_, 1, 0, None, 0, None) == EALIGN
    assert sp(4, 16, 256, A_, SA_, B_, SB_, D_, 1, 2, D_ + 8, 4096, None) == EALIGN   # workspace alignment
    assert sp(4, 16, 256, A_, SA_, B_, SB_, D_, 1, 2, A_, 4096, None) == EINVAL       # workspace over A
    nb = ctypes.c_size_t(7)
    assert lib.w4a8_fp6_workspace_size(256, 8192, 8192, 1, ctypes.byref(nb)) == OK and nb.value == 0
    assert lib.w4a8_fp6_workspace_size(256, 8192, 8192, 0, None) == EINVAL
    assert lib.w4a8_fp6_workspace_size(256, 8192, 200, 0, ctypes.byref(nb)) == EUNSUP


def test_binding_rejects_host_tensors():
    A = torch.zeros((4, 64), dtype=torch.uint8)
    s = torch.zeros((4, 4), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        fp4.mx_fp4_gemm(A, s, A, s)
    with pytest.raises(TypeError):
        fp4.mx_fp4_gemm(A.numpy(), s, A, s)


def test_split_validation(lib):
    """The K-split NVFP4 and W4A8 entry points: sizes, workspace rules (NULL with bytes,
    alignment, overlap with D or an input) and the workspace-size query, all refused or
    answered before any device call."""
    nv, w4, wp = lib.nv_fp4_gemm_split, lib.w4a8_gemm_split, lib.w4a8_gemm_prepacked_split
    W = 0x600000

    def nvc(L, M, N, K, D=D_, dt=1, splits=0, ws=W, wbytes=1 << 20, A=A_):
        return nv(L, M, N, K, A, SA_, 1.0, B_, SB_, 1.0, D, dt, splits, ws, wbytes, None)

    def w4c(L, M, N, K, D=D_, dt=1, splits=0, ws=W, wbytes=1 << 20, A=A_):
        return w4(L, M, N, K, A, SA_, B_, SB_, D, dt, splits, ws, wbytes, None)

    def wpc(M, N, K, D=D_, dt=1, splits=0, ws=W, wbytes=1 << 20, A=A_):
        return wp(M, N, K, A, SA_, B_, SB_, D, dt, splits, ws, wbytes, None)

    for call in (nvc, w4c):
        assert call(-1, 4, 4, 128) == EINVAL
        assert call(2, 4, 4, 128, splits=-1) == EINVAL
        assert call(2, 4, 4, 192) == EUNSUP
        assert call(2, 4, 4, 128, dt=3) == EINVAL
        assert call(65536, 4, 4, 128) == EUNSUP
        assert call(0, 4, 4, 128) == OK
        assert call(2, 64, 64, 1024, ws=None) == EINVAL                 # NULL workspace with bytes
        assert call(2, 64, 64, 1024, A=None) == EINVAL
        assert call(2, 64, 64, 1024, ws=W + 8) == EALIGN
        assert call(2, 64, 64, 1024, ws=D_) == EINVAL                   # workspace over D
        assert call(2, 64, 64, 1024, ws=B_) == EINVAL                   # workspace over B
    assert wpc(-1, 4, 128) == EINVAL
    assert wpc(4, 4, 128, splits=-1) == EINVAL
    assert wpc(64, 64, 1024, ws=None) == EINVAL
    assert wpc(64, 64, 1024, ws=W + 4) == EALIGN
    assert wpc(64, 64, 1024, ws=SA_) == EINVAL
    assert wpc(0, 64, 1024) == OK

    n = ctypes.c_size_t(7)
    for f in (lib.nv_fp4_gemm_workspace_size, lib.w4a8_gemm_workspace_size):
        assert f(1, 64, 8192, 8192, 1, ctypes.byref(n)) == OK and n.value == 0     # never splits
        assert f(1, 16, 8192, 8192, 0, ctypes.byref(n)) == OK and n.value == 0     # decode kernel
        assert f(1, 32, 8192, 8192, 4, ctypes.byref(n)) == OK and n.value == 0     # two token tiles
        assert f(1, 33, 8192, 8192, 4, ctypes.byref(n)) == OK and n.value == 4 * 33 * 8192 * 4
        assert f(1, 17, 8192, 8448, 2, ctypes.byref(n)) == OK and n.value == 2 * 17 * 8192 * 4   # K > 8192
        assert f(1, 64, 8192, 8192, 4, ctypes.byref(n)) == OK and n.value == 4 * 64 * 8192 * 4
        assert f(1, 64, 8192, 256, 16, ctypes.byref(n)) == OK and n.value <= 2 * 64 * 8192 * 4
        assert f(1, 64, 64, 1024, -1, ctypes.byref(n)) == EINVAL
        assert f(1, 64, 64, 1024, 0, None) == EINVAL
