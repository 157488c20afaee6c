"""Block-scaled FP4 GEMM for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libfp4gemm.so`` (declared in
``include/fp4gemm.h``).  Each function below has the name of the C entry point
it calls, checks and marshals its torch arguments (device memory and the
current stream only), and raises on a non-zero status.  All arithmetic runs in
the library's HIP kernels; there is no fallback.  If the library has not been
built, the first call raises ``ImportError`` naming the build step.

Layouts (uint8 tensors unless noted, all contiguous, all on one GPU):
  mx_fp4_gemm / fp4_gemv : A [M, K/2], sfA [M, K/32], B [N, K/2], sfB [N, K/32]
  nv_fp4_gemm            : A [M, K/2], sfA [M, K/16], B [N, K/2], sfB [N, K/16],
                           plus float global scales
  w4a8_gemm              : A [M, K] (E4M3 codes), sa [M] float32,
                           B [N, K/2] (INT4 nibbles), sB [N, K/128] bfloat16
Output D [M, N] float32 or bfloat16, row-major.  Packed nibbles: low nibble =
even k.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["mx_fp4_gemm", "mx_fp4_gemm_batched", "mx_fp4_gemm_batched_noalloc", "mx_fp4_gemm_workspace_size",
           "nv_fp4_gemm",
           "fp4_gemv_prepack_size", "fp4_gemv_prepack", "fp4_gemv_prepacked",
           "w4a8_prepack_size", "w4a8_prepack", "w4a8_prepack_e4m3", "w4a8_gemm_prepacked",
           "nv_fp4_gemm_batched", "w4a8_gemm_batched", "w4a8_gemm", "fp4_gemv", "mx_fp4_quantize", "nv_fp4_quantize",
           "nv_fp4_gemm_split", "w4a8_gemm_split", "w4a8_gemm_prepacked_split",
           "nv_fp4_gemm_workspace_size", "w4a8_gemm_workspace_size",
           "w4a8_prepack_fp6_size", "w4a8_prepack_fp6", "w4a8_gemm_prepacked_fp6",
           "w4a8_fp6_workspace_size", "w4a8_gemm_prepacked_fp6_split",
           "fp8_blockwise_gemm", "fp4g_status_string",
           "Fp4GemmError", "library_path", "load_library", "SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfp4gemm.so")
SYMBOLS = ("mx_fp4_gemm", "mx_fp4_gemm_batched", "mx_fp4_gemm_batched_noalloc", "mx_fp4_gemm_workspace_size",
           "nv_fp4_gemm",
           "nv_fp4_gemm_batched", "w4a8_gemm", "w4a8_gemm_batched", "fp4_gemv",
           "fp4_gemv_prepack_size", "fp4_gemv_prepack", "fp4_gemv_prepacked",
           "w4a8_prepack_size", "w4a8_prepack", "w4a8_prepack_e4m3", "w4a8_gemm_prepacked",
           "mx_fp4_quantize", "nv_fp4_quantize", "fp8_blockwise_gemm", "fp4g_status_string",
           "nv_fp4_gemm_workspace_size", "w4a8_gemm_workspace_size", "nv_fp4_gemm_split", "w4a8_gemm_split",
           "w4a8_gemm_prepacked_split", "w4a8_prepack_fp6_size", "w4a8_prepack_fp6", "w4a8_gemm_prepacked_fp6",
           "w4a8_fp6_workspace_size", "w4a8_gemm_prepacked_fp6_split")

OUT_F32, OUT_BF16 = 0, 1
IN_F32, IN_BF16 = 0, 1
_lib = None


class Fp4GemmError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: status {status}: {text}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfp4gemm.so (built by ``__graft_entry__.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`"
                          " or `python block_scaled_precision_e2m1_amd/_build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p, c_int, f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.mx_fp4_gemm.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.mx_fp4_gemm.restype = c_int
    lib.mx_fp4_gemm_batched.argtypes = [i64, i64, i64, i64, p, p, p, p, p, c_int, i64, p, ctypes.c_size_t, p]
    lib.mx_fp4_gemm_batched.restype = c_int
    lib.mx_fp4_gemm_batched_noalloc.argtypes = [i64, i64, i64, i64, p, p, p, p, p, c_int, i64, p]
    lib.mx_fp4_gemm_batched_noalloc.restype = c_int
    lib.mx_fp4_gemm_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.mx_fp4_gemm_workspace_size.restype = c_int
    lib.fp4_gemv_prepack_size.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.fp4_gemv_prepack_size.restype = c_int
    lib.fp4_gemv_prepack.argtypes = [i64, i64, p, p, p, p, p]
    lib.fp4_gemv_prepack.restype = c_int
    lib.fp4_gemv_prepacked.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.fp4_gemv_prepacked.restype = c_int
    lib.w4a8_prepack_size.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    lib.w4a8_prepack_size.restype = c_int
    lib.w4a8_prepack.argtypes = [i64, i64, p, p, p, p, p]
    lib.w4a8_prepack.restype = c_int
    lib.w4a8_prepack_e4m3.argtypes = [i64, i64, p, p, i64, p, p, p]
    lib.w4a8_prepack_e4m3.restype = c_int
    lib.w4a8_gemm_prepacked.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.w4a8_gemm_prepacked.restype = c_int
    lib.w4a8_prepack_fp6_size.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t)]
    lib.w4a8_prepack_fp6_size.restype = c_int
    lib.w4a8_prepack_fp6.argtypes = [i64, i64, p, p, p, p, p]
    lib.w4a8_prepack_fp6.restype = c_int
    lib.w4a8_gemm_prepacked_fp6.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.w4a8_gemm_prepacked_fp6.restype = c_int
    lib.w4a8_fp6_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.w4a8_fp6_workspace_size.restype = c_int
    lib.w4a8_gemm_prepacked_fp6_split.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, i64, p, ctypes.c_size_t, p]
    lib.w4a8_gemm_prepacked_fp6_split.restype = c_int
    lib.nv_fp4_gemm_batched.argtypes = [i64, i64, i64, i64, p, p, f, p, p, f, p, c_int, p]
    lib.nv_fp4_gemm_batched.restype = c_int
    lib.w4a8_gemm_batched.argtypes = [i64, i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.nv_fp4_gemm_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.w4a8_gemm_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.nv_fp4_gemm_split.argtypes = [i64, i64, i64, i64, p, p, f, p, p, f, p, c_int, i64, p, ctypes.c_size_t, p]
    lib.w4a8_gemm_split.argtypes = [i64, i64, i64, i64, p, p, p, p, p, c_int, i64, p, ctypes.c_size_t, p]
    lib.w4a8_gemm_prepacked_split.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, i64, p, ctypes.c_size_t, p]
    for name in ("nv_fp4_gemm_workspace_size", "w4a8_gemm_workspace_size", "nv_fp4_gemm_split", "w4a8_gemm_split",
                 "w4a8_gemm_prepacked_split"):
        getattr(lib, name).restype = c_int
    lib.w4a8_gemm_batched.restype = c_int
    lib.fp4_gemv.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.fp4_gemv.restype = c_int
    lib.nv_fp4_gemm.argtypes = [i64, i64, i64, p, p, f, p, p, f, p, c_int, p]
    lib.nv_fp4_gemm.restype = c_int
    lib.w4a8_gemm.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.w4a8_gemm.restype = c_int
    lib.fp8_blockwise_gemm.argtypes = [i64, i64, i64, p, p, p, p, p, c_int, p]
    lib.fp8_blockwise_gemm.restype = c_int
    lib.mx_fp4_quantize.argtypes = [i64, i64, p, c_int, p, p, p]
    lib.mx_fp4_quantize.restype = c_int
    lib.nv_fp4_quantize.argtypes = [i64, i64, p, c_int, f, p, p, p]
    lib.nv_fp4_quantize.restype = c_int
    lib.fp4g_status_string.argtypes = [c_int]
    lib.fp4g_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fp4g_status_string(status: int) -> str:
    return load_library().fp4g_status_string(int(status)).decode()


# ---- argument marshalling ------------------------------------------------------------------

def _check(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0)


def _out(out, M, N, out_dtype, device):
    if out is None:
        return torch.empty((M, N), dtype=out_dtype, device=device)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check(out, "out", out.dtype, (M, N), device)
    return out


def _device_of(A):
    if not isinstance(A, torch.Tensor):
        raise TypeError("A must be a torch.Tensor")
    if A.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {A.device}")
    return A.device


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _raise_on(fn, st):
    if st != 0:
        raise Fp4GemmError(fn, st, fp4g_status_string(st))


def _fp4_common(fn, V, A, sfA, B, sfB, out, out_dtype, max_m=None):
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape[0], A.shape[1] * 2
    N = B.shape[0]
    if K % V:
        raise ValueError(f"K={K} must be a multiple of {V}")
    _check(A, "A", torch.uint8, (M, K // 2), device)
    _check(sfA, "sfA", torch.uint8, (M, K // V), device)
    _check(B, "B", torch.uint8, (N, K // 2), device)
    _check(sfB, "sfB", torch.uint8, (N, K // V), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    return lib, device, M, N, K, D, dt


def mx_fp4_gemm(A, sfA, B, sfB, out=None, out_dtype=torch.bfloat16):
    """MXFP4 GEMM (E2M1 codes, E8M0 scale per 32 K elements); returns D [M, N]."""
    lib, dev, M, N, K, D, dt = _fp4_common("mx_fp4_gemm", 32, A, sfA, B, sfB, out, out_dtype)
    st = lib.mx_fp4_gemm(M, N, K, _ptr(A), _ptr(sfA), _ptr(B), _ptr(sfB), _ptr(D), dt, _stream(dev))
    _raise_on("mx_fp4_gemm", st)
    return D


def mx_fp4_gemm_workspace_size(L, M, N, K, splits=0) -> int:
    """Bytes of workspace mx_fp4_gemm_batched uses for these sizes on the current device."""
    n = ctypes.c_size_t(0)
    st = load_library().mx_fp4_gemm_workspace_size(L, M, N, K, splits, ctypes.byref(n))
    _raise_on("mx_fp4_gemm_workspace_size", st)
    return int(n.value)


def mx_fp4_gemm_batched(A, sfA, B, sfB, out=None, out_dtype=torch.bfloat16, splits=0, workspace=None):
    """Batched MXFP4 GEMM: A [L, M, K/2], sfA [L, M, K/32], B [L, N, K/2], sfB [L, N, K/32]
    -> D [L, M, N].  `splits` = 0 lets the library split K when the tiles are too few
    to fill the GPU, 1 never splits, s > 1 asks for s slices.  `workspace` is a uint8
    device tensor for the partial sums; None allocates the size the library asks for."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D [L, rows, K/2]")
    L, M, K = A.shape[0], A.shape[1], A.shape[2] * 2
    N = B.shape[1]
    if K % 32:
        raise ValueError(f"K={K} must be a multiple of 32")
    _check(A, "A", torch.uint8, (L, M, K // 2), device)
    _check(sfA, "sfA", torch.uint8, (L, M, K // 32), device)
    _check(B, "B", torch.uint8, (L, N, K // 2), device)
    _check(sfB, "sfB", torch.uint8, (L, N, K // 32), device)
    if out is None:
        D = torch.empty((L, M, N), dtype=out_dtype, device=device)
    else:
        if out.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out must be float32 or bfloat16")
        _check(out, "out", out.dtype, (L, M, N), device)
        D = out
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    if workspace is None:
        nbytes = mx_fp4_gemm_workspace_size(L, M, N, K, splits) if K % 128 == 0 else 0
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check(workspace, "workspace", torch.uint8, (workspace.numel(),), device)
    st = lib.mx_fp4_gemm_batched(L, M, N, K, _ptr(A), _ptr(sfA), _ptr(B), _ptr(sfB), _ptr(D), dt, splits,
                                 _ptr(workspace), workspace.numel(), _stream(device))
    _raise_on("mx_fp4_gemm_batched", st)
    return D


def mx_fp4_gemm_batched_noalloc(A, sfA, B, sfB, out, splits=0):
    """mx_fp4_gemm_batched without a workspace: a split of K uses the library's own 32 MiB
    scratch on this GPU, so the call allocates nothing (``out`` [L, M, N] float32 or
    bfloat16 must be given).  Calls that overlap in time on one GPU race on that scratch.
    A requested split that needs more than the scratch holds raises Fp4GemmError."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D [L, rows, K/2]")
    L, M, K = A.shape[0], A.shape[1], A.shape[2] * 2
    N = B.shape[1]
    if K % 32:
        raise ValueError(f"K={K} must be a multiple of 32")
    _check(A, "A", torch.uint8, (L, M, K // 2), device)
    _check(sfA, "sfA", torch.uint8, (L, M, K // 32), device)
    _check(B, "B", torch.uint8, (L, N, K // 2), device)
    _check(sfB, "sfB", torch.uint8, (L, N, K // 32), device)
    if out is None or out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be a float32 or bfloat16 tensor [L, M, N]")
    _check(out, "out", out.dtype, (L, M, N), device)
    dt = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    st = lib.mx_fp4_gemm_batched_noalloc(L, M, N, K, _ptr(A), _ptr(sfA), _ptr(B), _ptr(sfB), _ptr(out), dt,
                                         splits, _stream(device))
    _raise_on("mx_fp4_gemm_batched_noalloc", st)
    return out


def fp4_gemv(A, sfA, B, sfB, out=None, out_dtype=torch.bfloat16):
    """MXFP4 GEMV for 1 <= M <= 16 tokens, or 17 <= M <= 32 with K <= 16384 (same layouts
    as mx_fp4_gemm)."""
    lib, dev, M, N, K, D, dt = _fp4_common("fp4_gemv", 32, A, sfA, B, sfB, out, out_dtype)
    st = lib.fp4_gemv(M, N, K, _ptr(A), _ptr(sfA), _ptr(B), _ptr(sfB), _ptr(D), dt, _stream(dev))
    _raise_on("fp4_gemv", st)
    return D


def fp4_gemv_prepack_size(N, K):
    """(weight bytes, scale bytes) of the pre-packed layout of an N x K MXFP4 weight."""
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = load_library().fp4_gemv_prepack_size(N, K, ctypes.byref(wb), ctypes.byref(sb))
    _raise_on("fp4_gemv_prepack_size", st)
    return int(wb.value), int(sb.value)


def fp4_gemv_prepack(B, sfB):
    """Re-pack MXFP4 weights B [N, K/2] / sfB [N, K/32] into the GEMV's MFMA-register
    order; returns (Bp, Sp) as flat uint8 device tensors."""
    lib = load_library()
    device = _device_of(B)
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    N, K = B.shape[0], B.shape[1] * 2
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(B, "B", torch.uint8, (N, K // 2), device)
    _check(sfB, "sfB", torch.uint8, (N, K // 32), device)
    wb, sb = fp4_gemv_prepack_size(N, K)
    Bp = torch.empty(wb, dtype=torch.uint8, device=device)
    Sp = torch.empty(sb, dtype=torch.uint8, device=device)
    st = lib.fp4_gemv_prepack(N, K, _ptr(B), _ptr(sfB), _ptr(Bp), _ptr(Sp), _stream(device))
    _raise_on("fp4_gemv_prepack", st)
    return Bp, Sp


def fp4_gemv_prepacked(A, sfA, Bp, Sp, N, out=None, out_dtype=torch.bfloat16):
    """fp4_gemv with weights from fp4_gemv_prepack (N weight rows); returns D [M, N]."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2:
        raise ValueError("A must be 2-D")
    M, K = A.shape[0], A.shape[1] * 2
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (M, K // 2), device)
    _check(sfA, "sfA", torch.uint8, (M, K // 32), device)
    wb, sb = fp4_gemv_prepack_size(N, K)
    _check(Bp, "Bp", torch.uint8, (wb,), device)
    _check(Sp, "Sp", torch.uint8, (sb,), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    st = lib.fp4_gemv_prepacked(M, N, K, _ptr(A), _ptr(sfA), _ptr(Bp), _ptr(Sp), _ptr(D), dt, _stream(device))
    _raise_on("fp4_gemv_prepacked", st)
    return D


def nv_fp4_gemm(A, sfA, global_a, B, sfB, global_b, out=None, out_dtype=torch.bfloat16):
    """NVFP4 GEMM (E2M1 codes, E4M3 scale per 16 K elements, fp32 global scales)."""
    lib, dev, M, N, K, D, dt = _fp4_common("nv_fp4_gemm", 16, A, sfA, B, sfB, out, out_dtype)
    st = lib.nv_fp4_gemm(M, N, K, _ptr(A), _ptr(sfA), float(global_a), _ptr(B), _ptr(sfB),
                         float(global_b), _ptr(D), dt, _stream(dev))
    _raise_on("nv_fp4_gemm", st)
    return D


def w4a8_gemm(A, sa, B, sB, out=None, out_dtype=torch.bfloat16):
    """W4A8 GEMM: A [M, K] E4M3 codes (uint8), sa [M] float32, B [N, K/2] INT4 nibbles,
    sB [N, K/128] bfloat16 group scales."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N = B.shape[0]
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (M, K), device)
    _check(sa, "sa", torch.float32, (M,), device)
    _check(B, "B", torch.uint8, (N, K // 2), device)
    _check(sB, "sB", torch.bfloat16, (N, K // 128), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    st = lib.w4a8_gemm(M, N, K, _ptr(A), _ptr(sa), _ptr(B), _ptr(sB), _ptr(D), dt, _stream(device))
    _raise_on("w4a8_gemm", st)
    return D


def w4a8_prepack_size(N, K):
    """(weight bytes, scale bytes) of the pre-packed layout of an N x K W4A8 weight."""
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = load_library().w4a8_prepack_size(N, K, ctypes.byref(wb), ctypes.byref(sb))
    _raise_on("w4a8_prepack_size", st)
    return int(wb.value), int(sb.value)


def w4a8_prepack(B, sB):
    """Re-pack W4A8 weights B [N, K/2] (INT4) and sB [N, K/128] (bfloat16) for
    w4a8_gemm_prepacked; returns (Bp uint8, Sp float32) as flat device tensors."""
    lib = load_library()
    device = _device_of(B)
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    N, K = B.shape[0], B.shape[1] * 2
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(B, "B", torch.uint8, (N, K // 2), device)
    _check(sB, "sB", torch.bfloat16, (N, K // 128), device)
    wb, sb = w4a8_prepack_size(N, K)
    Bp = torch.empty(wb, dtype=torch.uint8, device=device)
    Sp = torch.empty(sb // 4, dtype=torch.float32, device=device)
    st = lib.w4a8_prepack(N, K, _ptr(B), _ptr(sB), _ptr(Bp), _ptr(Sp), _stream(device))
    _raise_on("w4a8_prepack", st)
    return Bp, Sp


def w4a8_prepack_fp6_size(N, K):
    """(weight bytes, scale bytes) of the FP6 re-encoded layout of an N x K W4A8 weight."""
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = load_library().w4a8_prepack_fp6_size(N, K, ctypes.byref(wb), ctypes.byref(sb))
    _raise_on("w4a8_prepack_fp6_size", st)
    return int(wb.value), int(sb.value)


def w4a8_prepack_fp6(B, sB):
    """Re-encode W4A8 weights B [N, K/2] (INT4) as FP6 and widen sB [N, K/128]
    (bfloat16) for w4a8_gemm_prepacked_fp6; returns (Bp6 uint8, Sp float32) as flat
    device tensors."""
    lib = load_library()
    device = _device_of(B)
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    N, K = B.shape[0], B.shape[1] * 2
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(B, "B", torch.uint8, (N, K // 2), device)
    _check(sB, "sB", torch.bfloat16, (N, K // 128), device)
    wb, sb = w4a8_prepack_fp6_size(N, K)
    Bp6 = torch.empty(wb, dtype=torch.uint8, device=device)
    Sp = torch.empty(sb // 4, dtype=torch.float32, device=device)
    st = lib.w4a8_prepack_fp6(N, K, _ptr(B), _ptr(sB), _ptr(Bp6), _ptr(Sp), _stream(device))
    _raise_on("w4a8_prepack_fp6", st)
    return Bp6, Sp


def w4a8_gemm_prepacked_fp6(A, sa, Bp6, Sp, N, out=None, out_dtype=torch.bfloat16):
    """w4a8_gemm with weights from w4a8_prepack_fp6 (N weight rows); returns D [M, N]."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2:
        raise ValueError("A must be 2-D")
    M, K = A.shape
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (M, K), device)
    _check(sa, "sa", torch.float32, (M,), device)
    wb, sb = w4a8_prepack_fp6_size(N, K)
    _check(Bp6, "Bp6", torch.uint8, (wb,), device)
    _check(Sp, "Sp", torch.float32, (sb // 4,), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    st = lib.w4a8_gemm_prepacked_fp6(M, N, K, _ptr(A), _ptr(sa), _ptr(Bp6), _ptr(Sp), _ptr(D), dt,
                                     _stream(device))
    _raise_on("w4a8_gemm_prepacked_fp6", st)
    return D


def w4a8_fp6_workspace_size(M, N, K, splits=0):
    """Workspace bytes w4a8_gemm_prepacked_fp6_split takes for these sizes and `splits`."""
    nb = ctypes.c_size_t(0)
    st = load_library().w4a8_fp6_workspace_size(M, N, K, splits, ctypes.byref(nb))
    _raise_on("w4a8_fp6_workspace_size", st)
    return int(nb.value)


def w4a8_gemm_prepacked_fp6_split(A, sa, Bp6, Sp, N, out=None, out_dtype=torch.bfloat16, splits=0, workspace=None):
    """w4a8_gemm_prepacked_fp6 with a split of K; `splits` and `workspace` as for
    nv_fp4_gemm_split."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2:
        raise ValueError("A must be 2-D")
    M, K = A.shape
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (M, K), device)
    _check(sa, "sa", torch.float32, (M,), device)
    wb, sb = w4a8_prepack_fp6_size(N, K)
    _check(Bp6, "Bp6", torch.uint8, (wb,), device)
    _check(Sp, "Sp", torch.float32, (sb // 4,), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    ws = _workspace(workspace, w4a8_fp6_workspace_size(M, N, K, splits) if workspace is None else 0, device)
    st = lib.w4a8_gemm_prepacked_fp6_split(M, N, K, _ptr(A), _ptr(sa), _ptr(Bp6), _ptr(Sp), _ptr(D), dt, splits,
                                           _ptr(ws), ws.numel(), _stream(device))
    _raise_on("w4a8_gemm_prepacked_fp6_split", st)
    return D


def w4a8_prepack_e4m3(B, sB8, scale_stride=1):
    """Re-pack W4A8 weights B [N, K/2] (INT4) with E4M3 group scales for
    w4a8_gemm_prepacked: sB8 uint8 [N, K/128] (scale_stride 1) or [N, K/128, 8] (the
    Array<E4M3, 8> packing, scale_stride 8); returns (Bp uint8, Sp float32)."""
    lib = load_library()
    device = _device_of(B)
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    N, K = B.shape[0], B.shape[1] * 2
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    if scale_stride not in (1, 8):
        raise ValueError("scale_stride must be 1 or 8")
    _check(B, "B", torch.uint8, (N, K // 2), device)
    _check(sB8, "sB8", torch.uint8, (N, K // 128) if scale_stride == 1 else (N, K // 128, 8), device)
    wb, sb = w4a8_prepack_size(N, K)
    Bp = torch.empty(wb, dtype=torch.uint8, device=device)
    Sp = torch.empty(sb // 4, dtype=torch.float32, device=device)
    st = lib.w4a8_prepack_e4m3(N, K, _ptr(B), _ptr(sB8), int(scale_stride), _ptr(Bp), _ptr(Sp), _stream(device))
    _raise_on("w4a8_prepack_e4m3", st)
    return Bp, Sp


def w4a8_gemm_prepacked(A, sa, Bp, Sp, N, out=None, out_dtype=torch.bfloat16):
    """w4a8_gemm with weights from w4a8_prepack (N weight rows); returns D [M, N]."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2:
        raise ValueError("A must be 2-D")
    M, K = A.shape
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (M, K), device)
    _check(sa, "sa", torch.float32, (M,), device)
    wb, sb = w4a8_prepack_size(N, K)
    _check(Bp, "Bp", torch.uint8, (wb,), device)
    _check(Sp, "Sp", torch.float32, (sb // 4,), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    st = lib.w4a8_gemm_prepacked(M, N, K, _ptr(A), _ptr(sa), _ptr(Bp), _ptr(Sp), _ptr(D), dt, _stream(device))
    _raise_on("w4a8_gemm_prepacked", st)
    return D


def _batched_out(out, L, M, N, out_dtype, device):
    if out is None:
        return torch.empty((L, M, N), dtype=out_dtype, device=device)
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check(out, "out", out.dtype, (L, M, N), device)
    return out


def nv_fp4_gemm_batched(A, sfA, global_a, B, sfB, global_b, out=None, out_dtype=torch.bfloat16):
    """Batched NVFP4 GEMM: A [L, M, K/2], sfA [L, M, K/16], B [L, N, K/2], sfB [L, N, K/16]
    -> D [L, M, N]; the global scales apply to every problem."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D [L, rows, K/2]")
    L, M, K = A.shape[0], A.shape[1], A.shape[2] * 2
    N = B.shape[1]
    if K % 16:
        raise ValueError(f"K={K} must be a multiple of 16")
    _check(A, "A", torch.uint8, (L, M, K // 2), device)
    _check(sfA, "sfA", torch.uint8, (L, M, K // 16), device)
    _check(B, "B", torch.uint8, (L, N, K // 2), device)
    _check(sfB, "sfB", torch.uint8, (L, N, K // 16), device)
    D = _batched_out(out, L, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    st = lib.nv_fp4_gemm_batched(L, M, N, K, _ptr(A), _ptr(sfA), float(global_a), _ptr(B), _ptr(sfB),
                                 float(global_b), _ptr(D), dt, _stream(device))
    _raise_on("nv_fp4_gemm_batched", st)
    return D


def w4a8_gemm_batched(A, sa, B, sB, out=None, out_dtype=torch.bfloat16):
    """Batched W4A8 GEMM: A [L, M, K] uint8 E4M3, sa [L, M] float32, B [L, N, K/2] uint8 INT4,
    sB [L, N, K/128] bfloat16 -> D [L, M, N]."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D")
    L, M, K = A.shape
    N = B.shape[1]
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (L, M, K), device)
    _check(sa, "sa", torch.float32, (L, M), device)
    _check(B, "B", torch.uint8, (L, N, K // 2), device)
    _check(sB, "sB", torch.bfloat16, (L, N, K // 128), device)
    D = _batched_out(out, L, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    st = lib.w4a8_gemm_batched(L, M, N, K, _ptr(A), _ptr(sa), _ptr(B), _ptr(sB), _ptr(D), dt, _stream(device))
    _raise_on("w4a8_gemm_batched", st)
    return D


def nv_fp4_gemm_workspace_size(L, M, N, K, splits=0) -> int:
    """Bytes of workspace nv_fp4_gemm_split uses for these sizes on the current device."""
    n = ctypes.c_size_t(0)
    _raise_on("nv_fp4_gemm_workspace_size", load_library().nv_fp4_gemm_workspace_size(L, M, N, K, splits, ctypes.byref(n)))
    return int(n.value)


def w4a8_gemm_workspace_size(L, M, N, K, splits=0) -> int:
    """Bytes of workspace w4a8_gemm_split (or, with L = 1, w4a8_gemm_prepacked_split) uses."""
    n = ctypes.c_size_t(0)
    _raise_on("w4a8_gemm_workspace_size", load_library().w4a8_gemm_workspace_size(L, M, N, K, splits, ctypes.byref(n)))
    return int(n.value)


def _workspace(workspace, nbytes, device):
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check(workspace, "workspace", torch.uint8, (workspace.numel(),), device)
    return workspace


def nv_fp4_gemm_split(A, sfA, global_a, B, sfB, global_b, out=None, out_dtype=torch.bfloat16, splits=0,
                      workspace=None):
    """nv_fp4_gemm_batched with a K split: `splits` = 0 lets the library choose, 1 never
    splits, s > 1 asks for at most s slices.  `workspace` is a uint8 device tensor for the
    partial products; None allocates the size the library asks for."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D [L, rows, K/2]")
    L, M, K = A.shape[0], A.shape[1], A.shape[2] * 2
    N = B.shape[1]
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (L, M, K // 2), device)
    _check(sfA, "sfA", torch.uint8, (L, M, K // 16), device)
    _check(B, "B", torch.uint8, (L, N, K // 2), device)
    _check(sfB, "sfB", torch.uint8, (L, N, K // 16), device)
    D = _batched_out(out, L, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    ws = _workspace(workspace, nv_fp4_gemm_workspace_size(L, M, N, K, splits) if workspace is None else 0, device)
    st = lib.nv_fp4_gemm_split(L, M, N, K, _ptr(A), _ptr(sfA), float(global_a), _ptr(B), _ptr(sfB), float(global_b),
                               _ptr(D), dt, splits, _ptr(ws), ws.numel(), _stream(device))
    _raise_on("nv_fp4_gemm_split", st)
    return D


def w4a8_gemm_split(A, sa, B, sB, out=None, out_dtype=torch.bfloat16, splits=0, workspace=None):
    """w4a8_gemm_batched with a K split (plain weights split only when K % 256 == 0);
    `splits` and `workspace` as for nv_fp4_gemm_split."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D")
    L, M, K = A.shape
    N = B.shape[1]
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (L, M, K), device)
    _check(sa, "sa", torch.float32, (L, M), device)
    _check(B, "B", torch.uint8, (L, N, K // 2), device)
    _check(sB, "sB", torch.bfloat16, (L, N, K // 128), device)
    D = _batched_out(out, L, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    ws = _workspace(workspace, w4a8_gemm_workspace_size(L, M, N, K, splits) if workspace is None else 0, device)
    st = lib.w4a8_gemm_split(L, M, N, K, _ptr(A), _ptr(sa), _ptr(B), _ptr(sB), _ptr(D), dt, splits, _ptr(ws),
                             ws.numel(), _stream(device))
    _raise_on("w4a8_gemm_split", st)
    return D


def w4a8_gemm_prepacked_split(A, sa, Bp, Sp, N, out=None, out_dtype=torch.bfloat16, splits=0, workspace=None):
    """w4a8_gemm_prepacked with a K split; `splits` and `workspace` as for
    nv_fp4_gemm_split."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2:
        raise ValueError("A must be 2-D")
    M, K = A.shape
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (M, K), device)
    _check(sa, "sa", torch.float32, (M,), device)
    wb, sb = w4a8_prepack_size(N, K)
    _check(Bp, "Bp", torch.uint8, (wb,), device)
    _check(Sp, "Sp", torch.float32, (sb // 4,), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    ws = _workspace(workspace, w4a8_gemm_workspace_size(1, M, N, K, splits) if workspace is None else 0, device)
    st = lib.w4a8_gemm_prepacked_split(M, N, K, _ptr(A), _ptr(sa), _ptr(Bp), _ptr(Sp), _ptr(D), dt, splits,
                                       _ptr(ws), ws.numel(), _stream(device))
    _raise_on("w4a8_gemm_prepacked_split", st)
    return D


def mx_fp4_quantize(X, codes=None, scales=None):
    """MX quantizer: X [rows, K] float32 or bfloat16 (K % 32 == 0) -> (codes [rows, K/2]
    uint8 packed E2M1, scales [rows, K/32] uint8 E8M0), the operand layout of
    mx_fp4_gemm / fp4_gemv, by the max-abs rule of include/fp4gemm.h."""
    lib = load_library()
    device = _device_of(X)
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    if X.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"X must be float32 or bfloat16, got {X.dtype}")
    rows, K = X.shape
    if K % 32:
        raise ValueError(f"K={K} must be a multiple of 32")
    _check(X, "X", X.dtype, (rows, K), device)
    if codes is None:
        codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=device)
    _check(codes, "codes", torch.uint8, (rows, K // 2), device)
    _check(scales, "scales", torch.uint8, (rows, K // 32), device)
    xt = IN_BF16 if X.dtype == torch.bfloat16 else IN_F32
    st = lib.mx_fp4_quantize(rows, K, _ptr(X), xt, _ptr(codes), _ptr(scales), _stream(device))
    _raise_on("mx_fp4_quantize", st)
    return codes, scales


def nv_fp4_quantize(X, global_scale, codes=None, scales=None):
    """NV quantizer: X [rows, K] float32 or bfloat16 (K % 16 == 0) and an fp32 global scale
    g > 0 -> (codes [rows, K/2] uint8 packed E2M1, scales [rows, K/16] uint8 E4M3), the
    operand layout of nv_fp4_gemm with global scale g, by the max-abs rule of
    include/fp4gemm.h."""
    lib = load_library()
    device = _device_of(X)
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    if X.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"X must be float32 or bfloat16, got {X.dtype}")
    rows, K = X.shape
    if K % 16:
        raise ValueError(f"K={K} must be a multiple of 16")
    _check(X, "X", X.dtype, (rows, K), device)
    if codes is None:
        codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=device)
    _check(codes, "codes", torch.uint8, (rows, K // 2), device)
    _check(scales, "scales", torch.uint8, (rows, K // 16), device)
    xt = IN_BF16 if X.dtype == torch.bfloat16 else IN_F32
    st = lib.nv_fp4_quantize(rows, K, _ptr(X), xt, float(global_scale), _ptr(codes), _ptr(scales), _stream(device))
    _raise_on("nv_fp4_quantize", st)
    return codes, scales


def fp8_blockwise_gemm(A, sA, B, sB, out=None, out_dtype=torch.bfloat16):
    """FP8 blockwise-scaled GEMM: A [M, K] and B [N, K] E4M3 codes (uint8), sA [M, K/128]
    and sB [N, K/128] float32 scales; returns D [M, N]."""
    lib = load_library()
    device = _device_of(A)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N = B.shape[0]
    if K % 128:
        raise ValueError(f"K={K} must be a multiple of 128")
    _check(A, "A", torch.uint8, (M, K), device)
    _check(sA, "sA", torch.float32, (M, K // 128), device)
    _check(B, "B", torch.uint8, (N, K), device)
    _check(sB, "sB", torch.float32, (N, K // 128), device)
    D = _out(out, M, N, out_dtype, device)
    dt = OUT_BF16 if D.dtype == torch.bfloat16 else OUT_F32
    st = lib.fp8_blockwise_gemm(M, N, K, _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(D), dt, _stream(device))
    _raise_on("fp8_blockwise_gemm", st)
    return D
