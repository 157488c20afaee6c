"""Seeded synthetic inputs for the block-scaled FP4 GEMM workloads.

This module is shared by the tests, the benchmark and the smoke check, and by
nothing else.  It draws codes and scales and packs them into the byte layouts
the library and the oracle consume; it holds none of the contraction's
arithmetic (no decode tables, no dot products).  The encoders below
(round-to-nearest-even onto the E2M1 grid, max-abs E8M0 block scales, E4M3
via torch's float8 cast, bf16 rounding) only turn normal samples into codes,
the way a producer of such tensors would.

Layouts (both sides read the same bytes):
  FP4 / INT4 operands  X[rows][K/2] uint8, low nibble = even k.
  MX scales            sf[rows][K/32] uint8 (E8M0 exponent codes).
  NV scales            sf[rows][K/16] uint8 (E4M3 codes), plus fp32 gA, gB.
  W4A8                 A[M][K] uint8 (E4M3 codes), sa[M] fp32,
                       B[N][K/2] uint8 (two's-complement nibbles),
                       sB[N][K/128] uint16 (bf16 bit patterns).

Random streams: numpy.random.default_rng(seed), drawn in the order A, sfA,
B, sfB, then any extra scales.
"""
from __future__ import annotations

import numpy as np

W4A8_GROUP = 128

# E8M0 exponent codes and E4M3 codes used by the uniform configurations.
MX_EXP_LO, MX_EXP_HI = 124, 130          # inclusive
NV_SCALE_CODE_LO, NV_SCALE_CODE_HI = 0x28, 0x48   # E4M3 0.25 .. 4.0, inclusive (33 codes)


# ---- packing ----------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows][K] codes in 0..15 -> [rows][K/2] bytes, low nibble = even k."""
    codes = np.asarray(codes)
    if codes.shape[-1] % 2:
        raise ValueError("K must be even")
    c = codes.astype(np.uint8) & np.uint8(0xF)
    return np.ascontiguousarray(c[..., 0::2] | (c[..., 1::2] << np.uint8(4)))


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: [rows][K/2] bytes -> [rows][K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out


# ---- encoders (input production only) ----------------------------------------------------

def _e2m1_rne_code(y: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even onto the E2M1 grid {0,.5,1,1.5,2,3,4,6}, saturating at 6.

    The magnitude code is the number of decision thresholds passed; a tie goes to
    the neighbour whose code is even (">=" where the upper neighbour is even).
    """
    mag = np.abs(y)
    code = ((mag > 0.25).astype(np.uint8) + (mag >= 0.75) + (mag > 1.25) + (mag >= 1.75)
            + (mag > 2.5) + (mag >= 3.5) + (mag > 5.0)).astype(np.uint8)
    return code | (np.signbit(y) & (code > 0)).astype(np.uint8) << np.uint8(3)


def quantize_mx(x: np.ndarray):
    """fp32 [rows][K] -> (packed E2M1 [rows][K/2], E8M0 codes [rows][K/32]).

    Per 32-element block: e = clamp(floor(log2 amax) - 2 + 127, 0, 254) (127 when
    the block is all zero), element = RNE_E2M1(x * 2^(127 - e)).
    """
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(xb), axis=2)
    _, ex = np.frexp(amax)                # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, ex.astype(np.int32) - 1 - 2 + 127, 127)
    e = np.clip(e, 0, 254).astype(np.int32)
    y = np.ldexp(xb, (127 - e)[:, :, None]).reshape(rows, K)
    codes = _e2m1_rne_code(y)
    return pack_nibbles(codes), e.astype(np.uint8)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def e4m3_codes(y: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3FN codes (round to nearest even, saturating at +-448)."""
    import torch
    t = torch.from_numpy(np.clip(np.asarray(y, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_e4m3_rows(x: np.ndarray):
    """fp32 [M][K] -> (E4M3 codes [M][K], fp32 row scales sa = amax_row / 448)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    sa = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return e4m3_codes(x / sa[:, None]), sa


# ---- generic random inputs ----------------------------------------------------------------

def random_mx(M, N, K, rng, exp_lo=MX_EXP_LO, exp_hi=MX_EXP_HI):
    """MXFP4 operands with codes uniform over all 16 and E8M0 codes uniform in [lo, hi]."""
    A = pack_nibbles(rng.integers(0, 16, (M, K), dtype=np.uint8))
    sfA = rng.integers(exp_lo, exp_hi + 1, (M, K // 32), dtype=np.uint8)
    B = pack_nibbles(rng.integers(0, 16, (N, K), dtype=np.uint8))
    sfB = rng.integers(exp_lo, exp_hi + 1, (N, K // 32), dtype=np.uint8)
    return {"A": A, "sfA": sfA, "B": B, "sfB": sfB}


def random_mx_gaussian(M, N, K, rng):
    """MXFP4 operands quantized from N(0,1) samples with max-abs E8M0 block scales."""
    A, sfA = quantize_mx(rng.standard_normal((M, K), dtype=np.float32))
    B, sfB = quantize_mx(rng.standard_normal((N, K), dtype=np.float32))
    return {"A": A, "sfA": sfA, "B": B, "sfB": sfB}


def random_nv(M, N, K, rng, gA=1.0, gB=1.0):
    """NVFP4 operands: codes uniform, E4M3 scale codes uniform over 0x28..0x48."""
    A = pack_nibbles(rng.integers(0, 16, (M, K), dtype=np.uint8))
    sfA = rng.integers(NV_SCALE_CODE_LO, NV_SCALE_CODE_HI + 1, (M, K // 16), dtype=np.uint8)
    B = pack_nibbles(rng.integers(0, 16, (N, K), dtype=np.uint8))
    sfB = rng.integers(NV_SCALE_CODE_LO, NV_SCALE_CODE_HI + 1, (N, K // 16), dtype=np.uint8)
    return {"A": A, "sfA": sfA, "B": B, "sfB": sfB,
            "gA": np.float32(gA), "gB": np.float32(gB)}


def random_w4a8(M, N, K, rng):
    """W4A8 operands: A from N(0,1) with per-row E4M3 scaling, B uniform INT4 in
    [-8, 7], sB uniform in [0.005, 0.05) rounded to bf16."""
    if K % W4A8_GROUP:
        raise ValueError("K must be a multiple of 128")
    A, sa = quantize_e4m3_rows(rng.standard_normal((M, K), dtype=np.float32))
    q = rng.integers(-8, 8, (N, K), dtype=np.int8)
    B = pack_nibbles(q.view(np.uint8) & np.uint8(0xF))
    sB = bf16_bits(rng.uniform(0.005, 0.05, (N, K // W4A8_GROUP)).astype(np.float32))
    return {"A": A, "sa": sa, "B": B, "sB": sB}


FP8_BLOCK = 128


def quantize_e4m3_blocks(x: np.ndarray):
    """fp32 [rows][K] -> (E4M3 codes [rows][K], fp32 scales [rows][K/128]): per row and
    128-element block, s = amax / 448 (1 for an all-zero block), code = E4M3(x / s)."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    xb = x.reshape(rows, K // FP8_BLOCK, FP8_BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return e4m3_codes((xb / s[:, :, None]).reshape(rows, K)), s


def random_fp8b(M, N, K, rng):
    """FP8 blockwise operands: A and B from N(0,1), each quantized to E4M3 with one fp32
    scale per row per 128-element K block."""
    if K % FP8_BLOCK:
        raise ValueError("K must be a multiple of 128")
    A, sA = quantize_e4m3_blocks(rng.standard_normal((M, K), dtype=np.float32))
    B, sB = quantize_e4m3_blocks(rng.standard_normal((N, K), dtype=np.float32))
    return {"A": A, "sA": sA, "B": B, "sB": sB}


# ---- the named workloads ------------------------------------------------------------------

# name -> (kind, M, N, K, output dtype, generator)
CONFIGS = {
    "mxfp4_256": ("mx", 256, 256, 256, "f32", "uniform"),
    "nvfp4_1024": ("nv", 1024, 1024, 1024, "bf16", "uniform"),
    "mxfp4_gemv_8x14336x4096": ("gemv", 8, 14336, 4096, "bf16", "gaussian"),
    "w4a8_256x8192x8192": ("w4a8", 256, 8192, 8192, "bf16", "gaussian"),
    "mxfp4_8192": ("mx", 8192, 8192, 8192, "bf16", "gaussian"),
    "fp8_block_4096": ("fp8b", 4096, 4096, 4096, "bf16", "gaussian"),
}


def make(name: str, seed: int = 0):
    """Inputs of a named workload (numpy arrays) plus its metadata."""
    kind, M, N, K, out, dist = CONFIGS[name]
    rng = np.random.default_rng(seed)
    if kind in ("mx", "gemv"):
        d = random_mx(M, N, K, rng) if dist == "uniform" else random_mx_gaussian(M, N, K, rng)
    elif kind == "nv":
        d = random_nv(M, N, K, rng)
    elif kind == "w4a8":
        d = random_w4a8(M, N, K, rng)
    elif kind == "fp8b":
        d = random_fp8b(M, N, K, rng)
    else:
        raise ValueError(kind)
    d.update({"kind": kind, "M": M, "N": N, "K": K, "out": out, "name": name})
    return d


def make_shape(kind: str, M: int, N: int, K: int, seed: int = 0, dist: str = "uniform"):
    """Inputs of an arbitrary shape for the parity tests."""
    rng = np.random.default_rng(seed)
    if kind in ("mx", "gemv"):
        d = random_mx(M, N, K, rng) if dist == "uniform" else random_mx_gaussian(M, N, K, rng)
    elif kind == "nv":
        d = random_nv(M, N, K, rng)
    elif kind == "w4a8":
        d = random_w4a8(M, N, K, rng)
    elif kind == "fp8b":
        d = random_fp8b(M, N, K, rng)
    else:
        raise ValueError(kind)
    d.update({"kind": kind, "M": M, "N": N, "K": K})
    return d
