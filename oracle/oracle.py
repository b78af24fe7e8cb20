"""CPU oracle for the block-scaled quantizers, dequantizer, grouped GEMM and
MoE glue.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package's smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It
shares no code with the HIP library and does not import it.

The encodings (MXFP8, NVFP4, bf16 rounding) live in ``pqo.c`` and are taken
by exact comparisons.  The grouped GEMM is its plain definition: binary64
products of the exactly decoded operands, summed by a library matmul per
group.  The glue (routing, SwiGLU, combine) is written in binary64 numpy.

Page titles cited:
  [BW] "Towards Blackwell-Native 8-bit and 4-bit RL"
  [MT] "miniTE technical report: stable training and efficient
       implementation of native NVFP4 RL"
  [PR] "PR #2396 report: docs: refresh MXFP8 and NVFP4 RL guide"
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pqo.c")
_LIB_PATH = os.path.join(_HERE, "libpqo.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
          "-fopenmp", "-shared", "-fPIC", "-Wall"]


def build(force: bool = False) -> str:
    """Compile pqo.c into libpqo.so next to it (gcc, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        Lg = ctypes.c_long
        L.pqo_quantize_mxfp8_rowwise.argtypes = [P, Lg, Lg, Lg, P, P]
        L.pqo_quantize_mxfp8_colwise.argtypes = [P, Lg, Lg, Lg, P, P]
        L.pqo_quantize_nvfp4.argtypes = [P, Lg, Lg, Lg, Lg, P, P, P]
        L.pqo_dequantize_mxfp8.argtypes = [P, P, Lg, Lg, P]
        L.pqo_dequantize_nvfp4.argtypes = [P, P, P, Lg, Lg, Lg, P]
        L.pqo_decode_mxfp8.argtypes = [P, P, Lg, Lg, P]
        L.pqo_decode_nvfp4.argtypes = [P, P, P, Lg, Lg, Lg, P]
        L.pqo_quantize_fp8_block.argtypes = [P, Lg, Lg, Lg, Lg, P, P]
        L.pqo_decode_fp8_block.argtypes = [P, P, Lg, Lg, Lg, P]
        L.pqo_e4m3_encode.argtypes = [ctypes.c_double, ctypes.c_double]
        L.pqo_e4m3_encode.restype = ctypes.c_uint8
        L.pqo_e2m1_encode.argtypes = [ctypes.c_double, ctypes.c_double]
        L.pqo_e2m1_encode.restype = ctypes.c_uint8
        L.pqo_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.pqo_e4m3_decode.restype = ctypes.c_double
        L.pqo_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.pqo_e2m1_decode.restype = ctypes.c_double
        L.pqo_mx_scale_exponent.argtypes = [ctypes.c_double]
        L.pqo_mx_scale_exponent.restype = ctypes.c_int
        L.pqo_bf16_round.argtypes = [ctypes.c_double]
        L.pqo_bf16_round.restype = ctypes.c_uint16
        L.pqo_bf16_round_array.argtypes = [P, Lg, P]
        L.pqo_inexact_count.restype = ctypes.c_long
        L.pqo_omp_threads.restype = ctypes.c_int
        L.pqo_fp32_div.argtypes = [ctypes.c_float, ctypes.c_float]
        L.pqo_fp32_div.restype = ctypes.c_float
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16 and x.ndim == 2, "bf16 bit patterns [R, C]"
    return x


# --------------------------------------------------------------------------
# Quantizers ([BW] Format background; Recipe 1; Recipe 2)
# --------------------------------------------------------------------------

def quantize_mxfp8_rowwise(x: np.ndarray):
    """1x32 E4M3 blocks along rows with a rounded-up E8M0 scale.
    Returns (q[R, C] u8, s[R, C/32] u8)."""
    x = _bf16(x)
    R, C = x.shape
    assert C % 32 == 0
    q = np.empty((R, C), np.uint8)
    s = np.empty((R, C // 32), np.uint8)
    lib().pqo_quantize_mxfp8_rowwise(_ptr(x), R, C, C, _ptr(q), _ptr(s))
    return q, s


def quantize_mxfp8_colwise(x: np.ndarray):
    """32x1 blocks down columns of the bf16 input, stored transposed.
    Returns (qT[C, R] u8, sT[C, R/32] u8)."""
    x = _bf16(x)
    R, C = x.shape
    assert R % 32 == 0
    q = np.empty((C, R), np.uint8)
    s = np.empty((C, R // 32), np.uint8)
    lib().pqo_quantize_mxfp8_colwise(_ptr(x), R, C, C, _ptr(q), _ptr(s))
    return q, s


def quantize_mxfp8(x: np.ndarray):
    """Both independent copies: (q, s, qT, sT)."""
    q, s = quantize_mxfp8_rowwise(x)
    qT, sT = quantize_mxfp8_colwise(x)
    return q, s, qT, sT


def quantize_nvfp4(x: np.ndarray, rows_per_group: int = 1):
    """NVFP4 with one FP32 outer scale per group of rows_per_group rows
    (1 = per token).  Returns (q[R, C/2] u8, sb[R, C/16] u8,
    sg[R/rows_per_group] f32)."""
    x = _bf16(x)
    R, C = x.shape
    assert C % 16 == 0 and rows_per_group >= 1 and R % rows_per_group == 0
    q = np.empty((R, C // 2), np.uint8)
    sb = np.empty((R, C // 16), np.uint8)
    sg = np.empty((R // rows_per_group,), np.float32)
    lib().pqo_quantize_nvfp4(_ptr(x), R, C, C, rows_per_group,
                             _ptr(q), _ptr(sb), _ptr(sg))
    return q, sb, sg


def quantize_fp8_block(x: np.ndarray, block_rows: int):
    """DeepSeek-V3-style block FP8: blocks of block_rows x 128 (1 for
    activation tiles, 128 for weight blocks), s = A/448 in binary32, q =
    nearest E4M3 of x/s.  Returns (q[R, C] u8, s[R/block_rows, C/128] f32)."""
    x = _bf16(x)
    R, C = x.shape
    assert C % 128 == 0 and block_rows >= 1 and R % block_rows == 0
    q = np.empty((R, C), np.uint8)
    s = np.empty((R // block_rows, C // 128), np.float32)
    lib().pqo_quantize_fp8_block(_ptr(x), R, C, C, block_rows, _ptr(q), _ptr(s))
    return q, s


def decode_fp8_block(q: np.ndarray, s: np.ndarray, block_rows: int) -> np.ndarray:
    """Exact binary64 values q * s."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.float32)
    R, C = q.shape
    assert s.shape == (R // block_rows, C // 128)
    out = np.empty((R, C), np.float64)
    lib().pqo_decode_fp8_block(_ptr(q), _ptr(s), R, C, block_rows, _ptr(out))
    return out


def dequantize_mxfp8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    R, C = q.shape
    assert s.shape == (R, C // 32)
    y = np.empty((R, C), np.uint16)
    lib().pqo_dequantize_mxfp8(_ptr(q), _ptr(s), R, C, _ptr(y))
    return y


def dequantize_nvfp4(q: np.ndarray, sb: np.ndarray, sg: np.ndarray,
                     rows_per_group: int = 1) -> np.ndarray:
    q = np.ascontiguousarray(q, np.uint8)
    sb = np.ascontiguousarray(sb, np.uint8)
    sg = np.ascontiguousarray(sg, np.float32)
    R, C2 = q.shape
    C = 2 * C2
    assert sb.shape == (R, C // 16) and sg.shape == (R // rows_per_group,)
    y = np.empty((R, C), np.uint16)
    lib().pqo_dequantize_nvfp4(_ptr(q), _ptr(sb), _ptr(sg), R, C,
                               rows_per_group, _ptr(y))
    return y


def decode_mxfp8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exact binary64 values q * 2^(s-127)."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    R, C = q.shape
    out = np.empty((R, C), np.float64)
    lib().pqo_decode_mxfp8(_ptr(q), _ptr(s), R, C, _ptr(out))
    return out


def decode_nvfp4(q, sb, sg, rows_per_group: int = 1) -> np.ndarray:
    """Exact binary64 values q * s_b * s_g ([MT] 2.2 decode formula)."""
    q = np.ascontiguousarray(q, np.uint8)
    sb = np.ascontiguousarray(sb, np.uint8)
    sg = np.ascontiguousarray(sg, np.float32)
    R, C2 = q.shape
    out = np.empty((R, 2 * C2), np.float64)
    lib().pqo_decode_nvfp4(_ptr(q), _ptr(sb), _ptr(sg), R, 2 * C2,
                           rows_per_group, _ptr(out))
    return out


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact binary64 values."""
    x = np.ascontiguousarray(x, np.uint16)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """Single round-to-nearest-even of binary64 values to bf16 bit patterns."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().pqo_bf16_round_array(_ptr(v), v.size, _ptr(out))
    return out


def inexact_count() -> int:
    """Number of midpoint products that were not exact (must be 0)."""
    return int(lib().pqo_inexact_count())


# --------------------------------------------------------------------------
# Grouped GEMM ([MT] 5.2 contiguous buffer + offsets; 5.4 epilogue;
# 6.2.1: GEMMs are compared against a golden built from dequantized operands)
# --------------------------------------------------------------------------

def grouped_gemm(a: np.ndarray, b: np.ndarray, offsets: np.ndarray,
                 rows: np.ndarray | None = None) -> np.ndarray:
    """Forward / dgrad: Y[m, :] = sum_k A[m, k] * B_g[:, k] for the group g
    holding row m (offsets[g] <= m < offsets[g+1]).

    a: [M, K] binary64 operand values; b: [G, N, K] binary64; offsets: [G+1].
    rows: optional subset of row indices to compute (sampling); the result
    then has len(rows) rows.  Accumulation is binary64.
    """
    offsets = np.asarray(offsets, np.int64)
    G = b.shape[0]
    assert offsets.shape == (G + 1,) and offsets[0] == 0
    M = a.shape[0]
    assert offsets[-1] == M
    if rows is None:
        y = np.zeros((M, b.shape[1]), np.float64)
        for g in range(G):
            lo, hi = int(offsets[g]), int(offsets[g + 1])
            if hi > lo:
                y[lo:hi] = a[lo:hi] @ b[g].T
        return y
    rows = np.asarray(rows, np.int64)
    grp = np.searchsorted(offsets, rows, side="right") - 1
    y = np.zeros((rows.size, b.shape[1]), np.float64)
    for i, (m, g) in enumerate(zip(rows, grp)):
        y[i] = b[g] @ a[m]
    return y


def grouped_gemm_wgrad(dy: np.ndarray, x: np.ndarray,
                       offsets: np.ndarray) -> np.ndarray:
    """Weight gradient per group: dW_g = dY_g^T X_g, contracting over the
    group's rows.  dy: [M, N], x: [M, K] -> [G, N, K] binary64."""
    offsets = np.asarray(offsets, np.int64)
    G = offsets.size - 1
    out = np.zeros((G, dy.shape[1], x.shape[1]), np.float64)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            out[g] = dy[lo:hi].T @ x[lo:hi]
    return out


# --------------------------------------------------------------------------
# MoE glue ([MT] 5.2 contiguous layout; 5.3/5.4 weighted SwiGLU; [BW] routed
# outputs are reduced in high precision)
# --------------------------------------------------------------------------

def route(topk_ids: np.ndarray, num_experts: int, shared_expert: bool = False):
    """Counting sort of token->expert assignments into a contiguous buffer.

    topk_ids: [T, k] expert ids.  Assignment (t, j) has flat index t*k + j.
    Returns (offsets[G+1] int64, src_row[M] int64 = flat index of the
    assignment stored at each position, slot[T, k] int64 = position of each
    assignment).  Within an expert, assignments keep their flat order.  With
    shared_expert, one more group of T rows follows (row T*k + t holds token
    t, flat index T*k + t) and G = num_experts + 1.
    """
    ids = np.asarray(topk_ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    counts = np.zeros(num_experts, np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    src_row = np.empty(T * k, np.int64)
    slot = np.empty(T * k, np.int64)
    for i, e in enumerate(flat):
        src_row[fill[e]] = i
        slot[i] = fill[e]
        fill[e] += 1
    if shared_expert:
        offsets = np.concatenate([offsets, [T * k + T]])
        src_row = np.concatenate([src_row, T * k + np.arange(T)])
    return offsets, src_row, slot.reshape(T, k)


def route_token(src_row: np.ndarray, T: int, k: int) -> np.ndarray:
    """Token of each stored row: t for assignment t*k + j, and t for the
    shared expert's row T*k + t."""
    src_row = np.asarray(src_row, np.int64)
    return np.where(src_row < T * k, src_row // k, src_row - T * k)


def pad_rows(x: np.ndarray, offsets: np.ndarray, align: int):
    """Per-expert padding ([MT] 5.3 pads the permuted activation before it
    is quantized; [BW] MXFP8 training: a column-wise 32 x 1 block must hold
    one expert's tokens only).  Group g's rows are moved to start at the sum
    of the earlier groups' sizes rounded up to multiples of `align`; the
    rows in between are zero.  Returns (padded x, padded offsets [G+1])."""
    offsets = np.asarray(offsets, np.int64)
    G = offsets.size - 1
    sizes = offsets[1:] - offsets[:-1]
    padded = [int(-(-int(n) // align) * align) for n in sizes]
    poff = np.zeros(G + 1, np.int64)
    for g in range(G):
        poff[g + 1] = poff[g] + padded[g]
    out = np.zeros((int(poff[-1]),) + x.shape[1:], x.dtype)
    for g in range(G):
        n = int(sizes[g])
        out[poff[g]:poff[g] + n] = x[offsets[g]:offsets[g] + n]
    return out, poff


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), in binary64."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_prob(c: np.ndarray, prob: np.ndarray) -> np.ndarray:
    """D = silu(gate) * up * prob with gate = c[:, :N/2], up = c[:, N/2:]
    ([MT] 5.4: D = act(gate, up) x prob, width N/2).  binary64 result."""
    c = np.asarray(c, np.float64)
    n = c.shape[1] // 2
    return silu(c[:, :n]) * c[:, n:] * np.asarray(prob, np.float64)[:, None]


def combine(y_rows: np.ndarray, slot: np.ndarray,
            shared: np.ndarray | None = None) -> np.ndarray:
    """out[t] = sum_j y_rows[slot[t, j]] (+ shared[t]) in binary64."""
    y_rows = np.asarray(y_rows, np.float64)
    out = y_rows[slot].sum(axis=1)
    if shared is not None:
        out = out + np.asarray(shared, np.float64)
    return out
