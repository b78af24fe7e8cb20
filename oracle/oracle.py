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
        L.pqo_quantize_nvfp4_given_scale.argtypes = [P, Lg, Lg, Lg, P, P, P]
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
        L.pqo_set_threads.argtypes = [ctypes.c_int]
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


def quantize_nvfp4_given_scale(x: np.ndarray, sg: np.ndarray):
    """The NVFP4 block encoding of each row of x under a caller-given FP32
    outer scale sg[r] (the running-amax scale of [MT] 5.6).  With sg[r] =
    fp32(max|x[r]| / 2688) this is quantize_nvfp4(x).  Returns
    (q[R, C/2] u8, sb[R, C/16] u8)."""
    x = _bf16(x)
    R, C = x.shape
    sg = np.ascontiguousarray(sg, np.float32)
    assert C % 16 == 0 and sg.shape == (R,)
    q = np.empty((R, C // 2), np.uint8)
    sb = np.empty((R, C // 16), np.uint8)
    lib().pqo_quantize_nvfp4_given_scale(_ptr(x), R, C, C, _ptr(sg), _ptr(q), _ptr(sb))
    return q, sb


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


def set_threads(n: int) -> None:
    """OpenMP threads of the C oracle's loops (timing only)."""
    lib().pqo_set_threads(int(n))


def threads() -> int:
    return int(lib().pqo_omp_threads())


def inexact_count() -> int:
    """Number of midpoint products that were not exact (must be 0)."""
    return int(lib().pqo_inexact_count())


# --------------------------------------------------------------------------
# Grouped GEMM ([MT] 5.2 contiguous buffer + offsets; 5.4 epilogue;
# 6.2.1: GEMMs are compared against a golden built from dequantized operands)
# --------------------------------------------------------------------------

def grouped_gemm(a: np.ndarray, b: np.ndarray, offsets: np.ndarray,
                 rows: np.ndarray | None = None,
                 bias: np.ndarray | None = None) -> np.ndarray:
    """Forward / dgrad: Y[m, :] = sum_k A[m, k] * B_g[:, k] (+ bias[g, :])
    for the group g holding row m (offsets[g] <= m < offsets[g+1]); the
    forward epilogue's additive term follows [MT] 5.4 (accumulator times the
    outer scales, plus bias).

    a: [M, K] binary64 operand values; b: [G, N, K] binary64; offsets: [G+1];
    bias: optional [G, N].  rows: optional subset of row indices to compute
    (sampling); the result then has len(rows) rows.  Accumulation is
    binary64.
    """
    offsets = np.asarray(offsets, np.int64)
    G = b.shape[0]
    assert offsets.shape == (G + 1,) and offsets[0] == 0
    M = a.shape[0]
    assert offsets[-1] == M
    if bias is not None:
        bias = np.asarray(bias, np.float64)
        assert bias.shape == (G, b.shape[1])
    if rows is None:
        y = np.zeros((M, b.shape[1]), np.float64)
        for g in range(G):
            lo, hi = int(offsets[g]), int(offsets[g + 1])
            if hi > lo:
                y[lo:hi] = a[lo:hi] @ b[g].T
                if bias is not None:
                    y[lo:hi] += bias[g]
        return y
    rows = np.asarray(rows, np.int64)
    grp = np.searchsorted(offsets, rows, side="right") - 1
    y = np.zeros((rows.size, b.shape[1]), np.float64)
    for i, (m, g) in enumerate(zip(rows, grp)):
        y[i] = b[g] @ a[m]
        if bias is not None:
            y[i] += bias[g]
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


# --------------------------------------------------------------------------
# Online amax compensation for a single-pass SwiGLU-FFN ([MT] 5.6)
# --------------------------------------------------------------------------
#
# The FC2 GEMM consumes the activation P = SwiGLU(gate, up) x prob tile by
# tile along its contraction dimension, before the row's full maximum (and
# hence its NVFP4 outer scale) is known.  Each row keeps a running maximum;
# tile i is encoded under the outer scale gs_i of the maximum so far, its FC2
# partial product dO_i carries the block scales but not gs_i, and the
# accumulator is moved to the new scale whenever gs grows:
#     O <- O * (gs_prev / gs_i) + dO_i,      Y = O * gs_last * gs_W2,
# so that O * gs_i equals sum_{j <= i} gs_j dO_j at every step.  Rows whose
# maximum is still zero skip the tile; an all-zero row gives Y = 0.
#
# Readings (the pages leave these open):
#  * P enters as bf16, the activation dtype of the two-pass path (the fused
#    SwiGLU + NVFP4 pass quantizes a bf16 D), so both paths encode the same
#    values with the same quantizer.
#  * gs_i = fp32(gamax_i / 2688), the FP32 outer scale of the per-token
#    quantizer, so a row whose maximum lies in its first non-zero tile gets
#    the two-pass encoding exactly.
#  * The loop runs in binary64 (acc=np.float64).  acc=np.float32 models a
#    binary32 accumulator: dO_i, the ratio gs_prev / gs_i, the product and the
#    sum are each rounded to binary32; the report uses it for the compensation
#    error of such an accumulator.
#  * W2 is NVFP4 with one outer scale for the whole [N, I] matrix.


def _nvfp4_block_values(q: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """Exact q * s_b (block scale applied, outer scale not)."""
    return decode_nvfp4(q, sb, np.ones(q.shape[0], np.float32))


def online_amax_fc2(p: np.ndarray, tile: int, w2q: np.ndarray, w2sb: np.ndarray,
                    w2sg: float, acc=np.float64):
    """The [MT] 5.6 loop over the K-tiles of FC2.

    p: bf16 bits [R, I] (the weighted SwiGLU output, consumed tile by tile);
    tile: K-tile width, a multiple of 16 dividing I; w2q [N, I/2], w2sb
    [N, I/16], w2sg: NVFP4 W2 (one outer scale).  Returns (Y [R, N] binary64,
    rec) with rec = dict(gs [R, n_tiles] fp32, 0 where the tile was skipped;
    q [R, I/2] and sb [R, I/16]: each tile's encoding under its running scale).
    """
    p = _bf16(p)
    R, I = p.shape
    N = w2q.shape[0]
    assert tile % 16 == 0 and I % tile == 0
    assert w2q.shape == (N, I // 2) and w2sb.shape == (N, I // 16)
    w2 = _nvfp4_block_values(w2q, w2sb)                  # [N, I], no gs_W2
    n_tiles = I // tile
    gamax = np.zeros(R, np.float32)
    gs_prev = np.zeros(R, np.float32)
    O = np.zeros((R, N), acc)
    gs_rec = np.zeros((R, n_tiles), np.float32)
    q_all = np.zeros((R, I // 2), np.uint8)
    sb_all = np.zeros((R, I // 16), np.uint8)
    for i in range(n_tiles):
        c0, c1 = i * tile, (i + 1) * tile
        p_i = np.ascontiguousarray(p[:, c0:c1])
        rowmax = np.abs(bf16_to_f64(p_i)).max(axis=1).astype(np.float32)
        gamax = np.maximum(gamax, rowmax)
        live = gamax > 0                                   # else: skip the tile
        gs = np.array([lib().pqo_fp32_div(float(a), 2688.0) for a in gamax], np.float32)
        q_i, sb_i = quantize_nvfp4_given_scale(p_i, np.where(live, gs, 0).astype(np.float32))
        q_all[:, c0 // 2:c1 // 2] = q_i
        sb_all[:, c0 // 16:c1 // 16] = sb_i
        dO = _nvfp4_block_values(q_i, sb_i) @ w2[:, c0:c1].T   # binary64
        for r in np.nonzero(live)[0]:
            if acc is np.float32:
                ratio = np.float32(gs_prev[r]) / np.float32(gs[r])
                O[r] = (O[r] * ratio) + dO[r].astype(np.float32)
            else:
                O[r] = O[r] * (float(gs_prev[r]) / float(gs[r])) + dO[r]
            gs_prev[r] = gs[r]
            gs_rec[r, i] = gs[r]
    Y = np.asarray(O, np.float64) * gs_prev.astype(np.float64)[:, None] * float(np.float32(w2sg))
    return Y, dict(gs=gs_rec, q=q_all, sb=sb_all)


def two_pass_fc2(p: np.ndarray, w2q: np.ndarray, w2sb: np.ndarray, w2sg: float):
    """Two-pass counterpart: the whole row of P is produced first, encoded
    per token under its full maximum, then FC2.  Returns (Y [R, N] binary64,
    (q, sb, sg))."""
    q, sb, sg = quantize_nvfp4(p)
    N = w2q.shape[0]
    w2 = decode_nvfp4(w2q, w2sb, np.full(1, w2sg, np.float32), rows_per_group=N)
    return decode_nvfp4(q, sb, sg) @ w2.T, (q, sb, sg)


def online_amax_report(p: np.ndarray, tile: int, w2q, w2sb, w2sg) -> dict:
    """Compensation error and quantization difference of the online loop
    ([MT] 5.6 evaluates both separately):

    * comp_rel_fp32: max over rows of ||Y_fp32acc - Y_exact|| / ||Y_exact||,
      where Y_exact = gs_W2 sum_i gs_i dO_i from the same encodings (the
      rescaling error of a binary32 accumulator);
    * comp_rel_fp64: the same for the binary64 loop;
    * blocks_changed: fraction of 16-blocks whose decoded values differ from
      the two-pass encoding (early encoding under a smaller outer scale);
    * rel_vs_two_pass: max and mean over rows of ||Y_online - Y_two_pass|| /
      ||Y_two_pass|| (zero rows excluded);
    * rel_two_pass_vs_exact / rel_online_vs_exact: the same against the
      unquantized product bf16(P) @ W2 (dequantized W2), for scale.
    """
    N = w2q.shape[0]
    y64, rec = online_amax_fc2(p, tile, w2q, w2sb, w2sg, np.float64)
    y32, _ = online_amax_fc2(p, tile, w2q, w2sb, w2sg, np.float32)
    y2, (q2, sb2, sg2) = two_pass_fc2(p, w2q, w2sb, w2sg)
    w2b = _nvfp4_block_values(w2q, w2sb)
    R, I = p.shape
    exact = np.zeros((R, N))
    vals = _nvfp4_block_values(rec["q"], rec["sb"])
    for i in range(rec["gs"].shape[1]):
        c0, c1 = i * tile, (i + 1) * tile
        exact += rec["gs"][:, i:i + 1].astype(np.float64) * (vals[:, c0:c1] @ w2b[:, c0:c1].T)
    exact *= float(np.float32(w2sg))
    w2 = w2b * float(np.float32(w2sg))
    ref = bf16_to_f64(_bf16(p)) @ w2.T

    def rel(a, b):
        nb = np.linalg.norm(b, axis=1)
        m = nb > 0
        return np.linalg.norm(a - b, axis=1)[m] / nb[m]

    # decoded values per block: online tile i under its own gs_i
    on_v = vals.copy()
    for i in range(rec["gs"].shape[1]):
        c0, c1 = i * tile, (i + 1) * tile
        on_v[:, c0:c1] *= rec["gs"][:, i:i + 1].astype(np.float64)
    two = decode_nvfp4(q2, sb2, sg2)
    changed = (on_v != two).reshape(R, -1, 16).any(axis=2)
    r64, r32, rv = rel(y64, exact), rel(y32, exact), rel(y64, y2)
    return dict(comp_rel_fp64=float(r64.max(initial=0.0)),
                comp_rel_fp32=float(r32.max(initial=0.0)),
                blocks_changed=float(changed.mean()),
                rel_vs_two_pass_max=float(rv.max(initial=0.0)),
                rel_vs_two_pass_mean=float(rv.mean()) if rv.size else 0.0,
                rel_two_pass_vs_exact=float(rel(y2, ref).mean()) if rv.size else 0.0,
                rel_online_vs_exact=float(rel(y64, ref).mean()) if rv.size else 0.0)
