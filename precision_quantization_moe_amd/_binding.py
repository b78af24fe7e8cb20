"""ctypes binding of libpqmoe.so.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpqmoe.so")

FMT_BF16, FMT_MXFP8, FMT_NVFP4, FMT_FP8_BLOCK = 0, 1, 2, 3
GEMM_FPROP, GEMM_DGRAD, GEMM_WGRAD = 0, 1, 2
OUT_BF16, OUT_FP32 = 0, 1

_STATUS = {0: "ok", 1: "PQM_ERR_NULL", 2: "PQM_ERR_SHAPE", 3: "PQM_ERR_ALIGN",
           4: "PQM_ERR_ENUM", 5: "PQM_ERR_WORKSPACE", 6: "PQM_ERR_HIP"}


class PqmError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(code, code)}")
        self.code = code


_lib = None

P, I64, SZ, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int

# name -> argtypes; every entry point declared in include/pqmoe.h
SIGNATURES = {
    "pqm_status_string": ([I32], ctypes.c_char_p),
    "pqm_abi_version": ([], I32),
    "pqm_quantize_mxfp8": ([P, I64, I64, I64, P, P, P, P, P], I32),
    "pqm_quantize_fp8_block": ([P, I64, I64, I64, I64, P, P, P], I32),
    "pqm_quantize_nvfp4_per_token": ([P, I64, I64, I64, I64, P, P, P, P, SZ, P], I32),
    "pqm_quantize_nvfp4_workspace": ([I64, I64, I64], SZ),
    "pqm_dequantize": ([I32, P, P, P, I64, I64, I64, P, P], I32),
    "pqm_moe_grouped_gemm": ([I32, I32, P, P, P, P, P, P, I64, P, P, I64, I64, I64, I64,
                              P, I32, P, SZ, P], I32),
    "pqm_moe_grouped_gemm_workspace_size": ([I32, I32], SZ),
    "pqm_moe_fc2_online_nvfp4": ([P, P, P, P, I64, P, I64, I64, I64, I64, P, I32, P, P, P, P],
                                 I32),
    "pqm_moe_fc2_online_nvfp4_split": ([P, P, P, P, I64, P, I64, I64, I64, I64, P, I32, P, P, P,
                                        P, P], I32),
    "pqm_moe_gemm_swiglu_quantize_mxfp8": ([P, P, P, P, P, I64, I64, I64, I64, P, P, P, P, P],
                                           I32),
    "pqm_moe_route": ([P, I64, I64, I64, I32, P, P, P, P, P, SZ, P], I32),
    "pqm_moe_route_workspace": ([I64, I64, I64], SZ),
    "pqm_moe_route_noalloc": ([P, I64, I64, I64, I32, P, P, P, P, P], I32),
    "pqm_moe_gather_rows": ([P, I64, I64, P, I64, I64, P, P], I32),
    "pqm_moe_pad_rows": ([P, I64, I64, P, I64, I64, P, P, I64, P], I32),
    "pqm_swiglu_prob": ([P, P, P, I64, I64, P, P], I32),
    "pqm_swiglu_prob_quantize_mxfp8": ([P, P, P, I64, I64, P, P, P, P], I32),
    "pqm_swiglu_prob_quantize_nvfp4": ([P, P, P, I64, I64, P, P, P, P, P], I32),
    "pqm_moe_combine": ([P, P, P, I64, I64, I64, P, P], I32),
    "pqm_validate_offsets": ([P, I64, I64, I64, P, P], I32),
}


def lib():
    """Load libpqmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m precision_quantization_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(code: int, what: str):
    if code != 0:
        raise PqmError(code, what)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _bf16_2d(x: torch.Tensor) -> torch.Tensor:
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise TypeError("expected a 2-D bfloat16 tensor")
    if not x.is_cuda:
        raise TypeError("expected a device tensor")
    if x.stride(1) != 1:
        raise ValueError("rows must be contiguous")
    return x


# ---------------------------------------------------------------- quantizers

def quantize_mxfp8(x: torch.Tensor, rowwise: bool = True, colwise: bool = True, out=None):
    """MXFP8 row-wise and/or column-wise copies of a bf16 [R, C] tensor.
    Returns (q[R, C], s[R, C/32], qT[C, R], sT[C, R/32]) as uint8 tensors,
    None for a copy that was not requested.  `out` may pass that tuple
    preallocated."""
    x = _bf16_2d(x)
    R, C = x.shape
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    if out is not None:
        q, s, qT, sT = out
    else:
        q = torch.empty((R, C), **u8) if rowwise else None
        s = torch.empty((R, C // 32), **u8) if rowwise else None
        qT = torch.empty((C, R), **u8) if colwise else None
        sT = torch.empty((C, R // 32), **u8) if colwise else None
    _check(lib().pqm_quantize_mxfp8(_ptr(x), R, C, x.stride(0), _ptr(q), _ptr(s),
                                    _ptr(qT), _ptr(sT), _stream(dev)),
           "pqm_quantize_mxfp8")
    return q, s, qT, sT


def quantize_fp8_block(x: torch.Tensor, block_rows: int = 1, out=None):
    """DeepSeek-style block FP8 of a bf16 [R, C] tensor: blocks of
    block_rows x 128 (1: activation tiles, 128: weight blocks).  Returns
    (q [R, C] uint8, s [R/block_rows, C/128] float32); `out` may pass them
    preallocated."""
    x = _bf16_2d(x)
    R, C = x.shape
    dev = x.device
    if out is not None:
        q, s = out
    else:
        q = torch.empty((R, C), dtype=torch.uint8, device=dev)
        s = torch.empty((R // block_rows, C // 128), dtype=torch.float32, device=dev)
    _check(lib().pqm_quantize_fp8_block(_ptr(x), R, C, x.stride(0), block_rows, _ptr(q),
                                        _ptr(s), _stream(dev)), "pqm_quantize_fp8_block")
    return q, s


def quantize_nvfp4_per_token(x: torch.Tensor, rows_per_scale: int = 1, out=None):
    """NVFP4 with one FP32 outer scale per rows_per_scale rows (1 = per
    token; an expert's [gate; up] row count = joint gate/up scale).
    Returns (q[R, C/2] uint8, s_block[R, C/16] uint8,
    s_outer[R/rows_per_scale] float32); `out` may pass them preallocated."""
    x = _bf16_2d(x)
    R, C = x.shape
    dev = x.device
    if out is not None:
        q, sb, sg = out
    else:
        q = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
        sb = torch.empty((R, C // 16), dtype=torch.uint8, device=dev)
        n_scales = R // rows_per_scale if rows_per_scale > 0 else 0
        sg = torch.empty((n_scales,), dtype=torch.float32, device=dev)
    L = lib()
    ws_bytes = L.pqm_quantize_nvfp4_workspace(R, C, rows_per_scale)
    ws = torch.empty((max(ws_bytes, 4),), dtype=torch.uint8, device=dev)
    _check(L.pqm_quantize_nvfp4_per_token(_ptr(x), R, C, x.stride(0), rows_per_scale,
                                          _ptr(q), _ptr(sb), _ptr(sg), _ptr(ws), ws_bytes,
                                          _stream(dev)),
           "pqm_quantize_nvfp4_per_token")
    return q, sb, sg


def dequantize(fmt: int, q: torch.Tensor, s_block: torch.Tensor,
               s_outer: torch.Tensor | None = None, rows_per_scale: int = 1, out=None):
    """bf16 [R, C] reconstruction of an MXFP8 or NVFP4 tensor."""
    R = q.shape[0]
    C = q.shape[1] * (2 if fmt == FMT_NVFP4 else 1)
    y = out if out is not None else torch.empty((R, C), dtype=torch.bfloat16, device=q.device)
    _check(lib().pqm_dequantize(fmt, _ptr(q), _ptr(s_block), _ptr(s_outer), R, C,
                                rows_per_scale, _ptr(y), _stream(q.device)),
           "pqm_dequantize")
    return y


# ---------------------------------------------------------------- GEMM

def moe_grouped_gemm(fmt: int, kind: int, a, b, offsets: torch.Tensor, N: int, K: int,
                     a_scale=None, a_outer=None, b_scale=None, b_outer=None,
                     b_rows_per_scale: int = 0, out_dtype: int = OUT_FP32, out=None,
                     workspace: bool = True, bias=None):
    """Grouped GEMM over experts; see pqm_moe_grouped_gemm in pqmoe.h for the
    operand layouts.  offsets: int64 [G+1] on the device.  workspace=False
    passes none (the MXFP8 weight gradient then deals its tiles in a fixed
    order instead of handing them out).  bias: float32 [G, N] on the device
    (forward only), added in the epilogue."""
    G = offsets.numel() - 1
    # the MXFP8 weight gradient takes the transposed column-wise copies
    M = a.shape[1] if (fmt == FMT_MXFP8 and kind == GEMM_WGRAD) else a.shape[0]
    dev = offsets.device
    odt = torch.float32 if out_dtype == OUT_FP32 else torch.bfloat16
    if out is None:
        shape = (G, N, K) if kind == GEMM_WGRAD else (M, N)
        out = torch.empty(shape, dtype=odt, device=dev)
    L = lib()
    ws_bytes = L.pqm_moe_grouped_gemm_workspace_size(fmt, kind) if workspace else 0
    ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev) if ws_bytes else None
    _check(L.pqm_moe_grouped_gemm(fmt, kind, _ptr(a), _ptr(a_scale), _ptr(a_outer),
                                  _ptr(b), _ptr(b_scale), _ptr(b_outer),
                                  b_rows_per_scale, _ptr(bias), _ptr(offsets), G, M, N, K,
                                  _ptr(out), out_dtype, _ptr(ws), ws_bytes, _stream(dev)),
           "pqm_moe_grouped_gemm")
    return out


def moe_fc2_online_nvfp4(p: torch.Tensor, w_q, w_scale, w_outer, offsets: torch.Tensor, N: int,
                         w_rows_per_scale: int = 0, out_dtype: int = OUT_BF16,
                         encodings: bool = False):
    """NVFP4 down projection with online amax compensation; see
    pqm_moe_fc2_online_nvfp4 in pqmoe.h.  p: bf16 [M, K] device.  Returns
    (y, gs) or, with encodings, (y, gs, q, sb): the output, each row's final
    outer scale, and the codes / block scales P was encoded with."""
    G = offsets.numel() - 1
    M, K = p.shape
    dev = p.device
    odt = torch.float32 if out_dtype == OUT_FP32 else torch.bfloat16
    y = torch.empty((M, N), dtype=odt, device=dev)
    gs = torch.empty((M,), dtype=torch.float32, device=dev)
    q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev) if encodings else None
    sb = torch.empty((M, K // 16), dtype=torch.uint8, device=dev) if encodings else None
    _check(lib().pqm_moe_fc2_online_nvfp4(_ptr(p), _ptr(w_q), _ptr(w_scale), _ptr(w_outer),
                                          w_rows_per_scale or N, _ptr(offsets), G, M, N, K,
                                          _ptr(y), out_dtype, _ptr(gs), _ptr(q), _ptr(sb),
                                          _stream(dev)),
           "pqm_moe_fc2_online_nvfp4")
    return (y, gs, q, sb) if encodings else (y, gs)


def moe_fc2_online_nvfp4_split(p: torch.Tensor, w_q, w_scale, w_outer, offsets: torch.Tensor,
                               N: int, w_rows_per_scale: int = 0, out_dtype: int = OUT_BF16,
                               encodings: bool = False):
    """The same FC2 split into two kernels (encode once, then the GEMM with
    the stored ratios); see pqm_moe_fc2_online_nvfp4_split in pqmoe.h.  The
    codes, block scales, gs and ratio buffers it needs are allocated here.
    Returns (y, gs) or, with encodings, (y, gs, q, sb, ratio)."""
    G = offsets.numel() - 1
    M, K = p.shape
    dev = p.device
    odt = torch.float32 if out_dtype == OUT_FP32 else torch.bfloat16
    y = torch.empty((M, N), dtype=odt, device=dev)
    gs = torch.empty((M,), dtype=torch.float32, device=dev)
    q = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sb = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    ratio = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    _check(lib().pqm_moe_fc2_online_nvfp4_split(_ptr(p), _ptr(w_q), _ptr(w_scale), _ptr(w_outer),
                                                w_rows_per_scale or N, _ptr(offsets), G, M, N, K,
                                                _ptr(y), out_dtype, _ptr(gs), _ptr(q), _ptr(sb),
                                                _ptr(ratio), _stream(dev)),
           "pqm_moe_fc2_online_nvfp4_split")
    return (y, gs, q, sb, ratio) if encodings else (y, gs)


# ---------------------------------------------------------------- MoE glue

def moe_route(topk_ids: torch.Tensor, num_experts: int, shared_expert: bool = False):
    """Counting sort of assignments by expert.  topk_ids int32 [T, k].
    Returns (offsets int64 [E+1(+1)], src_row int32 [M], token int32 [M],
    slot int32 [T, k]) with M = T*k (+T with a shared expert group)."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    sh = 1 if shared_expert else 0
    M = T * k + sh * T
    offsets = torch.empty((num_experts + 1 + sh,), dtype=torch.int64, device=dev)
    src = torch.empty((M,), dtype=torch.int32, device=dev)
    tok = torch.empty((M,), dtype=torch.int32, device=dev)
    slot = torch.empty((T, k), dtype=torch.int32, device=dev)
    L = lib()
    ws_bytes = L.pqm_moe_route_workspace(T, k, num_experts)
    ws = torch.empty((max(ws_bytes, 4),), dtype=torch.uint8, device=dev)
    _check(L.pqm_moe_route(_ptr(topk_ids), T, k, num_experts, sh, _ptr(offsets), _ptr(src),
                           _ptr(tok), _ptr(slot), _ptr(ws), ws_bytes, _stream(dev)),
           "pqm_moe_route")
    return offsets, src, tok, slot


def moe_route_noalloc(topk_ids: torch.Tensor, num_experts: int, shared_expert: bool = False,
                      out=None):
    """moe_route through the entry point that allocates nothing on the
    device: its scratch is the library's per-GPU array.  `out` may pass the
    (offsets, src_row, token, slot) tensors preallocated, so that the call
    itself allocates nothing."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    sh = 1 if shared_expert else 0
    M = T * k + sh * T
    if out is None:
        out = (torch.empty((num_experts + 1 + sh,), dtype=torch.int64, device=dev),
               torch.empty((M,), dtype=torch.int32, device=dev),
               torch.empty((M,), dtype=torch.int32, device=dev),
               torch.empty((T, k), dtype=torch.int32, device=dev))
    offsets, src, tok, slot = out
    _check(lib().pqm_moe_route_noalloc(_ptr(topk_ids), T, k, num_experts, sh, _ptr(offsets),
                                       _ptr(src), _ptr(tok), _ptr(slot), _stream(dev)),
           "pqm_moe_route_noalloc")
    return offsets, src, tok, slot


def moe_gather_rows(src: torch.Tensor, index: torch.Tensor, divisor: int = 1):
    """out[i] = src[index[i] // divisor] for a 2-D byte-addressable tensor."""
    n = index.numel()
    out = torch.empty((n,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    row_bytes = src.stride(0) * src.element_size()
    _check(lib().pqm_moe_gather_rows(_ptr(src), src.shape[0], row_bytes, _ptr(index), n,
                                     divisor, _ptr(out), _stream(src.device)),
           "pqm_moe_gather_rows")
    return out


def pad_rows_bound(rows: int, groups: int, align: int = 32) -> int:
    """Rows that any per-expert padding of `rows` rows in `groups` groups
    fits in, rounded up to a whole block."""
    n = rows + groups * (align - 1)
    return -(-n // align) * align


def moe_pad_rows(src: torch.Tensor, offsets: torch.Tensor, align: int = 32, out=None,
                 padded_offsets=None):
    """Each group's rows of a 2-D tensor moved to a start that is a multiple
    of `align`, padding rows zero.  Returns (out [pad_rows_bound(...), ...],
    padded_offsets int64 [G+1] on the device)."""
    G = offsets.numel() - 1
    rows = src.shape[0]
    if out is None:
        out = torch.empty((pad_rows_bound(rows, G, align),) + tuple(src.shape[1:]),
                          dtype=src.dtype, device=src.device)
    if padded_offsets is None:
        padded_offsets = torch.empty(G + 1, dtype=torch.int64, device=src.device)
    row_bytes = src.stride(0) * src.element_size()
    _check(lib().pqm_moe_pad_rows(_ptr(src), rows, row_bytes, _ptr(offsets), G, align,
                                  _ptr(padded_offsets), _ptr(out), out.shape[0],
                                  _stream(src.device)), "pqm_moe_pad_rows")
    return out, padded_offsets


def swiglu_prob(c: torch.Tensor, prob: torch.Tensor, src: torch.Tensor | None = None):
    """D = silu(gate) * up * prob per row, gate/up the two halves of c.
    prob float32 indexed by src[row] (flat assignment index) when given."""
    M, N2 = c.shape
    d = torch.empty((M, N2 // 2), dtype=torch.bfloat16, device=c.device)
    _check(lib().pqm_swiglu_prob(_ptr(c), _ptr(prob), _ptr(src), M, N2 // 2, _ptr(d),
                                 _stream(c.device)), "pqm_swiglu_prob")
    return d


def swiglu_prob_quantize_mxfp8(c: torch.Tensor, prob: torch.Tensor,
                               src: torch.Tensor | None = None, keep_d: bool = False):
    """swiglu_prob fused with the row-wise MXFP8 quantization of its output.
    Returns (q, s, d) with d None unless keep_d."""
    M, N2 = c.shape
    inter = N2 // 2
    q = torch.empty((M, inter), dtype=torch.uint8, device=c.device)
    s = torch.empty((M, inter // 32), dtype=torch.uint8, device=c.device)
    d = torch.empty((M, inter), dtype=torch.bfloat16, device=c.device) if keep_d else None
    _check(lib().pqm_swiglu_prob_quantize_mxfp8(_ptr(c), _ptr(prob), _ptr(src), M, inter,
                                                _ptr(d), _ptr(q), _ptr(s), _stream(c.device)),
           "pqm_swiglu_prob_quantize_mxfp8")
    return q, s, d


def swiglu_prob_quantize_nvfp4(c: torch.Tensor, prob: torch.Tensor,
                               src: torch.Tensor | None = None, keep_d: bool = False):
    """swiglu_prob fused with the per-token NVFP4 quantization of its output.
    Returns (q, s_block, s_outer, d) with d None unless keep_d."""
    M, N2 = c.shape
    inter = N2 // 2
    dev = c.device
    q = torch.empty((M, inter // 2), dtype=torch.uint8, device=dev)
    sb = torch.empty((M, inter // 16), dtype=torch.uint8, device=dev)
    sg = torch.empty((M,), dtype=torch.float32, device=dev)
    d = torch.empty((M, inter), dtype=torch.bfloat16, device=dev) if keep_d else None
    _check(lib().pqm_swiglu_prob_quantize_nvfp4(_ptr(c), _ptr(prob), _ptr(src), M, inter, _ptr(d),
                                                _ptr(q), _ptr(sb), _ptr(sg), _stream(dev)),
           "pqm_swiglu_prob_quantize_nvfp4")
    return q, sb, sg, d


def moe_gemm_swiglu_quantize_mxfp8(qa, sa, w1q, w1s, offsets: torch.Tensor, inter: int,
                                   prob: torch.Tensor, src: torch.Tensor | None = None):
    """MXFP8 gate_up grouped GEMM with SwiGLU x prob and the row-wise MXFP8
    quantization of D fused into its epilogue.  Returns (qd, sd)."""
    G = offsets.numel() - 1
    M, K = qa.shape
    q = torch.empty((M, inter), dtype=torch.uint8, device=qa.device)
    s = torch.empty((M, inter // 32), dtype=torch.uint8, device=qa.device)
    _check(lib().pqm_moe_gemm_swiglu_quantize_mxfp8(
        _ptr(qa), _ptr(sa), _ptr(w1q), _ptr(w1s), _ptr(offsets), G, M, inter, K, _ptr(prob),
        _ptr(src), _ptr(q), _ptr(s), _stream(qa.device)), "pqm_moe_gemm_swiglu_quantize_mxfp8")
    return q, s


def moe_combine(y_rows: torch.Tensor, slot: torch.Tensor, shared: torch.Tensor | None = None):
    """out[t] = sum_j y_rows[slot[t, j]] (+ shared[t]), bf16 output."""
    T, k = slot.shape
    N = y_rows.shape[1]
    out = torch.empty((T, N), dtype=torch.bfloat16, device=y_rows.device)
    _check(lib().pqm_moe_combine(_ptr(y_rows), _ptr(slot), _ptr(shared), T, k, N, _ptr(out),
                                 _stream(y_rows.device)), "pqm_moe_combine")
    return out


OFFSETS_FIRST_NOT_ZERO, OFFSETS_DECREASING, OFFSETS_MISALIGNED, OFFSETS_PAST_END = 1, 2, 3, 4


def validate_offsets(offsets: torch.Tensor, M_total: int, align: int = 1):
    """Opt-in check of an offsets array (int64 [G+1] on the device) against
    the grouped-GEMM contract.  Returns an int32 device tensor [2]: (first
    failing check or 0, its index or -1); see pqm_validate_offsets."""
    G = offsets.numel() - 1
    res = torch.empty((2,), dtype=torch.int32, device=offsets.device)
    _check(lib().pqm_validate_offsets(_ptr(offsets), G, M_total, align, _ptr(res),
                                      _stream(offsets.device)),
           "pqm_validate_offsets")
    return res
