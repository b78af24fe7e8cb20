"""MoE expert-layer forward passes composed from the library's entry points.

Each function only sequences calls into libpqmoe (routing, quantization,
gather, grouped GEMM, weighted SwiGLU, combine) on torch's current stream;
all arithmetic happens in the HIP kernels.  The structure follows the
pages: the routed experts run through one grouped GEMM per projection over a
contiguous, offset-delimited buffer ("miniTE technical report", 5.2); the
weighted SwiGLU feeds the FC2 quantizer (5.3/5.4); routed outputs are
reduced in high precision ("Towards Blackwell-Native 8-bit and 4-bit RL",
fine-grained precision control).  Weights are quantized once per update and
passed in quantized form.
"""
from __future__ import annotations

import torch

from . import _binding as b


def quantize_expert_weights_mxfp8(w1: torch.Tensor, w2: torch.Tensor):
    """w1 [E*2I, H] (gate rows then up rows per expert), w2 [E*H, I] bf16 ->
    row-wise MXFP8 (q, s) of each (blocks along the GEMM reduction axis)."""
    w1q, w1s, _, _ = b.quantize_mxfp8(w1, colwise=False)
    w2q, w2s, _, _ = b.quantize_mxfp8(w2, colwise=False)
    return w1q, w1s, w2q, w2s


def column_copies_mxfp8(w1: torch.Tensor, w2: torch.Tensor):
    """Column-wise MXFP8 copies (32 x 1 blocks, stored transposed) of the
    stacked expert weights, the data-gradient operands of the low-precision
    backward: w1 [E*2I, H] -> ([H, E*2I], [H, E*2I/32]); w2 [E*H, I] ->
    ([I, E*H], [I, E*H/32])."""
    _, _, w1T, w1sT = b.quantize_mxfp8(w1, rowwise=False)
    _, _, w2T, w2sT = b.quantize_mxfp8(w2, rowwise=False)
    return w1T, w1sT, w2T, w2sT


def saved_activation_mxfp8(rows: torch.Tensor, off: torch.Tensor):
    """The forward-side column-wise MXFP8 copy of an expert-sorted
    activation (FC1 input X or FC2 input D) for the weight gradient: each
    expert's rows padded to whole 32-row blocks, then quantized down the
    columns.  Returns (qT [C, Mp], sT [C, Mp/32], padded offsets)."""
    xp, poff = b.moe_pad_rows(rows, off)
    _, _, qT, sT = b.quantize_mxfp8(xp, rowwise=False)
    return qT, sT, poff


def mxfp8_expert_backward(dy, dc, saved_x, saved_d, w_col, off, inter: int):
    """MXFP8 low-precision backward of the two expert GEMMs ([BW] MXFP8
    training: the data- and weight-gradient GEMMs run in MXFP8 on the
    column-wise copies).
      dy [M, H] bf16   gradient of the down-projection output rows
      dc [M, 2I] bf16  gradient of the gate_up output rows
      saved_x, saved_d (qT, sT, padded offsets) from saved_activation_mxfp8
      w_col            column_copies_mxfp8(W1, W2)
    Both gradients are padded per expert (pqm_moe_pad_rows) and quantized
    once into their row-wise (data gradient) and column-wise (weight
    gradient) copies.  Returns dict(dd [Mp, I] bf16, dx [Mp, H] bf16,
    dw2 [E, H, I] fp32, dw1 [E, 2I, H] fp32, poff): dd and dx are in the
    padded row order (row poff[e] + j of expert e is routed row off[e] + j)."""
    H = dy.shape[1]
    w1T, w1sT, w2T, w2sT = w_col
    xT, xsT, _ = saved_x
    dT, dsT, _ = saved_d
    dyp, poff = b.moe_pad_rows(dy, off)
    dcp, _ = b.moe_pad_rows(dc, off)
    qy, sy, qyT, syT = b.quantize_mxfp8(dyp)
    qc, sc, qcT, scT = b.quantize_mxfp8(dcp)
    dd = b.moe_grouped_gemm(b.FMT_MXFP8, b.GEMM_DGRAD, qy, w2T, poff, inter, H,
                            a_scale=sy, b_scale=w2sT, out_dtype=b.OUT_BF16)
    dw2 = b.moe_grouped_gemm(b.FMT_MXFP8, b.GEMM_WGRAD, qyT, dT, poff, H, inter,
                             a_scale=syT, b_scale=dsT, out_dtype=b.OUT_FP32)
    dx = b.moe_grouped_gemm(b.FMT_MXFP8, b.GEMM_DGRAD, qc, w1T, poff, H, 2 * inter,
                            a_scale=sc, b_scale=w1sT, out_dtype=b.OUT_BF16)
    dw1 = b.moe_grouped_gemm(b.FMT_MXFP8, b.GEMM_WGRAD, qcT, xT, poff, 2 * inter, H,
                             a_scale=scT, b_scale=xsT, out_dtype=b.OUT_FP32)
    return dict(dd=dd, dx=dx, dw2=dw2, dw1=dw1, poff=poff)


def quantize_expert_weights_nvfp4(w1: torch.Tensor, w2: torch.Tensor, inter: int, hidden: int):
    """NVFP4 weights with one FP32 outer scale per expert tensor; gate and up
    of an expert share one scale (joint)."""
    w1q, w1b, w1g = b.quantize_nvfp4_per_token(w1, rows_per_scale=2 * inter)
    w2q, w2b, w2g = b.quantize_nvfp4_per_token(w2, rows_per_scale=hidden)
    return w1q, w1b, w1g, w2q, w2b, w2g


def mxfp8_moe_forward(x, topk_ids, prob_flat, w1q, w1s, w2q, w2s, num_experts: int,
                      inter: int, keep_intermediates: bool = True):
    """x [T, H] bf16; topk_ids [T, k] int32; prob_flat [T*k] float32.
    Returns a dict of every stage's output (out = [T, H] bf16).  With
    keep_intermediates the gate_up output c and d = SwiGLU(c) x prob are
    materialised (bf16; d and its MXFP8 encoding in one fused pass);
    without, the gate_up GEMM's epilogue produces the MXFP8 encoding of d
    directly and c, d are None (same bytes)."""
    T, H = x.shape
    off, src, tok, slot = b.moe_route(topk_ids, num_experts)
    qx, sx, _, _ = b.quantize_mxfp8(x, colwise=False)
    qa = b.moe_gather_rows(qx, tok)
    sa = b.moe_gather_rows(sx, tok)
    if keep_intermediates or inter % 128 or H % 128 or H > 2048:
        c = b.moe_grouped_gemm(b.FMT_MXFP8, b.GEMM_FPROP, qa, w1q, off, 2 * inter, H,
                               a_scale=sa, b_scale=w1s, out_dtype=b.OUT_BF16)
        qd, sd, d = b.swiglu_prob_quantize_mxfp8(c, prob_flat, src, keep_d=keep_intermediates)
    else:
        c = d = None
        qd, sd = b.moe_gemm_swiglu_quantize_mxfp8(qa, sa, w1q, w1s, off, inter, prob_flat, src)
    y = b.moe_grouped_gemm(b.FMT_MXFP8, b.GEMM_FPROP, qd, w2q, off, H, inter,
                           a_scale=sd, b_scale=w2s, out_dtype=b.OUT_BF16)
    out = b.moe_combine(y, slot)
    return dict(off=off, src=src, tok=tok, slot=slot, qa=qa, sa=sa, c=c, d=d, qd=qd, sd=sd,
                y=y, out=out)


def nvfp4_moe_forward(x, topk_ids, prob_all, w1q, w1b, w1g, w2q, w2b, w2g, num_experts: int,
                      inter: int, keep_intermediates: bool = True):
    """Routed experts plus one shared expert (group num_experts, every token)
    with per-token NVFP4 activations.  prob_all [T*k + T] float32: router
    probabilities, then 1.0 for each token's shared-expert row.  The weighted
    SwiGLU and the per-token NVFP4 quantization of its output D run as one
    fused pass; D is materialised (bf16) only with keep_intermediates (same
    bytes either way)."""
    T, H = x.shape
    k = topk_ids.shape[1]
    off, src, tok, slot = b.moe_route(topk_ids, num_experts, shared_expert=True)
    qx, sbx, sgx = b.quantize_nvfp4_per_token(x)
    qa = b.moe_gather_rows(qx, tok)
    sba = b.moe_gather_rows(sbx, tok)
    sga = b.moe_gather_rows(sgx.view(T, 1), tok).view(-1)
    c = b.moe_grouped_gemm(b.FMT_NVFP4, b.GEMM_FPROP, qa, w1q, off, 2 * inter, H,
                           a_scale=sba, a_outer=sga, b_scale=w1b, b_outer=w1g,
                           b_rows_per_scale=2 * inter, out_dtype=b.OUT_BF16)
    qd, sbd, sgd, d = b.swiglu_prob_quantize_nvfp4(c, prob_all, src, keep_d=keep_intermediates)
    y = b.moe_grouped_gemm(b.FMT_NVFP4, b.GEMM_FPROP, qd, w2q, off, H, inter,
                           a_scale=sbd, a_outer=sgd, b_scale=w2b, b_outer=w2g,
                           b_rows_per_scale=H, out_dtype=b.OUT_BF16)
    out = b.moe_combine(y[:T * k], slot, shared=y[T * k:])
    return dict(off=off, src=src, tok=tok, slot=slot, qa=qa, sba=sba, sga=sga, c=c, d=d,
                qd=qd, sbd=sbd, sgd=sgd, y=y, out=out)
