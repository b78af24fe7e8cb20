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
                      inter: int):
    """Routed experts plus one shared expert (group num_experts, every token)
    with per-token NVFP4 activations.  prob_all [T*k + T] float32: router
    probabilities, then 1.0 for each token's shared-expert row."""
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
    d = b.swiglu_prob(c, prob_all, src)
    qd, sbd, sgd = b.quantize_nvfp4_per_token(d)
    y = b.moe_grouped_gemm(b.FMT_NVFP4, b.GEMM_FPROP, qd, w2q, off, H, inter,
                           a_scale=sbd, a_outer=sgd, b_scale=w2b, b_outer=w2g,
                           b_rows_per_scale=H, out_dtype=b.OUT_BF16)
    out = b.moe_combine(y[:T * k], slot, shared=y[T * k:])
    return dict(off=off, src=src, tok=tok, slot=slot, qa=qa, sba=sba, sga=sga, c=c, d=d,
                qd=qd, sbd=sbd, sgd=sgd, y=y, out=out)
