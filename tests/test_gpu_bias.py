"""GPU parity of the grouped GEMM's forward epilogue bias ([MT] 5.4: the
accumulator times the outer scales, plus bias) against the oracle's
binary64 product plus bias[g, n], for every forward kernel path: the MXFP8
persistent, four-wave and register-staged kernels, the NVFP4 wide,
pipelined and register-staged kernels, block FP8, the BF16 pipelined and
register-staged kernels, and an empty contraction (the output is the bias).

Bar: relative L2 <= 1e-3 per row on binary32 output (+ 2^-8 for bf16)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import workloads as wl
from gpu_util import dev, dev_bf16, host, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 1e-3


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def _rel_rows(got, want):
    num = np.linalg.norm(got.astype(np.float64) - want, axis=1)
    den = np.linalg.norm(want, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def _operands(fmt, sizes, N, K, seed):
    """Device arguments of moe_grouped_gemm and the oracle's decoded A, B."""
    G, M = len(sizes), int(sum(sizes))
    x = wl.activations(max(M, 1), K, seed=seed)[:M]
    w = wl.normal_bf16((G * N, K), std=0.02, seed=seed + 1)
    if fmt == pqm.FMT_MXFP8:
        qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(x), colwise=False)
        qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w), colwise=False)
        kw = dict(a_scale=sa, b_scale=sb)
        ra, rsa = oracle.quantize_mxfp8_rowwise(x)
        rb, rsb = oracle.quantize_mxfp8_rowwise(w)
        A, B = oracle.decode_mxfp8(ra, rsa), oracle.decode_mxfp8(rb, rsb)
    elif fmt == pqm.FMT_NVFP4:
        qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(x))
        qb, sb, gb = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
        kw = dict(a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb, b_rows_per_scale=N)
        ra, rsa, rga = oracle.quantize_nvfp4(x)
        rb, rsb, rgb = oracle.quantize_nvfp4(w, rows_per_group=N)
        A, B = oracle.decode_nvfp4(ra, rsa, rga), oracle.decode_nvfp4(rb, rsb, rgb, N)
    elif fmt == pqm.FMT_FP8_BLOCK:
        qa, sa = pqm.quantize_fp8_block(dev_bf16(x), 1)
        qb, sb = pqm.quantize_fp8_block(dev_bf16(w), 128)
        kw = dict(a_outer=sa, b_outer=sb)
        ra, rsa = oracle.quantize_fp8_block(x, 1)
        rb, rsb = oracle.quantize_fp8_block(w, 128)
        A, B = oracle.decode_fp8_block(ra, rsa, 1), oracle.decode_fp8_block(rb, rsb, 128)
    else:
        qa, qb, kw = dev_bf16(x), dev_bf16(w), {}
        A, B = oracle.bf16_to_f64(x), oracle.bf16_to_f64(w)
    return qa, qb, kw, A, B.reshape(G, N, K)


@pytest.mark.parametrize("fmt,sizes,N,K,path", [
    (pqm.FMT_MXFP8, [300, 0, 513, 129], 512, 256, "persistent"),
    (pqm.FMT_MXFP8, [37, 0, 300, 129], 98, 256, "four-wave ring"),  # rows not whole 16 B
    (pqm.FMT_MXFP8, [37, 300], 128, 96, "register-staged"),
    (pqm.FMT_NVFP4, [300, 0, 513, 129, 64], 520, 512, "wide"),
    (pqm.FMT_NVFP4, [100, 60, 300], 256, 512, "pipelined"),
    (pqm.FMT_NVFP4, [64, 0, 200], 128, 336, "register-staged"),
    (pqm.FMT_FP8_BLOCK, [0, 37, 128, 1, 300], 256, 384, "block FP8"),
    (pqm.FMT_BF16, [0, 37, 128, 1, 300], 192, 320, "pipelined"),
    (pqm.FMT_BF16, [64, 64], 136, 72, "register-staged"),
])
@pytest.mark.parametrize("out_dtype", [pqm.OUT_FP32, pqm.OUT_BF16])
def test_forward_bias(fmt, sizes, N, K, path, out_dtype):
    G = len(sizes)
    qa, qb, kw, A, B = _operands(fmt, sizes, N, K, seed=51)
    off = _offsets(sizes)
    want0 = oracle.grouped_gemm(A, B, off)
    rng = np.random.Generator(np.random.PCG64(52))
    scale = float(np.abs(want0).mean()) if want0.size else 1.0
    bias = (rng.standard_normal((G, N)) * scale).astype(np.float32)
    print(f"[bias] fmt={fmt} {path} sizes={sizes} N={N} K={K} out={out_dtype}", flush=True)
    y = pqm.moe_grouped_gemm(fmt, pqm.GEMM_FPROP, qa, qb, dev(off), N, K, out_dtype=out_dtype,
                             bias=dev(bias), **kw)
    torch.cuda.synchronize()
    want = oracle.grouped_gemm(A, B, off, bias=bias)
    r = _rel_rows(host(y.float()), want)
    bar = TOL if out_dtype == pqm.OUT_FP32 else TOL + 2.0 ** -8
    print(f"[bias] max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= bar, (float(r.max()), int(r.argmax()))


@pytest.mark.parametrize("out_dtype", [pqm.OUT_FP32, pqm.OUT_BF16])
def test_empty_contraction_with_bias_writes_bias_rows(out_dtype):
    sizes, N = [5, 0, 17, 3], 40
    G, M = len(sizes), sum(sizes)
    off = _offsets(sizes)
    bias = np.random.Generator(np.random.PCG64(53)).standard_normal((G, N)).astype(np.float32)
    a = torch.empty((M, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((G * N, 0), dtype=torch.bfloat16, device="cuda")
    y = pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_FPROP, a, b, dev(off), N, 0,
                             out_dtype=out_dtype, bias=dev(bias))
    torch.cuda.synchronize()
    want = np.repeat(bias, sizes, axis=0)
    got = host(y.float())
    if out_dtype == pqm.OUT_FP32:
        assert np.array_equal(got, want)
    else:
        assert np.array_equal(got, torch.from_numpy(want).to(torch.bfloat16).float().numpy())
