"""GPU parity of the grouped GEMMs on seeded random shapes: the persistent
paths (the MXFP8 forward and dgrad on the eight-wave 256 x 256 kernel, the
NVFP4 forward on 128 x 512 tiles), and every other path (MXFP8 and NVFP4
shapes below those tiles, the MXFP8 weight gradient, block FP8 and the BF16
forward, dgrad and weight gradient, forward cases with and without bias).
Each case draws an expert count and expert sizes (empty experts, tails of
every fragment count, several row tiles), N and K from the sizes the path
takes.

Bars, per case:
  * bf16 output bit for bit the nearest-even rounding of the same call's
    binary32 output;
  * binary32 output within relative L2 1e-3 per row of the oracle's
    binary64 product of the exactly decoded operands."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import workloads as wl
from gpu_util import assert_bytes_equal, dev, dev_bf16, host, host_u16, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 1e-3
SIZES = [0, 0, 1, 7, 31, 32, 33, 64, 97, 128, 129, 255, 256, 300, 513]


def _cases(n=18, seed=2024):
    """n cases of (kind, sizes, N, K), the weights' element count kept small
    enough for the oracle (G N K <= 4e7)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        kind = ("mxfp8", "mxfp8_dgrad", "nvfp4")[len(out) % 3]
        G = int(rng.choice([1, 2, 5, 17, 64, 300]))
        sizes = rng.choice(SIZES, size=G).tolist()
        if sum(sizes) == 0:
            sizes[0] = 5
        if kind == "nvfp4":
            N, K = int(rng.choice([512, 544, 1024])), int(rng.choice([768, 1024, 1280]))
        else:
            N = int(rng.choice([256, 288, 544, 1024]))
            K = int(rng.choice([512, 640, 1024]))
        if G * N * K > 4e7 or sum(sizes) > 6000:
            continue
        out.append((kind, sizes, N, K, int(rng.integers(1 << 30))))
    return out


def _rne_bf16_bits(f32: np.ndarray) -> np.ndarray:
    u = f32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _rel_rows(got, want):
    num = np.linalg.norm(got.astype(np.float64) - want, axis=1)
    den = np.linalg.norm(want, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-G{len(c[1])}-{c[2]}x{c[3]}")
def test_random_shapes(case):
    kind, sizes, N, K, seed = case
    G, M = len(sizes), int(sum(sizes))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    x = wl.activations(M, K, seed=seed)
    print(f"[random] {kind} G={G} M={M} N={N} K={K}", flush=True)
    if kind == "mxfp8":
        w = wl.normal_bf16((G * N, K), std=0.02, seed=seed + 1)
        qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(x), colwise=False)
        qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w), colwise=False)
        args = (pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, dev(off), N, K)
        kw = dict(a_scale=sa, b_scale=sb)
        ra, rsa = oracle.quantize_mxfp8_rowwise(x)
        rb, rsb = oracle.quantize_mxfp8_rowwise(w)
        B = oracle.decode_mxfp8(rb, rsb).reshape(G, N, K)
        A = oracle.decode_mxfp8(ra, rsa)
    elif kind == "mxfp8_dgrad":
        w = wl.normal_bf16((G * K, N), std=0.02, seed=seed + 1)
        qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(x), colwise=False)
        _, _, qT, sT = pqm.quantize_mxfp8(dev_bf16(w), rowwise=False)
        args = (pqm.FMT_MXFP8, pqm.GEMM_DGRAD, qa, qT, dev(off), N, K)
        kw = dict(a_scale=sa, b_scale=sT)
        ra, rsa = oracle.quantize_mxfp8_rowwise(x)
        rT, rsT = oracle.quantize_mxfp8_colwise(w)
        B = np.ascontiguousarray(oracle.decode_mxfp8(rT, rsT).reshape(N, G, K).transpose(1, 0, 2))
        A = oracle.decode_mxfp8(ra, rsa)
    else:
        w = wl.normal_bf16((G * N, K), std=0.01, seed=seed + 1)
        qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(x))
        qb, sb, gb = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
        args = (pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, dev(off), N, K)
        kw = dict(a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb, b_rows_per_scale=N)
        ra, rsa, rga = oracle.quantize_nvfp4(x)
        rb, rsb, rgb = oracle.quantize_nvfp4(w, rows_per_group=N)
        B = oracle.decode_nvfp4(rb, rsb, rgb, N).reshape(G, N, K)
        A = oracle.decode_nvfp4(ra, rsa, rga)
    y16 = pqm.moe_grouped_gemm(*args, out_dtype=pqm.OUT_BF16, **kw)
    y32 = pqm.moe_grouped_gemm(*args, out_dtype=pqm.OUT_FP32, **kw)
    torch.cuda.synchronize()
    assert_bytes_equal(host_u16(y16), _rne_bf16_bits(host(y32)), f"{kind} bf16 vs RNE(binary32)")
    r = _rel_rows(host(y32), oracle.grouped_gemm(A, B, off))
    print(f"[random] max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL, (kind, float(r.max()), int(r.argmax()))


# ------------------------------------------ every other grouped-GEMM path

KINDS = ("mxfp8_small", "mxfp8_wgrad", "nvfp4_small", "fp8_block", "bf16", "bf16_dgrad",
         "bf16_wgrad")
SMALL_SIZES = [0, 1, 17, 32, 33, 64, 100, 128, 200, 256, 300]


def _path_cases(n=21, seed=7):
    """n cases over the paths the persistent kernels leave to others: MXFP8
    forward with N or K below a tile (register-staged and four-wave kernels),
    the MXFP8 weight gradient, NVFP4 with N below the wide tile, block FP8,
    and the BF16 forward, dgrad and weight gradient.  Forward cases draw a
    bias in two of five; every N is a multiple of 8 so that both output
    types take the same kernel."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        kind = KINDS[len(out) % len(KINDS)]
        G = int(rng.choice([1, 3, 9, 40]))
        sizes = rng.choice(SMALL_SIZES, size=G).tolist()
        if sum(sizes) == 0:
            sizes[0] = 3
        N, K = {
            "mxfp8_small": lambda: (int(rng.choice([64, 96, 200, 288])), int(rng.choice([64, 128, 384]))),
            "mxfp8_wgrad": lambda: (int(rng.choice([64, 96, 160, 288])), int(rng.choice([64, 96, 256]))),
            "nvfp4_small": lambda: (int(rng.choice([128, 256, 336])), int(rng.choice([256, 512, 768]))),
            "fp8_block": lambda: (int(rng.choice([128, 256, 384])), int(rng.choice([128, 256, 512]))),
        }.get(kind, lambda: (int(rng.choice([64, 136, 192, 520])), int(rng.choice([64, 72, 128, 320]))))()
        if G * N * K > 3e7 or sum(sizes) * max(N, K) > 3e7:
            continue
        bias = kind in ("mxfp8_small", "nvfp4_small", "fp8_block", "bf16") and rng.random() < 0.4
        out.append((kind, sizes, N, K, bias, int(rng.integers(1 << 30))))
    return out


def _pad32(x, sizes):
    """Each expert's rows followed by zero rows up to a multiple of 32."""
    blocks, lo = [], 0
    for s in sizes:
        b = np.zeros((-(-s // 32) * 32, x.shape[1]), x.dtype)
        b[:s] = x[lo:lo + s]
        blocks.append(b)
        lo += s
    return np.concatenate(blocks)


def _path_case(kind, sizes, N, K, use_bias, seed):
    """(call(out_dtype), expected binary64 output as rows)."""
    G, M = len(sizes), int(sum(sizes))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    rng = np.random.default_rng(seed)
    bias = (rng.standard_normal((G, N)) * 0.1).astype(np.float32) if use_bias else None
    kw = {"bias": dev(bias)} if use_bias else {}
    if kind in ("mxfp8_wgrad", "bf16_wgrad"):
        dy, x = wl.activations(M, N, seed=seed), wl.activations(M, K, seed=seed + 1)
        if kind == "bf16_wgrad":
            args = (pqm.FMT_BF16, pqm.GEMM_WGRAD, dev_bf16(dy), dev_bf16(x), dev(off), N, K)
            want = oracle.grouped_gemm_wgrad(oracle.bf16_to_f64(dy), oracle.bf16_to_f64(x), off)
        else:
            dyp, xp = _pad32(dy, sizes), _pad32(x, sizes)
            offp = np.concatenate([[0], np.cumsum([-(-s // 32) * 32 for s in sizes])]).astype(np.int64)
            _, _, aT, asT = pqm.quantize_mxfp8(dev_bf16(dyp), rowwise=False)
            _, _, bT, bsT = pqm.quantize_mxfp8(dev_bf16(xp), rowwise=False)
            args = (pqm.FMT_MXFP8, pqm.GEMM_WGRAD, aT, bT, dev(offp), N, K)
            kw = dict(a_scale=asT, b_scale=bsT)
            rA, rsA = oracle.quantize_mxfp8_colwise(dyp)
            rB, rsB = oracle.quantize_mxfp8_colwise(xp)
            want = oracle.grouped_gemm_wgrad(oracle.decode_mxfp8(rA, rsA).T,
                                             oracle.decode_mxfp8(rB, rsB).T, offp)
        return (lambda od: pqm.moe_grouped_gemm(*args, out_dtype=od, **kw)), want.reshape(-1, K)
    x = wl.activations(M, K, seed=seed)
    if kind == "bf16_dgrad":
        w = wl.normal_bf16((G * K, N), std=0.02, seed=seed + 1)
        args = (pqm.FMT_BF16, pqm.GEMM_DGRAD, dev_bf16(x), dev_bf16(w), dev(off), N, K)
        B = np.ascontiguousarray(oracle.bf16_to_f64(w).reshape(G, K, N).transpose(0, 2, 1))
        return (lambda od: pqm.moe_grouped_gemm(*args, out_dtype=od)), \
            oracle.grouped_gemm(oracle.bf16_to_f64(x), B, off)
    w = wl.normal_bf16((G * N, K), std=0.02, seed=seed + 1)
    if kind == "mxfp8_small":
        qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(x), colwise=False)
        qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w), colwise=False)
        args, kw = (pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb), dict(kw, a_scale=sa, b_scale=sb)
        ra, rsa = oracle.quantize_mxfp8_rowwise(x)
        rb, rsb = oracle.quantize_mxfp8_rowwise(w)
        A, B = oracle.decode_mxfp8(ra, rsa), oracle.decode_mxfp8(rb, rsb)
    elif kind == "nvfp4_small":
        qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(x))
        qb, sb, gb = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
        args = (pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb)
        kw = dict(kw, a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb, b_rows_per_scale=N)
        ra, rsa, rga = oracle.quantize_nvfp4(x)
        rb, rsb, rgb = oracle.quantize_nvfp4(w, rows_per_group=N)
        A, B = oracle.decode_nvfp4(ra, rsa, rga), oracle.decode_nvfp4(rb, rsb, rgb, N)
    elif kind == "fp8_block":
        qa, sa = pqm.quantize_fp8_block(dev_bf16(x), 1)
        qb, sb = pqm.quantize_fp8_block(dev_bf16(w), 128)
        args, kw = (pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, qa, qb), dict(kw, a_outer=sa, b_outer=sb)
        ra, rsa = oracle.quantize_fp8_block(x, 1)
        rb, rsb = oracle.quantize_fp8_block(w, 128)
        A, B = oracle.decode_fp8_block(ra, rsa, 1), oracle.decode_fp8_block(rb, rsb, 128)
    else:
        args = (pqm.FMT_BF16, pqm.GEMM_FPROP, dev_bf16(x), dev_bf16(w))
        A, B = oracle.bf16_to_f64(x), oracle.bf16_to_f64(w)
    want = oracle.grouped_gemm(A, B.reshape(G, N, K), off, bias=bias)
    return (lambda od: pqm.moe_grouped_gemm(*args, dev(off), N, K, out_dtype=od, **kw)), want


@pytest.mark.parametrize("case", _path_cases(),
                         ids=lambda c: f"{c[0]}-G{len(c[1])}-{c[2]}x{c[3]}{'-bias' if c[4] else ''}")
def test_random_paths(case):
    """Same bars as the persistent cases: bf16 output bit for bit the
    nearest-even rounding of the binary32 output, binary32 within 1e-3 per
    row of the oracle (weight gradients: per row of each expert's N x K)."""
    kind, sizes, N, K, use_bias, seed = case
    print(f"[random] {kind} G={len(sizes)} M={sum(sizes)} N={N} K={K} bias={use_bias}", flush=True)
    call, want = _path_case(kind, sizes, N, K, use_bias, seed)
    y32 = call(pqm.OUT_FP32)
    y16 = call(pqm.OUT_BF16)
    torch.cuda.synchronize()
    got = host(y32).reshape(want.shape)
    assert_bytes_equal(host_u16(y16).reshape(-1), _rne_bf16_bits(got).reshape(-1),
                       f"{kind} bf16 vs RNE(binary32)")
    r = _rel_rows(got, want)
    print(f"[random] max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL, (kind, float(r.max()), int(r.argmax()))
