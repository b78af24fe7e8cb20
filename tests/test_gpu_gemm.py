"""GPU parity of the grouped GEMMs against the oracle's binary64 product of
the same exactly-decoded operands.

Bar: relative L2 <= 1e-3 on binary32 output, per row (a row whose oracle
values overflow binary32 is excluded).  bf16 output adds one rounding of
at most 2^-9 relative per element to that bar.

The oracle quantizes the operands itself from the same generated bf16 bytes
(byte equality of the two quantizers is established separately)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import workloads as wl
from gpu_util import dev, dev_bf16, host, host_u16, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL = 1e-3
F32_MAX = float(np.finfo(np.float32).max)


def rel_l2_rows(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    got = got.astype(np.float64)
    ok = np.isfinite(want).all(axis=1) & (np.abs(want).max(axis=1) < F32_MAX)
    num = np.linalg.norm(got - want, axis=1)
    den = np.linalg.norm(want, axis=1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return np.where(ok, out, 0.0)


def check_rows(got, want, what):
    r = rel_l2_rows(got, want)
    print(f"[gemm] {what}: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL, (what, float(r.max()), int(r.argmax()))


def bf16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(key(a_bits) - key(b_bits))


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


# ------------------------------------------------------------------ MXFP8

def _mxfp8_case(sizes, N, K, seed, out_dtype=pqm.OUT_FP32):
    G = len(sizes)
    M = int(sum(sizes))
    x = wl.activations(max(M, 1), K, seed=seed)[:M]
    w = wl.normal_bf16((G * N, K), std=0.02, seed=seed + 1)
    off = _offsets(sizes)
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(x), colwise=False)
    qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w), colwise=False)
    y = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, dev(off), N, K,
                             a_scale=sa, b_scale=sb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ra, rsa = oracle.quantize_mxfp8_rowwise(x)
    rb, rsb = oracle.quantize_mxfp8_rowwise(w)
    want = oracle.grouped_gemm(oracle.decode_mxfp8(ra, rsa),
                               oracle.decode_mxfp8(rb, rsb).reshape(G, N, K), off)
    return y, want


@pytest.mark.parametrize("case", [
    ([0, 37, 128, 1, 300], 192, 320),
    ([128], 256, 256),
    ([5, 0, 0, 250], 96, 64),
    ([513], 128, 4096),
    ([0, 37, 128, 1, 300], 200, 384),        # K % 128 == 0: large-tile kernel
    ([260, 0, 3], 1536, 768),
])
def test_mxfp8_fprop_ragged(case):
    sizes, N, K = case
    y, want = _mxfp8_case(sizes, N, K, seed=3)
    check_rows(host(y), want, f"mxfp8 {sizes} N={N} K={K}")


def test_mxfp8_fprop_bf16_out():
    """bf16 output vs the binary64 product: the GEMM bar (1e-3) plus one
    bf16 rounding of the output (at most 2^-9 relative per element)."""
    y, want = _mxfp8_case([64, 0, 100], 128, 256, seed=4, out_dtype=pqm.OUT_BF16)
    got = oracle.bf16_to_f64(host_u16(y))
    r = rel_l2_rows(got, want)
    print(f"[gemm] mxfp8 bf16 out vs fp64: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL + 2.0 ** -9


def test_mxfp8_tiny_contract_expert_gemm():
    """128 x 256 contract tensor (outliers, a zero row, a bf16-max row)
    times a 256 x 256 expert weight."""
    x = wl.tiny_contract_tensor()
    w = wl.normal_bf16((256, 256), std=0.02, seed=5)
    off = np.array([0, 128], np.int64)
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(x), colwise=False)
    qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w), colwise=False)
    y = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, dev(off), 256, 256,
                             a_scale=sa, b_scale=sb)
    ra, rsa = oracle.quantize_mxfp8_rowwise(x)
    rb, rsb = oracle.quantize_mxfp8_rowwise(w)
    want = oracle.grouped_gemm(oracle.decode_mxfp8(ra, rsa),
                               oracle.decode_mxfp8(rb, rsb)[None], off)
    got = host(y)
    assert not got[1].any()                        # the all-zero row
    check_rows(got, want, "tiny contract")


def test_mxfp8_qwen3_gate_up_full_sampled():
    """Full Qwen3-30B-A3B FC1 shape: 8192 tokens x top-8 over 128 experts
    with Zipf(1.1) load (65536 rows), N = 1536, K = 2048.  All rows are
    computed on the GPU; sampled rows of every expert are checked."""
    T, E, k, H, N = 8192, 128, 8, 2048, 1536
    ids = wl.zipf_routing(T, E, k)
    off, src, _ = oracle.route(ids, E)
    x = wl.activations(T, H)
    xg = x[src // k]                                # expert-sorted rows
    M = xg.shape[0]
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(xg), colwise=False)
    w = wl.expert_weights(E, N, H, 0.02)
    qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w.reshape(E * N, H)), colwise=False)
    y = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, dev(off), N, H,
                             a_scale=sa, b_scale=sb)
    torch.cuda.synchronize()
    yh = host(y)
    rng = np.random.Generator(np.random.PCG64(17))
    experts = sorted(set(rng.choice(E, 12, replace=False).tolist()) | {0, E - 1})
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 6)]))
        ra, rsa = oracle.quantize_mxfp8_rowwise(xg[rows])
        rb, rsb = oracle.quantize_mxfp8_rowwise(w[e])
        want = oracle.decode_mxfp8(ra, rsa) @ oracle.decode_mxfp8(rb, rsb).T
        check_rows(yh[rows], want, f"qwen3 fc1 expert {e} ({hi - lo} rows)")
    assert M == T * k


def test_mxfp8_qwen3_down_full_sampled():
    """Full Qwen3-30B-A3B FC2 shape (the two-workgroups-per-CU kernel that
    runs K <= 1024): 65536 routed rows of D [.., 768] under Zipf(1.1) load,
    N = 2048, K = 768, bf16 output as in the layer; sampled rows of every
    checked expert against the binary64 product (bar + one bf16 rounding)."""
    T, E, k, H, I = 8192, 128, 8, 2048, 768
    ids = wl.zipf_routing(T, E, k)
    off, _, _ = oracle.route(ids, E)
    M = T * k
    d = wl.activations(M, I, seed=9)
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(d), colwise=False)
    w = wl.expert_weights(E, H, I, 0.02, tag=1)
    qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w.reshape(E * H, I)), colwise=False)
    y = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, dev(off), H, I,
                             a_scale=sa, b_scale=sb, out_dtype=pqm.OUT_BF16)
    torch.cuda.synchronize()
    yh = oracle.bf16_to_f64(host_u16(y))
    rng = np.random.Generator(np.random.PCG64(18))
    experts = sorted(set(rng.choice(E, 12, replace=False).tolist()) | {0, E - 1})
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 6)]))
        ra, rsa = oracle.quantize_mxfp8_rowwise(d[rows])
        rb, rsb = oracle.quantize_mxfp8_rowwise(w[e])
        want = oracle.decode_mxfp8(ra, rsa) @ oracle.decode_mxfp8(rb, rsb).T
        r = rel_l2_rows(yh[rows], want)
        print(f"[gemm] qwen3 fc2 expert {e} ({hi - lo} rows): max row rel-L2 {r.max():.3e}",
              flush=True)
        assert r.max() <= TOL + 2.0 ** -9, (e, float(r.max()))


# ------------------------------------------------- MXFP8 backward GEMMs

def _colwise_b_groups(qT, sT, G, K):
    """Exact values of the column-wise copy of a stacked [G*K, N] weight as
    per-expert B_g[n, k] = W_g[k, n]: [G, N, K]."""
    v = oracle.decode_mxfp8(qT, sT)                  # [N, G*K]
    N = v.shape[0]
    return np.ascontiguousarray(v.reshape(N, G, K).transpose(1, 0, 2))


@pytest.mark.parametrize("sizes,N,K", [([0, 37, 128, 1, 300], 192, 384), ([260, 0, 3], 160, 128),
                                         ([513], 224, 2048), ([70, 330], 288, 1536)])
def test_mxfp8_dgrad(sizes, N, K):
    """dX[m, n] = sum_k dY[m, k] W_g[k, n] with dY row-wise (blocks along k)
    and W from its column-wise copy (blocks along k, down W's columns)."""
    G, M = len(sizes), int(sum(sizes))
    dy = wl.activations(max(M, 1), K, seed=21)[:M]
    w = wl.normal_bf16((G * K, N), std=0.02, seed=22)
    off = _offsets(sizes)
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(dy), colwise=False)
    _, _, qT, sT = pqm.quantize_mxfp8(dev_bf16(w), rowwise=False)
    y = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_DGRAD, qa, qT, dev(off), N, K,
                             a_scale=sa, b_scale=sT)
    torch.cuda.synchronize()
    ra, rsa = oracle.quantize_mxfp8_rowwise(dy)
    rT, rsT = oracle.quantize_mxfp8_colwise(w)
    want = oracle.grouped_gemm(oracle.decode_mxfp8(ra, rsa), _colwise_b_groups(rT, rsT, G, K), off)
    check_rows(host(y), want, f"mxfp8 dgrad {sizes} N={N} K={K}")


def _padded(sizes, align=32):
    return [-(-s // align) * align for s in sizes]


def _pad_rows(x, sizes, align=32):
    """Each group's rows followed by zero rows up to a multiple of align."""
    out, lo = [], 0
    for s in sizes:
        blk = np.zeros((-(-s // align) * align, x.shape[1]), x.dtype)
        blk[:s] = x[lo:lo + s]
        out.append(blk)
        lo += s
    return np.concatenate(out) if out else x[:0]


def _mxfp8_wgrad_case(sizes, N, K, seed, out_dtype=pqm.OUT_FP32):
    G, M = len(sizes), int(sum(sizes))
    dy = _pad_rows(wl.activations(max(M, 1), N, seed=seed)[:M], sizes)
    x = _pad_rows(wl.activations(max(M, 1), K, seed=seed + 1)[:M], sizes)
    off = _offsets(_padded(sizes))
    _, _, aT, asT = pqm.quantize_mxfp8(dev_bf16(dy), rowwise=False)
    _, _, bT, bsT = pqm.quantize_mxfp8(dev_bf16(x), rowwise=False)
    y = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_WGRAD, aT, bT, dev(off), N, K,
                             a_scale=asT, b_scale=bsT, out_dtype=out_dtype)
    torch.cuda.synchronize()
    rA, rsA = oracle.quantize_mxfp8_colwise(dy)
    rB, rsB = oracle.quantize_mxfp8_colwise(x)
    want = oracle.grouped_gemm_wgrad(oracle.decode_mxfp8(rA, rsA).T,
                                     oracle.decode_mxfp8(rB, rsB).T, off)
    return y, want


@pytest.mark.parametrize("sizes,N,K", [
    ([0, 37, 128, 1, 300], 192, 320),   # empty, one-row and ragged experts
    ([2500, 3, 70], 256, 160),           # a 2048-token pass plus a tail
    ([100, 0, 33, 257], 544, 288),       # output edges inside a tile
    ([4200], 64, 512),                   # three passes
])
def test_mxfp8_wgrad(sizes, N, K):
    """dW_g = dY_g^T X_g from the column-wise copies, each expert's rows
    padded with zero rows to whole 32-row blocks."""
    y, want = _mxfp8_wgrad_case(sizes, N, K, seed=23)
    got = host(y)
    assert got.shape == (len(sizes), N, K)
    for g, s in enumerate(sizes):
        if s == 0:
            assert not got[g].any()
        else:
            check_rows(got[g], want[g], f"mxfp8 wgrad {sizes} group {g}")


def test_mxfp8_wgrad_bf16_out():
    y, want = _mxfp8_wgrad_case([300, 0, 129], 288, 192, seed=25, out_dtype=pqm.OUT_BF16)
    got = host_u16(y)
    for g in (0, 2):
        r = rel_l2_rows(oracle.bf16_to_f64(got[g]), want[g])
        print(f"[gemm] mxfp8 wgrad bf16 out group {g}: max row rel-L2 {r.max():.3e}", flush=True)
        assert r.max() <= TOL + 2.0 ** -9
    assert not got[1].any()


# ------------------------------------------------------ block-scaled FP8

def _fp8b_case(sizes, N, K, seed, out_dtype=pqm.OUT_FP32):
    G, M = len(sizes), int(sum(sizes))
    x = wl.activations(max(M, 1), K, seed=seed)[:M]
    w = wl.normal_bf16((G * N, K), std=0.02, seed=seed + 1)
    off = _offsets(sizes)
    qa, sa = pqm.quantize_fp8_block(dev_bf16(x), 1)
    qb, sb = pqm.quantize_fp8_block(dev_bf16(w), 128)
    y = pqm.moe_grouped_gemm(pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, qa, qb, dev(off), N, K,
                             a_outer=sa, b_outer=sb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ra, rsa = oracle.quantize_fp8_block(x, 1)
    rb, rsb = oracle.quantize_fp8_block(w, 128)
    want = oracle.grouped_gemm(oracle.decode_fp8_block(ra, rsa, 1),
                               oracle.decode_fp8_block(rb, rsb, 128).reshape(G, N, K), off)
    return y, want


@pytest.mark.parametrize("sizes,N,K", [([0, 37, 128, 1, 300], 256, 384),
                                         ([260, 0, 3], 384, 128),
                                         ([513], 128, 7168),
                                         ([70, 330], 1536, 2048)])
def test_fp8_block_fprop(sizes, N, K):
    """Y = sum over 128-K blocks of sa sb (block sum of E4M3 products)
    against the oracle's binary64 product of the decoded operands."""
    y, want = _fp8b_case(sizes, N, K, seed=61)
    check_rows(host(y), want, f"fp8 block {sizes} N={N} K={K}")


def test_fp8_block_fprop_bf16_out_and_contract_tensor():
    y, want = _fp8b_case([64, 0, 100], 256, 256, seed=62, out_dtype=pqm.OUT_BF16)
    r = rel_l2_rows(oracle.bf16_to_f64(host_u16(y)), want)
    assert r.max() <= TOL + 2.0 ** -9
    x = wl.tiny_contract_tensor()
    w = wl.normal_bf16((256, 256), std=0.02, seed=63)
    off = np.array([0, 128], np.int64)
    qa, sa = pqm.quantize_fp8_block(dev_bf16(x), 1)
    qb, sb = pqm.quantize_fp8_block(dev_bf16(w), 128)
    y = pqm.moe_grouped_gemm(pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, qa, qb, dev(off), 256, 256,
                             a_outer=sa, b_outer=sb)
    ra, rsa = oracle.quantize_fp8_block(x, 1)
    rb, rsb = oracle.quantize_fp8_block(w, 128)
    want = oracle.grouped_gemm(oracle.decode_fp8_block(ra, rsa, 1),
                               oracle.decode_fp8_block(rb, rsb, 128)[None], off)
    got = host(y)
    assert not got[1].any()
    check_rows(got, want, "fp8 block tiny contract")


def test_fp8_block_qwen3_gate_up_full_sampled():
    """The Qwen3-30B-A3B FC1 shape in block FP8 (65536 routed rows, Zipf
    loads, N = 1536, K = 2048), all rows on the GPU, sampled rows of sampled
    experts against the oracle."""
    T, E, k, H, N = 8192, 128, 8, 2048, 1536
    ids = wl.zipf_routing(T, E, k)
    off, src, _ = oracle.route(ids, E)
    x = wl.activations(T, H)
    xg = x[src // k]
    w = wl.expert_weights(E, N, H, 0.02)
    qa, sa = pqm.quantize_fp8_block(dev_bf16(xg), 1)
    qb, sb = pqm.quantize_fp8_block(dev_bf16(w.reshape(E * N, H)), 128)
    y = pqm.moe_grouped_gemm(pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, qa, qb, dev(off), N, H,
                             a_outer=sa, b_outer=sb)
    torch.cuda.synchronize()
    yh = host(y)
    rng = np.random.Generator(np.random.PCG64(64))
    for e in sorted(set(rng.choice(E, 8, replace=False).tolist()) | {0, E - 1}):
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 6)]))
        ra, rsa = oracle.quantize_fp8_block(xg[rows], 1)
        rb, rsb = oracle.quantize_fp8_block(w[e], 128)
        want = oracle.decode_fp8_block(ra, rsa, 1) @ oracle.decode_fp8_block(rb, rsb, 128).T
        check_rows(yh[rows], want, f"fp8 block qwen3 fc1 expert {e} ({hi - lo} rows)")


# ------------------------------------------------------------------- BF16

def _bf16_operands(M, N, K, G, seed):
    a = wl.normal_bf16((M, K), seed=seed)
    b = wl.normal_bf16((G, N, K), std=0.05, seed=seed + 1)
    return a, b


@pytest.mark.parametrize("sizes,N,K", [([0, 37, 128, 1, 300], 192, 320), ([200], 256, 64),
                                         ([300, 0, 513, 129, 64], 520, 384)])
def test_bf16_fprop(sizes, N, K):
    G = len(sizes)
    M = int(sum(sizes))
    a, b = _bf16_operands(M, N, K, G, 7)
    off = _offsets(sizes)
    y = pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_FPROP, dev_bf16(a),
                             dev_bf16(b.reshape(G * N, K)), dev(off), N, K)
    want = oracle.grouped_gemm(oracle.bf16_to_f64(a),
                               oracle.bf16_to_f64(b.reshape(-1, K)).reshape(G, N, K), off)
    check_rows(host(y), want, f"bf16 fprop {sizes}")


@pytest.mark.parametrize("sizes,N,K", [([0, 37, 128, 1, 300], 192, 320), ([64, 64], 136, 72),
                                         ([300, 0, 513, 129, 64], 520, 384)])
def test_bf16_dgrad(sizes, N, K):
    """dX[m, n] = sum_k dY[m, k] W_g[k, n]: W stored [G, K, N] (the forward
    weight [out, in] with the contraction over its rows)."""
    G = len(sizes)
    M = int(sum(sizes))
    dy = wl.normal_bf16((M, K), seed=9)
    w = wl.normal_bf16((G, K, N), std=0.05, seed=10)
    off = _offsets(sizes)
    y = pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, dev_bf16(dy),
                             dev_bf16(w.reshape(G * K, N)), dev(off), N, K)
    wt = np.ascontiguousarray(np.transpose(oracle.bf16_to_f64(w.reshape(-1, N)).reshape(G, K, N),
                                           (0, 2, 1)))
    want = oracle.grouped_gemm(oracle.bf16_to_f64(dy), wt, off)
    check_rows(host(y), want, f"bf16 dgrad {sizes}")


def test_bf16_dgrad_bf16_out():
    """bf16 output: the GEMM bar plus one bf16 rounding (2^-9 relative)."""
    sizes, N, K = [300, 0, 129, 64], 264, 192
    G, M = len(sizes), sum(sizes)
    dy = wl.normal_bf16((M, K), seed=13)
    w = wl.normal_bf16((G, K, N), std=0.05, seed=14)
    off = _offsets(sizes)
    y = pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, dev_bf16(dy),
                             dev_bf16(w.reshape(G * K, N)), dev(off), N, K,
                             out_dtype=pqm.OUT_BF16)
    wt = np.ascontiguousarray(np.transpose(oracle.bf16_to_f64(w.reshape(-1, N)).reshape(G, K, N),
                                           (0, 2, 1)))
    want = oracle.grouped_gemm(oracle.bf16_to_f64(dy), wt, off)
    r = rel_l2_rows(oracle.bf16_to_f64(host_u16(y)), want)
    print(f"[gemm] bf16 dgrad bf16 out: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL + 2.0 ** -9


@pytest.mark.parametrize("sizes,N,K", [([0, 37, 128, 1, 300], 192, 320), ([700], 64, 136),
                                         ([1000, 0, 33, 257], 520, 264)])
def test_bf16_wgrad(sizes, N, K):
    G = len(sizes)
    M = int(sum(sizes))
    dy = wl.normal_bf16((max(M, 1), N), seed=11)[:M]
    x = wl.normal_bf16((max(M, 1), K), seed=12)[:M]
    off = _offsets(sizes)
    y = pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_WGRAD, dev_bf16(dy), dev_bf16(x),
                             dev(off), N, K)
    want = oracle.grouped_gemm_wgrad(oracle.bf16_to_f64(dy), oracle.bf16_to_f64(x), off)
    got = host(y)
    assert got.shape == (G, N, K)
    for g in range(G):
        if sizes[g] == 0:
            assert not got[g].any()
        else:
            check_rows(got[g], want[g], f"bf16 wgrad group {g}")


# ------------------------------------------------------------------ NVFP4

def _nvfp4_case(sizes, N, K, seed, brps=None):
    """A per-token NVFP4, B one outer scale per expert tensor (brps = N) or
    per half (gate / up separately)."""
    G = len(sizes)
    M = int(sum(sizes))
    brps = brps or N
    x = wl.activations(max(M, 1), K, seed=seed)[:M]
    w = wl.normal_bf16((G * N, K), std=0.01, seed=seed + 1)
    off = _offsets(sizes)
    qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(x))
    qb, sb, gb = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=brps)
    y = pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, dev(off), N, K,
                             a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb,
                             b_rows_per_scale=brps)
    torch.cuda.synchronize()
    ra, rsa, rga = oracle.quantize_nvfp4(x)
    rb, rsb, rgb = oracle.quantize_nvfp4(w, rows_per_group=brps)
    want = oracle.grouped_gemm(oracle.decode_nvfp4(ra, rsa, rga),
                               oracle.decode_nvfp4(rb, rsb, rgb, brps).reshape(G, N, K), off)
    return y, want


@pytest.mark.parametrize("case", [
    ([0, 37, 128, 1, 300], 192, 320, None),
    ([64, 0, 200], 128, 336, None),           # K % 64 == 16: remainder step
    ([100, 60], 256, 512, 128),               # gate and up scaled separately
    ([300, 0, 513, 129, 64], 520, 768, None),  # 256- and 128-row tiles, ragged N
    ([300, 0, 513, 129, 64], 520, 512, 260),   # scale boundaries inside 8-column runs
])
def test_nvfp4_fprop_ragged(case):
    sizes, N, K, brps = case
    y, want = _nvfp4_case(sizes, N, K, seed=21, brps=brps)
    check_rows(host(y), want, f"nvfp4 {sizes} N={N} K={K}")


def test_nvfp4_tiny_contract_expert_gemm():
    x = wl.tiny_contract_tensor()
    w = wl.normal_bf16((256, 256), std=0.02, seed=5)
    off = np.array([0, 128], np.int64)
    qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(x))
    qb, sb, gb = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=256)
    y = pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, dev(off), 256, 256,
                             a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb,
                             b_rows_per_scale=256)
    ra, rsa, rga = oracle.quantize_nvfp4(x)
    rb, rsb, rgb = oracle.quantize_nvfp4(w, rows_per_group=256)
    want = oracle.grouped_gemm(oracle.decode_nvfp4(ra, rsa, rga),
                               oracle.decode_nvfp4(rb, rsb, rgb, 256)[None], off)
    got = host(y)
    assert not got[1].any()
    check_rows(got, want, "nvfp4 tiny contract")


def test_nvfp4_deepseek_gate_up_full_sampled():
    """DeepSeek-V3 expert shape: 4096 tokens top-8 over 256 routed experts
    (half uniform, half Zipf) plus the shared expert as group 256 with every
    token; gate_up N = 4096, K = 7168; weights N(0, 0.01) drawn on the GPU
    from a seeded generator, quantized with one outer scale per expert
    (joint gate/up).  Sampled rows of sampled experts vs the oracle."""
    T, E, k, H, N = 4096, 256, 8, 7168, 4096
    ids = wl.uniform_plus_zipf_routing(T, E, k)
    off_r, src, _ = oracle.route(ids, E)
    M_r = T * k
    off = np.concatenate([off_r, [M_r + T]]).astype(np.int64)
    x = wl.activations(T, H, seed=5)
    rows_tok = np.concatenate([src // k, np.arange(T)])
    xg = x[rows_tok]
    gen = torch.Generator(device="cuda").manual_seed(1234)
    w = (torch.randn((E + 1) * N, H, generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(xg))
    qb, sb, gb = pqm.quantize_nvfp4_per_token(w, rows_per_scale=N)
    y = pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, dev(off), N, H,
                             a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb,
                             b_rows_per_scale=N, out_dtype=pqm.OUT_FP32)
    torch.cuda.synchronize()
    yh = host(y)
    rng = np.random.Generator(np.random.PCG64(23))
    for e in [0, int(rng.integers(1, E)), E - 1, E]:        # E = the shared expert
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 4)]))
        we = host_u16(w[e * N:(e + 1) * N])
        ra, rsa, rga = oracle.quantize_nvfp4(xg[rows])
        rb, rsb, rgb = oracle.quantize_nvfp4(we, rows_per_group=N)
        want = oracle.decode_nvfp4(ra, rsa, rga) @ oracle.decode_nvfp4(rb, rsb, rgb, N).T
        check_rows(yh[rows], want, f"deepseek fc1 expert {e} ({hi - lo} rows)")
    del w, qb


# ------------------------------------------------- bf16 output rounding

def _rne_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bits of finite binary32 values (host reference)."""
    u = f32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt,sizes,N,K", [
    ("mxfp8", [300, 0, 513, 129, 64], 520, 2048),  # 256 x 256 kernel
    ("mxfp8", [300, 0, 513, 129, 64], 520, 768),   # 128 x 256 two-per-CU kernel
    ("nvfp4", [300, 0, 513, 129, 64], 520, 768),
])
def test_bf16_output_is_rne_of_binary32_output(fmt, sizes, N, K):
    """The bf16-output epilogue rounds the same binary32 accumulators the
    binary32-output epilogue stores: every element must be their nearest-
    even bf16 (checks the hardware pair conversion on ~0.5 M values)."""
    G, M = len(sizes), int(sum(sizes))
    off = dev(_offsets(sizes))
    x = dev_bf16(wl.activations(M, K, seed=31))
    w = dev_bf16(wl.normal_bf16((G * N, K), std=0.02, seed=32))
    if fmt == "mxfp8":
        qa, sa, _, _ = pqm.quantize_mxfp8(x, colwise=False)
        qb, sb, _, _ = pqm.quantize_mxfp8(w, colwise=False)
        kw = dict(a_scale=sa, b_scale=sb)
        f = pqm.FMT_MXFP8
    else:
        qa, sa, ga = pqm.quantize_nvfp4_per_token(x)
        qb, sb, gb = pqm.quantize_nvfp4_per_token(w, rows_per_scale=N)
        kw = dict(a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb, b_rows_per_scale=N)
        f = pqm.FMT_NVFP4
    y32 = pqm.moe_grouped_gemm(f, pqm.GEMM_FPROP, qa, qb, off, N, K, out_dtype=pqm.OUT_FP32, **kw)
    y16 = pqm.moe_grouped_gemm(f, pqm.GEMM_FPROP, qa, qb, off, N, K, out_dtype=pqm.OUT_BF16, **kw)
    torch.cuda.synchronize()
    want = _rne_bf16_bits(host(y32))
    got = host_u16(y16)
    assert np.isfinite(host(y32)).all()
    bad = int((got != want).sum())
    print(f"[gemm] {fmt} K={K} bf16 output vs RNE(binary32 output): {bad} mismatches "
          f"of {got.size}", flush=True)
    assert bad == 0
