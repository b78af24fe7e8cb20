"""GPU parity of the grouped GEMMs against the oracle's binary64 product of
the same exactly-decoded operands.

Bar: relative L2 <= 1e-3 on binary32 output, per row (a row whose oracle
values overflow binary32 is excluded).  bf16 output adds one nearest-even
rounding to 8 significant bits, at most 2^-8 relative per element, to that
bar.

The oracle quantizes the operands itself from the same generated bf16 bytes
(byte equality of the two quantizers is established separately)."""
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


@pytest.mark.parametrize("N", [128, 100])
def test_mxfp8_fprop_bf16_out(N):
    """bf16 output vs the binary64 product: the GEMM bar (1e-3) plus one
    bf16 rounding of the output (at most 2^-8 relative per element).  N =
    100 (rows of 200 bytes, not whole 16-byte vectors) runs the
    non-persistent kernel."""
    y, want = _mxfp8_case([64, 0, 100, 300], N, 256, seed=4, out_dtype=pqm.OUT_BF16)
    got = oracle.bf16_to_f64(host_u16(y))
    r = rel_l2_rows(got, want)
    print(f"[gemm] mxfp8 bf16 out vs fp64: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL + 2.0 ** -8


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
    """Full Qwen3-30B-A3B FC2 shape (the persistent 256 x 256 kernel, bf16
    output): 65536 routed rows of D [.., 768] under Zipf(1.1) load,
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
        assert r.max() <= TOL + 2.0 ** -8, (e, float(r.max()))


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


@pytest.mark.parametrize("sizes,N,K", [
    ([0, 37, 128, 1, 300, 513], 544, 768),    # ragged, a last column tile 32 wide, 6 steps
    ("many", 256, 512),                       # 600 mostly tiny experts: many tiles per workgroup
])
def test_mxfp8_dgrad_bf16_out(sizes, N, K):
    """The dgrad on the persistent kernel (B's row stride G K, expert stride
    K) with bf16 output: bit for bit the nearest-even rounding of its binary32
    output, and the oracle bar plus one bf16 rounding."""
    if sizes == "many":
        sizes = _many_small_groups(600, seed=23)
    G, M = len(sizes), int(sum(sizes))
    dy = wl.activations(M, K, seed=24)
    w = wl.normal_bf16((G * K, N), std=0.02, seed=25)
    off = _offsets(sizes)
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(dy), colwise=False)
    _, _, qT, sT = pqm.quantize_mxfp8(dev_bf16(w), rowwise=False)
    print(f"[gemm] mxfp8 dgrad bf16 G={G} M={M} N={N} K={K}", flush=True)
    y16 = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_DGRAD, qa, qT, dev(off), N, K,
                               a_scale=sa, b_scale=sT, out_dtype=pqm.OUT_BF16)
    y32 = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_DGRAD, qa, qT, dev(off), N, K,
                               a_scale=sa, b_scale=sT, out_dtype=pqm.OUT_FP32)
    torch.cuda.synchronize()
    got = host_u16(y16)
    assert_bytes_equal(got, _rne_bf16_bits(host(y32)), "bf16 vs RNE(binary32)")
    ra, rsa = oracle.quantize_mxfp8_rowwise(dy)
    rT, rsT = oracle.quantize_mxfp8_colwise(w)
    want = oracle.grouped_gemm(oracle.decode_mxfp8(ra, rsa), _colwise_b_groups(rT, rsT, G, K), off)
    r = rel_l2_rows(oracle.bf16_to_f64(got), want)
    print(f"[gemm] mxfp8 dgrad bf16: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL + 2.0 ** -8, (float(r.max()), int(r.argmax()))


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


@pytest.mark.parametrize("sizes,N,K", [
    ([0, 37, 128, 1, 300], 192, 320),
    ([5000, 0, 0, 96, 64, 32, 160], 544, 288),
    ([int(v) for v in np.random.Generator(np.random.PCG64(61)).integers(0, 90, 300)], 64, 96),
])
@pytest.mark.parametrize("out_dtype", [pqm.OUT_FP32, pqm.OUT_BF16])
def test_mxfp8_wgrad_kernels_agree(sizes, N, K, out_dtype):
    """The persistent weight-gradient kernel against the general one, which
    runs when an output row is not a whole number of 16-byte vectors (here
    K - 1 columns of the same operands): the same MFMAs in the same token
    order, so the same bits (empty experts, tails of 32 to 96 tokens, 300
    experts over fewer workgroups than tiles); and with the tiles handed out
    through the workspace counter or dealt in a fixed order."""
    M = int(sum(sizes))
    dy = _pad_rows(wl.activations(max(M, 1), N, seed=71)[:M], sizes)
    x = _pad_rows(wl.activations(max(M, 1), K, seed=72)[:M], sizes)
    off = dev(_offsets(_padded(sizes)))
    _, _, aT, asT = pqm.quantize_mxfp8(dev_bf16(dy), rowwise=False)
    _, _, bT, bsT = pqm.quantize_mxfp8(dev_bf16(x), rowwise=False)
    y1 = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_WGRAD, aT, bT, off, N, K,
                              a_scale=asT, b_scale=bsT, out_dtype=out_dtype)
    y2 = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_WGRAD, aT, bT[:K - 1], off, N, K - 1,
                              a_scale=asT, b_scale=bsT[:K - 1], out_dtype=out_dtype)
    y3 = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_WGRAD, aT, bT, off, N, K,
                              a_scale=asT, b_scale=bsT, out_dtype=out_dtype, workspace=False)
    torch.cuda.synchronize()
    it = torch.int32 if out_dtype == pqm.OUT_FP32 else torch.int16
    a1, a2, a3 = (y.view(it).cpu().numpy() for y in (y1, y2, y3))
    assert np.array_equal(a1[:, :, :K - 1], a2), f"wgrad kernels differ {sizes[:8]} N={N} K={K}"
    assert np.array_equal(a1, a3), "handed-out and fixed tile orders differ"
    for g, s in enumerate(sizes):
        if s == 0:
            assert not a1[g].any()


def test_mxfp8_wgrad_bf16_out():
    y, want = _mxfp8_wgrad_case([300, 0, 129], 288, 192, seed=25, out_dtype=pqm.OUT_BF16)
    got = host_u16(y)
    for g in (0, 2):
        r = rel_l2_rows(oracle.bf16_to_f64(got[g]), want[g])
        print(f"[gemm] mxfp8 wgrad bf16 out group {g}: max row rel-L2 {r.max():.3e}", flush=True)
        assert r.max() <= TOL + 2.0 ** -8
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
    assert r.max() <= TOL + 2.0 ** -8
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
    """bf16 output: the GEMM bar plus one bf16 rounding (2^-8 relative)."""
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
    assert r.max() <= TOL + 2.0 ** -8


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
    ([300, 0, 513, 129, 64], 520, 768, None),  # 128 x 512 tiles (<= 256 rows per expert on average)
    ([300, 0, 513, 129, 64], 520, 512, 260),   # scale boundaries inside 8-column runs
    ([600, 0, 513, 129], 520, 768, None),      # > 256 rows per expert on average: 256- and 128-row tiles
    ([300, 0, 513, 129, 64], 384, 512, None),  # N < 512: 256- and 128-row tiles
    # 128 x 512 tiles whose last 32-row groups are partly empty: 1, 2, 3 and 4
    # groups multiplied, tails of 1, 32, 33, 64, 65, 96, 97, 127 rows
    ([70, 100, 127, 33, 32, 96, 0, 1, 128, 65, 64, 97], 520, 512, None),
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
    ("mxfp8", [300, 0, 513, 129, 64], 520, 2048),  # the persistent 256 x 256 kernel
    ("mxfp8", [300, 0, 513, 129, 64], 520, 768),
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


@pytest.mark.parametrize("case", [
    # tails of 1 .. 128 rows (1, 2, 3 and 4 fragments), 4 steps per tile
    ([70, 100, 127, 33, 32, 96, 0, 1, 128, 65, 64, 97], 520, 512),
    ([400, 0, 513, 129, 64], 1024, 1024),    # experts of several row tiles, 2 column tiles
    ("many", 512, 768),                       # 300 mostly tiny experts: many tiles per workgroup
    ([1], 512, 512),                          # one tile: every other workgroup has none
])
def test_nvfp4_persistent_bf16(case):
    """The persistent NVFP4 kernel (bf16 output of the 128 x 512 tile path):
    against the oracle at the bar plus one bf16 rounding, and bit for bit
    the nearest-even rounding of the binary32 output (another kernel, the
    same accumulation order and scaling)."""
    sizes, N, K = case
    if sizes == "many":
        sizes = _many_small_groups(300, seed=94)
    G, M = len(sizes), int(sum(sizes))
    assert M <= 256 * G
    x = wl.activations(M, K, seed=95)
    w = wl.normal_bf16((G * N, K), std=0.01, seed=96)
    off = _offsets(sizes)
    qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(x))
    qb, sb, gb = pqm.quantize_nvfp4_per_token(dev_bf16(w), rows_per_scale=N)
    kw = dict(a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb, b_rows_per_scale=N)
    print(f"[gemm] nvfp4 persistent G={G} M={M} N={N} K={K}", flush=True)
    y16 = pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, dev(off), N, K,
                               out_dtype=pqm.OUT_BF16, **kw)
    y32 = pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, dev(off), N, K,
                               out_dtype=pqm.OUT_FP32, **kw)
    torch.cuda.synchronize()
    got = host_u16(y16)
    assert_bytes_equal(got, _rne_bf16_bits(host(y32)), "bf16 vs RNE(binary32)")
    ra, rsa, rga = oracle.quantize_nvfp4(x)
    rb, rsb, rgb = oracle.quantize_nvfp4(w, rows_per_group=N)
    want = oracle.grouped_gemm(oracle.decode_nvfp4(ra, rsa, rga),
                               oracle.decode_nvfp4(rb, rsb, rgb, N).reshape(G, N, K), off)
    r = rel_l2_rows(oracle.bf16_to_f64(got), want)
    print(f"[gemm] nvfp4 persistent: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL + 2.0 ** -8, (float(r.max()), int(r.argmax()))


@pytest.mark.parametrize("case", [
    # tails of 1 .. 128 rows (the waves of rows 128..255 idle), 4 steps per tile
    ([70, 100, 127, 33, 32, 96, 0, 1, 128, 65, 64, 97], 520, 512),
    ([400, 0, 513, 129, 64], 1024, 640),     # several row tiles, 4 column tiles, 5 steps
    ("many", 256, 512),                       # 600 mostly tiny experts: many tiles per workgroup
    ([1], 264, 1024),                         # one row, two column tiles (the second 8 wide)
])
def test_mxfp8_persistent_bf16(case):
    """The persistent MXFP8 kernel's bf16 epilogue (pairs packed, then traded
    between the half-waves and transposed within quads): against the oracle
    at the bar plus one bf16 rounding, and bit for bit the nearest-even
    rounding of the same kernel's binary32 output."""
    sizes, N, K = case
    if sizes == "many":
        sizes = _many_small_groups(600, seed=97)
    G, M = len(sizes), int(sum(sizes))
    x = wl.activations(M, K, seed=98)
    w = wl.normal_bf16((G * N, K), std=0.02, seed=99)
    off = _offsets(sizes)
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(x), colwise=False)
    qb, sb, _, _ = pqm.quantize_mxfp8(dev_bf16(w), colwise=False)
    print(f"[gemm] mxfp8 persistent G={G} M={M} N={N} K={K}", flush=True)
    y16 = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, dev(off), N, K,
                               a_scale=sa, b_scale=sb, out_dtype=pqm.OUT_BF16)
    y32 = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, dev(off), N, K,
                               a_scale=sa, b_scale=sb, out_dtype=pqm.OUT_FP32)
    torch.cuda.synchronize()
    got = host_u16(y16)
    assert_bytes_equal(got, _rne_bf16_bits(host(y32)), "bf16 vs RNE(binary32)")
    ra, rsa = oracle.quantize_mxfp8_rowwise(x)
    rb, rsb = oracle.quantize_mxfp8_rowwise(w)
    want = oracle.grouped_gemm(oracle.decode_mxfp8(ra, rsa),
                               oracle.decode_mxfp8(rb, rsb).reshape(G, N, K), off)
    r = rel_l2_rows(oracle.bf16_to_f64(got), want)
    print(f"[gemm] mxfp8 persistent: max row rel-L2 {r.max():.3e}", flush=True)
    assert r.max() <= TOL + 2.0 ** -8, (float(r.max()), int(r.argmax()))


# ------------------------------------------------- degenerate and large-G

_SENTINEL = 0x7F


@pytest.mark.parametrize("fmt,kind,N", [
    (pqm.FMT_MXFP8, pqm.GEMM_FPROP, 520), (pqm.FMT_MXFP8, pqm.GEMM_DGRAD, 520),
    (pqm.FMT_NVFP4, pqm.GEMM_FPROP, 520), (pqm.FMT_NVFP4, pqm.GEMM_FPROP, 384),
    (pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, 512), (pqm.FMT_BF16, pqm.GEMM_FPROP, 520),
    (pqm.FMT_BF16, pqm.GEMM_DGRAD, 520)])
@pytest.mark.parametrize("out_dtype", [pqm.OUT_FP32, pqm.OUT_BF16])
def test_empty_contraction_writes_zero_rows(fmt, kind, N, out_dtype):
    """K = 0: the sum over an empty contraction is 0 for every routed row
    (rows 0 .. offsets[G]-1), rows past offsets[G] are left untouched, and
    no operand is read (the operands are empty)."""
    sizes, M = [3, 0, 700], 710                       # rows 703 .. 709 are not routed
    off = dev(_offsets(sizes))
    dt = torch.float32 if out_dtype == pqm.OUT_FP32 else torch.bfloat16
    out = torch.empty((M, N), dtype=dt, device="cuda")
    out.view(torch.uint8).fill_(_SENTINEL)
    a = torch.empty((M, 0), dtype=torch.bfloat16 if fmt == pqm.FMT_BF16 else torch.uint8,
                    device="cuda")
    b = torch.empty((len(sizes) * N, 0), dtype=a.dtype, device="cuda")
    print(f"[gemm] K=0 fmt={fmt} kind={kind} N={N} out={out_dtype}", flush=True)
    pqm.moe_grouped_gemm(fmt, kind, a, b, off, N, 0, b_rows_per_scale=N,
                         out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    raw = host(out.view(torch.uint8)).reshape(M, -1)
    assert not raw[:703].any()
    assert (raw[703:] == _SENTINEL).all()


def _many_small_groups(G, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    sizes = rng.choice([0, 0, 1, 2, 5, 33], size=G).tolist()
    sizes[G // 2] = 300                                # one expert with several row tiles
    return sizes


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_more_than_512_groups(fmt):
    """About 600 mostly empty or tiny experts: the tile lookup's general
    path (more groups than one round of offset loads covers)."""
    sizes = _many_small_groups(600, seed=91)
    if fmt == "mxfp8":
        y, want = _mxfp8_case(sizes, 256, 256, seed=92)
    else:
        y, want = _nvfp4_case(sizes, 512, 256, seed=93)
    check_rows(host(y), want, f"{fmt} G=600 ({sum(sizes)} rows)")


# ------------------------------------------------------------ determinism

def _det_cases():
    sizes = [300, 0, 513, 129, 64]
    return [("mxfp8", 1536, 2048), ("mxfp8", 2048, 768), ("mxfp8_dgrad", 768, 2048),
            ("mxfp8_wgrad", 512, 768), ("nvfp4", 1024, 1024), ("nvfp4", 384, 512),
            ("bf16", 520, 384), ("bf16_dgrad", 520, 384), ("bf16_wgrad", 520, 384),
            ("fp8b", 512, 1024)], sizes


@pytest.mark.parametrize("case", _det_cases()[0], ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}")
def test_grouped_gemm_is_deterministic(case):
    """Two calls on the same operands give bitwise identical outputs (fixed
    reduction order, no split-K atomics: the deterministic mode of [MT]
    4.5), for every kernel family the dispatcher picks."""
    name, N, K = case
    sizes = _det_cases()[1]
    G, M = len(sizes), sum(sizes)
    pad = name == "mxfp8_wgrad"           # column-wise copies: 32-row expert blocks
    off = dev(_offsets([-(-s // 32) * 32 for s in sizes] if pad else sizes))
    Mp = int(host(off)[-1])
    x = dev_bf16(wl.activations(max(M, Mp), max(K, N), seed=95))
    w = dev_bf16(wl.normal_bf16((G * max(N, K), max(K, N)), std=0.02, seed=96))
    if name == "mxfp8":
        qa, sa, _, _ = pqm.quantize_mxfp8(x[:M, :K].contiguous(), colwise=False)
        qb, sb, _, _ = pqm.quantize_mxfp8(w[:G * N, :K].contiguous(), colwise=False)
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, qb, off, N, K,
                                            a_scale=sa, b_scale=sb, out_dtype=pqm.OUT_BF16)
    elif name == "mxfp8_dgrad":
        qa, sa, _, _ = pqm.quantize_mxfp8(x[:M, :K].contiguous(), colwise=False)
        _, _, qT, sT = pqm.quantize_mxfp8(w[:G * K, :N].contiguous(), rowwise=False)
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_DGRAD, qa, qT, off, N, K,
                                            a_scale=sa, b_scale=sT)
    elif name == "mxfp8_wgrad":
        _, _, aT, asT = pqm.quantize_mxfp8(x[:Mp, :N].contiguous(), rowwise=False)
        _, _, bT, bsT = pqm.quantize_mxfp8(x[:Mp, :K].contiguous() * 0.5, rowwise=False)
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_WGRAD, aT, bT, off, N, K,
                                            a_scale=asT, b_scale=bsT)
    elif name == "nvfp4":
        qa, sa, ga = pqm.quantize_nvfp4_per_token(x[:M, :K].contiguous())
        qb, sb, gb = pqm.quantize_nvfp4_per_token(w[:G * N, :K].contiguous(), rows_per_scale=N)
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, off, N, K,
                                            a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb,
                                            b_rows_per_scale=N, out_dtype=pqm.OUT_BF16)
    elif name == "fp8b":
        qa, sa = pqm.quantize_fp8_block(x[:M, :K].contiguous(), 1)
        qb, sb = pqm.quantize_fp8_block(w[:G * N, :K].contiguous(), 128)
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, qa, qb, off, N, K,
                                            a_outer=sa, b_outer=sb)
    elif name == "bf16":
        a, b = x[:M, :K].contiguous(), w[:G * N, :K].contiguous()
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_FPROP, a, b, off, N, K)
    elif name == "bf16_dgrad":
        a, b = x[:M, :K].contiguous(), w[:G * K, :N].contiguous()
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, a, b, off, N, K)
    else:
        a, b = x[:M, :N].contiguous(), x[:M, :K].contiguous() * 0.5
        call = lambda: pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_WGRAD, a, b, off, N, K)
    print(f"[gemm] determinism {name} N={N} K={K}", flush=True)
    y1 = call()
    y2 = call()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.uint8), y2.view(torch.uint8)), name


# ------------------------------------------- full-size sampled: DeepSeek FC2

def test_nvfp4_deepseek_down_full_sampled():
    """DeepSeek-V3 down projection at full size: 32768 routed rows (half
    uniform, half Zipf over 256 experts) plus the shared expert's 4096 rows,
    N = 7168, K = 2048, weights [257, 7168, 2048] N(0, 0.01) drawn on the
    GPU, one outer scale per expert tensor (b_rows_per_scale = 7168), bf16
    output as in the layer.  Sampled rows of sampled experts against the
    binary64 product (bar + one bf16 rounding)."""
    T, E, k, H, I = 4096, 256, 8, 7168, 2048
    ids = wl.uniform_plus_zipf_routing(T, E, k)
    off_r, _, _ = oracle.route(ids, E)
    off = np.concatenate([off_r, [T * k + T]]).astype(np.int64)
    M = T * k + T
    d = wl.activations(M, I, seed=24)
    gen = torch.Generator(device="cuda").manual_seed(4321)
    w = (torch.randn((E + 1) * H, I, generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    qa, sa, ga = pqm.quantize_nvfp4_per_token(dev_bf16(d))
    qb, sb, gb = pqm.quantize_nvfp4_per_token(w, rows_per_scale=H)
    y = pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, qa, qb, dev(off), H, I,
                             a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb,
                             b_rows_per_scale=H, out_dtype=pqm.OUT_BF16)
    torch.cuda.synchronize()
    yh = oracle.bf16_to_f64(host_u16(y))
    rng = np.random.Generator(np.random.PCG64(25))
    experts = sorted(set(rng.choice(E, 5, replace=False).tolist()) | {0, E - 1, E})
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 4)]))
        we = host_u16(w[e * H:(e + 1) * H])
        ra, rsa, rga = oracle.quantize_nvfp4(d[rows])
        rb, rsb, rgb = oracle.quantize_nvfp4(we, rows_per_group=H)
        want = oracle.decode_nvfp4(ra, rsa, rga) @ oracle.decode_nvfp4(rb, rsb, rgb, H).T
        r = rel_l2_rows(yh[rows], want)
        print(f"[gemm] deepseek fc2 expert {e} ({hi - lo} rows): max row rel-L2 {r.max():.3e}",
              flush=True)
        assert r.max() <= TOL + 2.0 ** -8, (e, float(r.max()))
    del w, qb


# ------------------------------- full-size sampled: Qwen3 BF16 backward

def _q3_bwd_setup():
    T, E, k, H, I = 8192, 128, 8, 2048, 768
    ids = wl.zipf_routing(T, E, k)
    off, _, _ = oracle.route(ids, E)
    M = T * k
    gen = torch.Generator(device="cuda").manual_seed(555)
    rnd = lambda *shape, std=1.0: (torch.randn(*shape, generator=gen, device="cuda")
                                   * std).to(torch.bfloat16)
    return T, E, k, H, I, off, M, rnd


@pytest.mark.parametrize("proj", ["fc2", "fc1"])
def test_bf16_backward_qwen3_full_sampled(proj):
    """The BF16 backward GEMMs at the Qwen3-30B-A3B layer shapes the
    benchmark runs (65536 routed rows, Zipf(1.1) loads, experts up to ~7400
    rows): dgrad (bf16 output) on sampled rows and wgrad (binary32 output)
    on sampled output rows of sampled experts, against binary64 sums."""
    T, E, k, H, I, off, M, rnd = _q3_bwd_setup()
    if proj == "fc2":      # dD = dY W2 (W2 [E, H, I]); dW2 = dY^T D
        Nd, Kd = I, H
    else:                  # dX = dC W1 (W1 [E, 2I, H]); dW1 = dC^T X
        Nd, Kd = H, 2 * I
    dy = rnd(M, Kd)
    w = rnd(E * Kd, Nd, std=0.02)
    xs = rnd(M, Nd)
    offd = dev(off)
    dx = pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, dy, w, offd, Nd, Kd,
                              out_dtype=pqm.OUT_BF16)
    dw = pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_WGRAD, dy, xs, offd, Kd, Nd,
                              out_dtype=pqm.OUT_FP32)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(26))
    sizes = np.diff(off)
    experts = sorted({int(np.argmax(sizes)), int(np.argmin(sizes)), 0, E - 1}
                     | set(rng.choice(E, 3, replace=False).tolist()))
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 4)]))
        we = oracle.bf16_to_f64(host_u16(w[e * Kd:(e + 1) * Kd]))          # [Kd, Nd]
        ri = torch.from_numpy(rows).cuda()
        want = oracle.bf16_to_f64(host_u16(dy[ri])) @ we
        r = rel_l2_rows(oracle.bf16_to_f64(host_u16(dx[ri])), want)
        print(f"[gemm] qwen3 {proj} bf16 dgrad expert {e} ({hi - lo} rows): "
              f"max row rel-L2 {r.max():.3e}", flush=True)
        assert r.max() <= TOL + 2.0 ** -8, (e, float(r.max()))
        outs = np.unique(np.concatenate([[0, Kd - 1], rng.integers(0, Kd, 6)]))
        dyg = oracle.bf16_to_f64(host_u16(dy[lo:hi]))
        xg = oracle.bf16_to_f64(host_u16(xs[lo:hi]))
        want_w = dyg[:, outs].T @ xg                                      # [len(outs), Nd]
        got_w = host(dw[e])[outs]
        check_rows(got_w, want_w, f"qwen3 {proj} bf16 wgrad expert {e} ({hi - lo} rows)")
