"""Guarded outputs: every entry point is called through the C ABI with each
output buffer placed between two guard regions filled with a sentinel byte;
after the call both guards must be unchanged, and where the contract leaves
part of an output unwritten (grouped-GEMM rows from offsets[G] on, routed
GEMM rows of an empty contraction) that part must keep the sentinel too.
Shapes are ragged so that the edge tiles and tail blocks of every kernel
run.  Values are checked elsewhere; this file checks where the kernels
write."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import workloads as wl
from gpu_util import dev, dev_bf16, host, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

GUARD = 4096          # bytes on each side; keeps 256-byte alignment
SENT = 0xA5


class Guarded:
    """A device buffer of `nbytes` between two sentinel-filled guards."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.base = torch.full((GUARD + self.nbytes + GUARD,), SENT, dtype=torch.uint8,
                               device="cuda")

    @property
    def ptr(self):
        return ctypes.c_void_p(self.base.data_ptr() + GUARD)

    def body(self) -> np.ndarray:
        return host(self.base[GUARD:GUARD + self.nbytes])

    def check(self, what: str):
        b = host(self.base)
        head, tail = b[:GUARD], b[GUARD + self.nbytes:]
        assert (head == SENT).all(), f"{what}: wrote before the buffer"
        assert (tail == SENT).all(), f"{what}: wrote past the buffer " \
                                     f"(first at +{int(np.argmax(tail != SENT))})"


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _run(code, what, *bufs):
    assert code == 0, f"{what}: status {code}"
    torch.cuda.synchronize()
    for i, b in enumerate(bufs):
        b.check(f"{what} output {i}")


def test_quantizers_stay_inside_outputs():
    L = pqm.lib()
    R, C = 96, 352                                     # a 96-column edge tile
    x = dev_bf16(wl.activations(R, C, seed=1))
    q, s, qT, sT = Guarded(R * C), Guarded(R * C // 32), Guarded(R * C), Guarded(R * C // 32)
    print("[canary] mxfp8", flush=True)
    _run(L.pqm_quantize_mxfp8(_p(x), R, C, C, q.ptr, s.ptr, qT.ptr, sT.ptr, _stream()),
         "mxfp8", q, s, qT, sT)
    for rps, R2, C2 in ((1, 37, 272), (32, 96, 272), (1, 5, 16)):
        x = dev_bf16(wl.activations(R2, C2, seed=2))
        q, sb, sg = Guarded(R2 * C2 // 2), Guarded(R2 * C2 // 16), Guarded(4 * (R2 // rps))
        nws = L.pqm_quantize_nvfp4_workspace(R2, C2, rps)
        ws = Guarded(max(nws, 4))
        print(f"[canary] nvfp4 rps={rps} {R2}x{C2}", flush=True)
        _run(L.pqm_quantize_nvfp4_per_token(_p(x), R2, C2, C2, rps, q.ptr, sb.ptr, sg.ptr,
                                            ws.ptr, nws, _stream()), "nvfp4", q, sb, sg, ws)
    for br, R2, C2 in ((1, 37, 384), (128, 256, 384)):
        x = dev_bf16(wl.activations(R2, C2, seed=3))
        q, s = Guarded(R2 * C2), Guarded(4 * (R2 // br) * (C2 // 128))
        print(f"[canary] fp8 block {br}", flush=True)
        _run(L.pqm_quantize_fp8_block(_p(x), R2, C2, C2, br, q.ptr, s.ptr, _stream()),
             "fp8 block", q, s)


def test_dequantize_stays_inside_output():
    L = pqm.lib()
    R, C = 37, 288
    x = dev_bf16(wl.activations(R, C, seed=4))
    q, s, _, _ = pqm.quantize_mxfp8(x, colwise=False)
    y = Guarded(R * C * 2)
    print("[canary] dequant mxfp8", flush=True)
    _run(L.pqm_dequantize(pqm.FMT_MXFP8, _p(q), _p(s), None, R, C, 1, y.ptr, _stream()),
         "dequant mxfp8", y)
    nq, nsb, nsg = pqm.quantize_nvfp4_per_token(x)
    y = Guarded(R * C * 2)
    print("[canary] dequant nvfp4", flush=True)
    _run(L.pqm_dequantize(pqm.FMT_NVFP4, _p(nq), _p(nsb), _p(nsg), R, C, 1, y.ptr, _stream()),
         "dequant nvfp4", y)


def _gemm_operands(fmt, kind, sizes, M, N, K):
    G = len(sizes)
    x = dev_bf16(wl.activations(M, max(N, K), seed=5))
    w = dev_bf16(wl.normal_bf16((G * max(N, K), max(N, K)), std=0.02, seed=6))
    none = dict(a_scale=None, a_outer=None, b_scale=None, b_outer=None)
    if fmt == pqm.FMT_MXFP8 and kind == pqm.GEMM_FPROP:
        qa, sa, _, _ = pqm.quantize_mxfp8(x[:, :K].contiguous(), colwise=False)
        qb, sb, _, _ = pqm.quantize_mxfp8(w[:G * N, :K].contiguous(), colwise=False)
        return qa, qb, dict(none, a_scale=sa, b_scale=sb)
    if fmt == pqm.FMT_MXFP8 and kind == pqm.GEMM_DGRAD:
        qa, sa, _, _ = pqm.quantize_mxfp8(x[:, :K].contiguous(), colwise=False)
        _, _, qT, sT = pqm.quantize_mxfp8(w[:G * K, :N].contiguous(), rowwise=False)
        return qa, qT, dict(none, a_scale=sa, b_scale=sT)
    if fmt == pqm.FMT_MXFP8:                           # WGRAD: column-wise copies
        _, _, aT, asT = pqm.quantize_mxfp8(x[:, :N].contiguous(), rowwise=False)
        _, _, bT, bsT = pqm.quantize_mxfp8(x[:, :K].contiguous(), rowwise=False)
        return aT, bT, dict(none, a_scale=asT, b_scale=bsT)
    if fmt == pqm.FMT_NVFP4:
        qa, sa, ga = pqm.quantize_nvfp4_per_token(x[:, :K].contiguous())
        qb, sb, gb = pqm.quantize_nvfp4_per_token(w[:G * N, :K].contiguous(), rows_per_scale=N)
        return qa, qb, dict(a_scale=sa, a_outer=ga, b_scale=sb, b_outer=gb)
    if fmt == pqm.FMT_FP8_BLOCK:
        qa, sa = pqm.quantize_fp8_block(x[:, :K].contiguous(), 1)
        qb, sb = pqm.quantize_fp8_block(w[:G * N, :K].contiguous(), 128)
        return qa, qb, dict(none, a_outer=sa, b_outer=sb)
    if kind == pqm.GEMM_FPROP:
        return x[:, :K].contiguous(), w[:G * N, :K].contiguous(), none
    if kind == pqm.GEMM_DGRAD:
        return x[:, :K].contiguous(), w[:G * K, :N].contiguous(), none
    return x[:, :N].contiguous(), x[:, :K].contiguous(), none


@pytest.mark.parametrize("fmt,kind,N,K", [
    (pqm.FMT_MXFP8, pqm.GEMM_FPROP, 520, 2048), (pqm.FMT_MXFP8, pqm.GEMM_FPROP, 520, 768),
    (pqm.FMT_MXFP8, pqm.GEMM_FPROP, 200, 320), (pqm.FMT_MXFP8, pqm.GEMM_DGRAD, 544, 384),
    (pqm.FMT_MXFP8, pqm.GEMM_WGRAD, 544, 288), (pqm.FMT_NVFP4, pqm.GEMM_FPROP, 1040, 512),
    (pqm.FMT_NVFP4, pqm.GEMM_FPROP, 384, 512), (pqm.FMT_NVFP4, pqm.GEMM_FPROP, 200, 336),
    (pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, 384, 256), (pqm.FMT_BF16, pqm.GEMM_FPROP, 520, 384),
    (pqm.FMT_BF16, pqm.GEMM_DGRAD, 520, 384), (pqm.FMT_BF16, pqm.GEMM_WGRAD, 520, 384),
    (pqm.FMT_BF16, pqm.GEMM_FPROP, 200, 72)])
@pytest.mark.parametrize("out_dtype", [pqm.OUT_BF16, pqm.OUT_FP32])
def test_grouped_gemm_stays_inside_output(fmt, kind, N, K, out_dtype):
    """Rows offsets[G] .. M_total-1 (not routed) and the guards keep the
    sentinel; WGRAD writes exactly G x N x K values."""
    wgrad = kind == pqm.GEMM_WGRAD
    sizes = [32, 0, 320, 96] if (wgrad and fmt == pqm.FMT_MXFP8) else [37, 0, 300, 129]
    M = sum(sizes) + (0 if wgrad else 19)             # 19 rows past offsets[G]
    G = len(sizes)
    a, b, kw = _gemm_operands(fmt, kind, sizes, M, N, K)
    off = dev(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64))
    es = 4 if out_dtype == pqm.OUT_FP32 else 2
    out = Guarded((G * N * K if wgrad else M * N) * es)
    print(f"[canary] gemm fmt={fmt} kind={kind} N={N} K={K} out={out_dtype}", flush=True)
    L = pqm.lib()
    code = L.pqm_moe_grouped_gemm(fmt, kind, _p(a), *(None if kw[n] is None else _p(kw[n])
                                                      for n in ("a_scale", "a_outer")),
                                  _p(b), *(None if kw[n] is None else _p(kw[n])
                                           for n in ("b_scale", "b_outer")),
                                  N, None, _p(off), G, M, N, K, out.ptr, out_dtype, None, 0,
                                  _stream())
    _run(code, "gemm", out)
    if not wgrad:
        body = out.body().reshape(M, -1)
        assert (body[sum(sizes):] == SENT).all(), "wrote rows past offsets[G]"


def test_glue_stays_inside_outputs():
    L = pqm.lib()
    T, E, k = 301, 20, 3
    rng = np.random.Generator(np.random.PCG64(7))
    ids = dev(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32))
    for sh in (0, 1):
        M = T * k + sh * T
        off, src, tok = Guarded(8 * (E + 1 + sh)), Guarded(4 * M), Guarded(4 * M)
        slot = Guarded(4 * T * k)
        nws = L.pqm_moe_route_workspace(T, k, E)
        ws = Guarded(max(nws, 8))
        print(f"[canary] route shared={sh}", flush=True)
        _run(L.pqm_moe_route(_p(ids), T, k, E, sh, off.ptr, src.ptr, tok.ptr, slot.ptr, ws.ptr,
                             nws, _stream()), "route", off, src, tok, slot, ws)
    offs, srcs, toks, slots = pqm.moe_route(ids, E)
    # gather: 48-byte rows
    x = dev(rng.integers(0, 255, (T, 48), dtype=np.uint8))
    n = T * k
    g = Guarded(n * 48)
    print("[canary] gather", flush=True)
    _run(L.pqm_moe_gather_rows(_p(x), T, 48, _p(toks), n, 1, g.ptr, _stream()), "gather", g)
    # per-expert padding
    rows = pqm.pad_rows_bound(n, E)
    po, pout = Guarded(8 * (E + 1)), Guarded(rows * 48)
    xs = dev(rng.integers(0, 255, (n, 48), dtype=np.uint8))
    print("[canary] pad rows", flush=True)
    _run(L.pqm_moe_pad_rows(_p(xs), n, 48, _p(offs), E, 32, po.ptr, pout.ptr, rows, _stream()),
         "pad rows", po, pout)
    # SwiGLU x prob, unfused and fused with the MXFP8 encoding of D
    I = 96
    c = dev_bf16(wl.normal_bf16((n, 2 * I), std=2.0, seed=8))
    prob = dev(rng.random(n).astype(np.float32))
    d = Guarded(n * I * 2)
    print("[canary] swiglu", flush=True)
    _run(L.pqm_swiglu_prob(_p(c), _p(prob), _p(srcs), n, I, d.ptr, _stream()), "swiglu", d)
    d, q, s = Guarded(n * I * 2), Guarded(n * I), Guarded(n * I // 32)
    print("[canary] swiglu + mxfp8", flush=True)
    _run(L.pqm_swiglu_prob_quantize_mxfp8(_p(c), _p(prob), _p(srcs), n, I, d.ptr, q.ptr, s.ptr,
                                          _stream()), "swiglu+mxfp8", d, q, s)
    I2 = 272
    c2 = dev_bf16(wl.normal_bf16((n, 2 * I2), std=2.0, seed=14))
    d, q, sbk, sgo = Guarded(n * I2 * 2), Guarded(n * I2 // 2), Guarded(n * I2 // 16), Guarded(4 * n)
    print("[canary] swiglu + nvfp4", flush=True)
    _run(L.pqm_swiglu_prob_quantize_nvfp4(_p(c2), _p(prob), _p(srcs), n, I2, d.ptr, q.ptr, sbk.ptr,
                                          sgo.ptr, _stream()), "swiglu+nvfp4", d, q, sbk, sgo)
    # combine, with and without a shared-expert term
    y = dev_bf16(wl.normal_bf16((n, 136), seed=9))
    shared = dev_bf16(wl.normal_bf16((T, 136), seed=10))
    for sh_t in (None, shared):
        o = Guarded(T * 136 * 2)
        print(f"[canary] combine shared={sh_t is not None}", flush=True)
        _run(L.pqm_moe_combine(_p(y), _p(slots), None if sh_t is None else _p(sh_t), T, k, 136,
                               o.ptr, _stream()), "combine", o)


def test_fused_gate_up_epilogue_stays_inside_outputs():
    L = pqm.lib()
    sizes, I, K = [300, 0, 513, 129, 64], 256, 256
    G, M = len(sizes), sum(sizes)
    off = dev(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64))
    qa, sa, _, _ = pqm.quantize_mxfp8(dev_bf16(wl.activations(M, K, seed=11)), colwise=False)
    qw, sw, _, _ = pqm.quantize_mxfp8(dev_bf16(wl.normal_bf16((G * 2 * I, K), 0.05, 12)),
                                      colwise=False)
    prob = dev(np.random.Generator(np.random.PCG64(13)).random(M).astype(np.float32))
    q, s = Guarded(M * I), Guarded(M * I // 32)
    print("[canary] gate_up + swiglu + mxfp8 epilogue", flush=True)
    _run(L.pqm_moe_gemm_swiglu_quantize_mxfp8(_p(qa), _p(sa), _p(qw), _p(sw), _p(off), G, M, I,
                                              K, _p(prob), None, q.ptr, s.ptr, _stream()),
         "fused epilogue", q, s)
