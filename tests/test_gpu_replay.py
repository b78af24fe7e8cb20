"""Stage-wise reference replay of the MoE glue at the full layer shapes.

Each glue stage is recomputed by the oracle from the GPU's own input to that
stage (not from the raw layer inputs), so the comparison isolates the stage
("miniTE technical report", 4.4: dump intermediate tensors and replay them
through the reference; 6.2.1: quantization, GEMM and glue verified
separately):

* SwiGLU x prob: D = bf16(silu(gate) up prob) replayed in binary64 from the
  GPU's bf16 C.  The GPU computes in binary32 with the hardware exponential
  and reciprocal, so an element may differ by one bf16 ulp where the exact
  value lies within about 2^-20 relative of a rounding boundary; the bar is
  <= 1 ulp everywhere and >= 99.9 % of elements identical.
* The FC2 operand: the GPU's encoding of its own D equals the oracle's
  encoding of that D byte for byte (MXFP8 row-wise for the Qwen3 layer,
  per-token NVFP4 for the DeepSeek layer); the gate_up GEMM with the fused
  epilogue gives the same bytes as the unfused chain, and wherever a 32-block
  of the GPU's D equals the oracle's replayed D, its bytes equal the
  oracle's encoding of the replayed D.
* Combine: out[t] = bf16(sum_j Y[slot(t, j)] (+ shared)) replayed in binary64
  from the GPU's bf16 Y; the GPU sums in binary32 in j order, so <= 1 ulp,
  and >= 99.9 % identical.

Layer inputs follow the layer benchmark: Qwen3-30B-A3B (8192 tokens, top-8 of
128 experts, Zipf(1.1), H = 2048, I = 768, MXFP8) and DeepSeek-V3 (4096
tokens, top-8 of 256 routed experts half uniform / half Zipf(1.1) plus the
shared expert, H = 7168, I = 2048, NVFP4, gate/up jointly scaled); weights
are drawn on the GPU from a seeded generator."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import moe_layer
from precision_quantization_moe_amd import workloads as wl
from gpu_util import (assert_bytes_equal, dev, dev_bf16, gpu_normal_bf16, host, host_u16,
                      requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


def ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two bf16 bit patterns (+0 == -0)."""
    def key(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(key(a_bits) - key(b_bits))


@pytest.fixture(scope="module")
def qwen3():
    T, E, k, H, I = 8192, 128, 8, 2048, 768
    print("[replay] qwen3 layer", flush=True)
    x = dev_bf16(wl.activations(T, H, seed=0))
    ids = dev(wl.zipf_routing(T, E, k))
    prob = dev(wl.router_probs(T, k).reshape(-1))
    w1 = gpu_normal_bf16(E * 2 * I, H, 0.02, seed=301)
    w2 = gpu_normal_bf16(E * H, I, 0.02, seed=302)
    wq = moe_layer.quantize_expert_weights_mxfp8(w1, w2)
    del w1, w2
    g = moe_layer.mxfp8_moe_forward(x, ids, prob, *wq, E, I, keep_intermediates=True)
    f = moe_layer.mxfp8_moe_forward(x, ids, prob, *wq, E, I, keep_intermediates=False)
    torch.cuda.synchronize()
    return dict(T=T, k=k, I=I, prob=host(prob), g=g, f=f)


@pytest.fixture(scope="module")
def deepseek():
    T, E, k, H, I = 4096, 256, 8, 7168, 2048
    print("[replay] deepseek layer", flush=True)
    x = dev_bf16(wl.activations(T, H, seed=0))
    ids = dev(wl.uniform_plus_zipf_routing(T, E, k))
    prob = wl.router_probs(T, k).reshape(-1)
    prob_all = torch.cat([dev(prob), torch.ones(T, dtype=torch.float32, device="cuda")])
    w1 = gpu_normal_bf16((E + 1) * 2 * I, H, 0.01, seed=303)
    w2 = gpu_normal_bf16((E + 1) * H, I, 0.01, seed=304)
    wq = moe_layer.quantize_expert_weights_nvfp4(w1, w2, I, H)
    del w1, w2
    g = moe_layer.nvfp4_moe_forward(x, ids, prob_all, *wq, E, I)
    torch.cuda.synchronize()
    return dict(T=T, k=k, I=I, prob=host(prob_all), g=g)


def _sample_rows(M, n, seed, extra=()):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, n), list(extra)])
                     .astype(np.int64))


def _replay_d(layer, rows):
    g = layer["g"]
    ri = torch.from_numpy(rows).cuda()
    c = host_u16(g["c"][ri])
    p = layer["prob"][host(g["src"][ri])]
    want = oracle.f64_to_bf16(oracle.swiglu_prob(oracle.bf16_to_f64(c), p))
    return host_u16(g["d"][ri]), want


def _check_d(got, want, what):
    u = ulp_diff(got, want)
    same = float((u == 0).mean())
    print(f"[replay] {what}: max {int(u.max())} ulp, {same:.6f} identical", flush=True)
    assert u.max() <= 1, what
    assert same >= 0.999, what


def test_swiglu_replay_qwen3(qwen3):
    M = qwen3["T"] * qwen3["k"]
    rows = _sample_rows(M, 4096, seed=1)
    got, want = _replay_d(qwen3, rows)
    _check_d(got, want, "qwen3 D = SwiGLU(C) x prob")


def test_swiglu_replay_deepseek(deepseek):
    T, k = deepseek["T"], deepseek["k"]
    rows = _sample_rows(T * k + T, 2048, seed=2, extra=T * k + np.arange(0, T, 97))
    got, want = _replay_d(deepseek, rows)
    _check_d(got, want, "deepseek D = SwiGLU(C) x prob (shared rows included)")


def test_fc2_operand_replay_qwen3(qwen3):
    """MXFP8 bytes of the FC2 operand: the GPU's encoding of its own D is
    the oracle's; the fused gate_up epilogue (C and D never stored) gives
    the same bytes as the unfused chain on every row; 32-blocks whose D
    matches the replayed D carry the oracle's bytes of the replayed D."""
    g, f = qwen3["g"], qwen3["f"]
    assert_bytes_equal(host(f["qd"]), host(g["qd"]), "fused epilogue q vs unfused")
    assert_bytes_equal(host(f["sd"]), host(g["sd"]), "fused epilogue s vs unfused")
    M = qwen3["T"] * qwen3["k"]
    rows = _sample_rows(M, 4096, seed=3)
    got_d, want_d = _replay_d(qwen3, rows)
    ri = torch.from_numpy(rows).cuda()
    q, s = host(g["qd"][ri]), host(g["sd"][ri])
    rq, rs = oracle.quantize_mxfp8_rowwise(got_d)
    assert_bytes_equal(q, rq, "FC2 operand q (oracle encoding of the GPU's D)")
    assert_bytes_equal(s, rs, "FC2 operand s")
    wq, ws = oracle.quantize_mxfp8_rowwise(want_d)
    agree = (got_d == want_d).reshape(rows.size, -1, 32).all(axis=2)      # per 32-block
    print(f"[replay] qwen3 FC2 operand: {agree.mean():.6f} of blocks with D identical", flush=True)
    assert agree.mean() >= 0.99
    assert np.array_equal(s[agree], ws[agree])
    qb, wqb = q.reshape(rows.size, -1, 32), wq.reshape(rows.size, -1, 32)
    assert np.array_equal(qb[agree], wqb[agree])


def test_fc2_operand_replay_deepseek(deepseek):
    """Per-token NVFP4 of the GPU's D equals the oracle's on sampled rows
    (routed and shared), and agrees with the oracle's NVFP4 of the replayed
    D wherever the whole row of D matches."""
    T, k = deepseek["T"], deepseek["k"]
    g = deepseek["g"]
    rows = _sample_rows(T * k + T, 1024, seed=4, extra=T * k + np.arange(0, T, 211))
    got_d, want_d = _replay_d(deepseek, rows)
    ri = torch.from_numpy(rows).cuda()
    q, sb, sg = host(g["qd"][ri]), host(g["sbd"][ri]), host(g["sgd"][ri])
    rq, rsb, rsg = oracle.quantize_nvfp4(got_d)
    assert_bytes_equal(sg.view(np.uint32), rsg.view(np.uint32), "FC2 operand s_g")
    assert_bytes_equal(sb, rsb, "FC2 operand s_b")
    assert_bytes_equal(q, rq, "FC2 operand q")
    same = (got_d == want_d).all(axis=1)
    print(f"[replay] deepseek FC2 operand: {same.mean():.4f} of rows with D identical", flush=True)
    assert same.any()
    wq, wsb, wsg = oracle.quantize_nvfp4(want_d[same])
    assert np.array_equal(q[same], wq) and np.array_equal(sb[same], wsb)
    assert np.array_equal(sg[same].view(np.uint32), wsg.view(np.uint32))


def _check_combine(layer, shared):
    g = layer["g"]
    T, k = layer["T"], layer["k"]
    y = oracle.bf16_to_f64(host_u16(g["y"]))
    slot = host(g["slot"]).astype(np.int64)
    want = oracle.f64_to_bf16(oracle.combine(y[:T * k], slot, y[T * k:] if shared else None))
    got = host_u16(g["out"])
    u = ulp_diff(got, want)
    same = float((u == 0).mean())
    print(f"[replay] combine ({'with' if shared else 'no'} shared): max {int(u.max())} ulp, "
          f"{same:.6f} identical", flush=True)
    assert u.max() <= 1
    assert same >= 0.999


def test_combine_replay_qwen3(qwen3):
    _check_combine(qwen3, shared=False)


def test_combine_replay_deepseek(deepseek):
    _check_combine(deepseek, shared=True)
