"""Benchmark of the block-scaled quantizer + MoE grouped-GEMM hot path on one
MI355X.

One step is one pass of every hot-path row over one batch of synthetic,
seeded input, with all inputs resident in HBM:

  mxfp8_quant       MXFP8 row-wise + column-wise quantize, 16384 x 2048 bf16
                    activations (Qwen3-30B-A3B hidden size)  <- headline value
  nvfp4_token       per-token NVFP4 quantize of same-shaped activations
  nvfp4_joint_w     joint gate/up NVFP4 quantize, 128 experts' [1536 x 2048]
  q3_wquant         Qwen3-30B-A3B experts: MXFP8 quantize of W1 and W2
  q3_fwd            MXFP8 MoE expert layer forward: 8192 tokens, top-8 of 128
                    experts (Zipf 1.1): route, token quantize, gather,
                    gate_up GEMM with SwiGLU x prob and the FC2 operand's
                    MXFP8 quantize in its epilogue, down GEMM, combine
  q3_gemm           the two MXFP8 grouped GEMMs of q3_fwd alone
  q3_gemm_fp8b      the same two grouped GEMMs in DeepSeek-style block FP8
                    (1x128 activation tiles, 128x128 weight blocks, FP32
                    scales applied around the matrix core); operands
                    quantized outside the step
  q3_dequant        dequantize of the forward operands (dequantized backward)
  q3_bwd            BF16 dgrad + wgrad of both expert GEMMs on them
  q3_bwd_mx         MXFP8 low-precision backward of both expert GEMMs: the
                    two output gradients padded per expert to 32-row blocks
                    and quantized (row-wise + column-wise, one pass each),
                    then dgrad on the weights' column-wise copies and wgrad
                    on the column-wise copies of gradient and saved input
                    (those forward-side copies are made outside the step)
  ds_wquant         DeepSeek-V3 experts (256 routed + 1 shared, hidden 7168,
                    intermediate 2048): NVFP4 weights, gate/up jointly scaled
  ds_fwd            NVFP4 MoE expert layer forward, 4096 tokens top-8 + shared
                    (the weighted SwiGLU and the FC2 operand's per-token
                    NVFP4 quantize in one fused pass)
  ds_gemm           the two NVFP4 grouped GEMMs of ds_fwd alone
  ds_fc2_online     ds_fwd's down projection with online amax compensation:
                    the weighted SwiGLU output (bf16, made once from the
                    layer's gate_up output) encoded tile by tile under each
                    row's running maximum (one pass over the rows), then the
                    FC2 GEMM moving its accumulator to each new outer scale
  ds_reconstruct    bf16 reconstruction of the forward operands (activations
                    and all 257 experts' weights) for the dequantized backward

Not part of a step unless named in --rows:
  q3_gemm_uniform   q3_gemm's two MXFP8 GEMMs with uniform routing (every
                    expert 512 rows on average): the balanced-load reference
  hbm_copy          torch's device copy of 512 MiB: a plain copy kernel of
                    known size whose FETCH_SIZE / WRITE_SIZE counter readings
                    calibrate the counters read on the other kernels

The two activation-quantizer rows launch their kernel --reps times per step,
rotating over --sets input/output buffer sets (about 1 GB in all, well above
the 256 MB Infinity Cache) so that their rate is HBM's; their time is per
launch.  Each row is timed with HIP events on the stream its kernels run on
(torch's current stream); `value` is the MXFP8 quantizer's HBM rate
(algorithmic bytes / kernel time).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows a,b,...]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense MFMA FP8
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA BF16 / FP16

ALL_ROWS = ["mxfp8_quant", "nvfp4_token", "nvfp4_joint_w", "q3_wquant", "q3_fwd", "q3_gemm",
            "q3_gemm_fp8b",
            "q3_dequant", "q3_bwd", "q3_bwd_mx", "ds_wquant", "ds_fwd", "ds_gemm", "ds_fc2_online",
            "ds_reconstruct"]
EXTRA_ROWS = ["q3_gemm_uniform", "hbm_copy"]
COPY_BYTES = 512 << 20
REPEAT_ROWS = ("mxfp8_quant", "nvfp4_token")

# HBM bytes of one launch of the headline kernel, from two rocprofv3 counter
# runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
#   bench.py --rows mxfp8_quant,nvfp4_token,hbm_copy --steps 3 --warmup 1 --sets 3
# each scaled by what the same counter reads on the 512 MiB device copy of the
# hbm_copy row (FETCH_SIZE reads 0.5x the copied bytes, WRITE_SIZE 1.0x).
# The figure belongs to the kernel source it was taken on: it is reported only
# while the files hash to the values below.
TRAFFIC = {
    "kernel": "k_quantize_mxfp8<true,true,true,1>",
    "fetch_kib": 32803.5, "fetch_scale": 2.0,
    "write_kib": 74808.1, "write_scale": 1.0,
    "sources": {
        "precision_quantization_moe_amd/csrc/quantize_mxfp8.hip": "a727c5bb5e20ea240bf590cd8cc6e5b4291706f59a371d3780213255d131a389",
        "precision_quantization_moe_amd/csrc/pqm_device.hpp": "1fa07f9f6ad3d957cca7456e309273ff26fe2f29a742feb2ed85e3343dd18317",
    },
}


def measured_traffic():
    import hashlib
    for rel, want in TRAFFIC["sources"].items():
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != want:
                return None
    return (TRAFFIC["fetch_kib"] * TRAFFIC["fetch_scale"]
            + TRAFFIC["write_kib"] * TRAFFIC["write_scale"]) * 1024.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--sets", type=int, default=8, help="rotating quantizer input sets")
    p.add_argument("--reps", type=int, default=10,
                   help="launches per step of the activation-quantizer rows")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--rows", default="all", help="comma list of rows (default all)")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU runs are "
                          "not part of this build", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import precision_quantization_moe_amd as pqm
    from precision_quantization_moe_amd import moe_layer
    from precision_quantization_moe_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs an MI355X GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    order = ALL_ROWS + EXTRA_ROWS
    sel = ALL_ROWS if args.rows == "all" else [r for r in order if r in args.rows.split(",")]
    need = lambda *names: any(n in sel for n in names)

    def to_dev(a: np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(dev)

    def gpu_normal(rows, cols, std, seed, chunk_rows=1 << 16):
        g = torch.Generator(device=dev).manual_seed(seed)
        out = torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)
        for r in range(0, rows, chunk_rows):
            n = min(chunk_rows, rows - r)
            out[r:r + n] = (torch.randn(n, cols, generator=g, device=dev) * std).to(torch.bfloat16)
        return out

    # ------------------------------------------------------------ inputs
    T2, H = 16384, 2048
    log("generating inputs")
    st = {}
    if need("mxfp8_quant", "nvfp4_token"):
        st["sets"] = [to_dev(wl.activations(T2, H, seed=100 + i)) for i in range(args.sets)]
    E, I2 = 128, 1536
    if need("nvfp4_joint_w"):
        st["w_joint"] = to_dev(wl.expert_weights(E, I2, H, 0.02, tag=7).reshape(E * I2, H))
    # Qwen3-30B-A3B expert layer
    T4, K4, I4 = 8192, 8, 768
    M4 = T4 * K4
    if need("q3_wquant", "q3_fwd", "q3_gemm", "q3_gemm_fp8b", "q3_dequant", "q3_bwd", "q3_bwd_mx",
            "q3_gemm_uniform"):
        st["x4"] = to_dev(wl.activations(T4, H, seed=4))
        st["ids4"] = torch.from_numpy(wl.zipf_routing(T4, E, K4)).to(dev)
        st["prob4"] = torch.from_numpy(wl.router_probs(T4, K4).reshape(-1)).to(dev)
        st["W1"] = to_dev(wl.expert_weights(E, 2 * I4, H, 0.02).reshape(E * 2 * I4, H))
        st["W2"] = to_dev(wl.expert_weights(E, H, I4, 0.02, tag=1).reshape(E * H, I4))
        st["dY"] = to_dev(wl.output_grad(M4, H))
        st["dC"] = to_dev(wl.output_grad(M4, 2 * I4, seed=5))
        st["c4"] = torch.empty((M4, 2 * I4), dtype=torch.bfloat16, device=dev)  # q3_gemm's C
    if need("q3_gemm_fp8b"):
        off4, _, tok4, _ = pqm.moe_route(st["ids4"], E)
        xr = pqm.moe_gather_rows(st["x4"], tok4)
        st["fp8b"] = dict(
            off=off4, x=pqm.quantize_fp8_block(xr, 1),
            d=pqm.quantize_fp8_block(to_dev(wl.activations(M4, I4, seed=9)), 1),
            w1=pqm.quantize_fp8_block(st["W1"], 128), w2=pqm.quantize_fp8_block(st["W2"], 128),
            c=torch.empty((M4, 2 * I4), dtype=torch.bfloat16, device=dev),
            y=torch.empty((M4, H), dtype=torch.bfloat16, device=dev))
        del xr
    if need("q3_gemm_uniform"):
        ids_u = torch.from_numpy(wl.uniform_routing(T4, E, K4)).to(dev)
        off_u, _, tok_u, _ = pqm.moe_route(ids_u, E)
        xu = pqm.moe_gather_rows(st["x4"], tok_u)
        st["uni"] = dict(off=off_u, x=pqm.quantize_mxfp8(xu, colwise=False),
                         d=pqm.quantize_mxfp8(to_dev(wl.activations(M4, I4, seed=9)), colwise=False),
                         c=torch.empty((M4, 2 * I4), dtype=torch.bfloat16, device=dev),
                         y=torch.empty((M4, H), dtype=torch.bfloat16, device=dev))
        del xu
    if need("q3_bwd_mx"):
        # forward-side operands of the low-precision backward: the weights'
        # column-wise copies and those of the padded FC1 input X (the
        # routed token rows) and FC2 input D
        off4, _, tok4, _ = pqm.moe_route(st["ids4"], E)
        xr = pqm.moe_gather_rows(st["x4"], tok4)
        st["bwmx"] = dict(
            off=off4, wcol=moe_layer.column_copies_mxfp8(st["W1"], st["W2"]),
            sx=moe_layer.saved_activation_mxfp8(xr, off4),
            sd=moe_layer.saved_activation_mxfp8(to_dev(wl.activations(M4, I4, seed=8)), off4))
        del xr
    # DeepSeek-V3 expert layer (weights drawn on the GPU from a seeded stream)
    T5, K5, E5, H5, I5 = 4096, 8, 256, 7168, 2048
    M5 = T5 * K5 + T5
    if need("ds_wquant", "ds_fwd", "ds_gemm", "ds_fc2_online", "ds_reconstruct"):
        st["x5"] = to_dev(wl.activations(T5, H5, seed=6))
        st["ids5"] = torch.from_numpy(wl.uniform_plus_zipf_routing(T5, E5, K5)).to(dev)
        p5 = torch.from_numpy(wl.router_probs(T5, K5, seed=7).reshape(-1)).to(dev)
        st["prob5"] = torch.cat([p5, torch.ones(T5, dtype=torch.float32, device=dev)])
        st["W1d"] = gpu_normal((E5 + 1) * 2 * I5, H5, 0.01, seed=11)
        st["W2d"] = gpu_normal((E5 + 1) * H5, I5, 0.01, seed=12)
    if need("hbm_copy"):
        st["cp_src"] = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        st["cp_dst"] = torch.empty_like(st["cp_src"])
    torch.cuda.synchronize()
    log("inputs ready")

    # ------------------------------------------------------------- rows
    # outputs of the quantizer rows are allocated once (one per input set),
    # so the timed region holds only the kernels
    if need("mxfp8_quant"):
        st["mx_out"] = [pqm.quantize_mxfp8(x) for x in st["sets"]]
    if need("nvfp4_token"):
        st["nv_out"] = [pqm.quantize_nvfp4_per_token(x) for x in st["sets"]]
    if need("nvfp4_joint_w"):
        st["jw_out"] = pqm.quantize_nvfp4_per_token(st["w_joint"], rows_per_scale=I2)

    nset = args.sets

    def r_mxfp8(s):
        for j in range(args.reps):
            k = (s * args.reps + j) % nset
            pqm.quantize_mxfp8(st["sets"][k], out=st["mx_out"][k])

    def r_nvfp4(s):
        for j in range(args.reps):
            k = (s * args.reps + j) % nset
            pqm.quantize_nvfp4_per_token(st["sets"][k], out=st["nv_out"][k])

    def r_joint(s):
        pqm.quantize_nvfp4_per_token(st["w_joint"], rows_per_scale=I2, out=st["jw_out"])

    def r_q3_wquant(s):
        st["q3w"] = moe_layer.quantize_expert_weights_mxfp8(st["W1"], st["W2"])

    def r_q3_fwd(s):
        st["q3"] = moe_layer.mxfp8_moe_forward(st["x4"], st["ids4"], st["prob4"], *st["q3w"], E,
                                               I4, keep_intermediates=False)

    def r_q3_gemm(s):
        o, (w1q, w1s, w2q, w2s) = st["q3"], st["q3w"]
        pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, o["qa"], w1q, o["off"], 2 * I4, H,
                             a_scale=o["sa"], b_scale=w1s, out_dtype=pqm.OUT_BF16, out=st["c4"])
        pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, o["qd"], w2q, o["off"], H, I4,
                             a_scale=o["sd"], b_scale=w2s, out_dtype=pqm.OUT_BF16, out=o["y"])

    def r_q3_gemm_uniform(s):
        u, (w1q, w1s, w2q, w2s) = st["uni"], st["q3w"]
        pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, u["x"][0], w1q, u["off"], 2 * I4, H,
                             a_scale=u["x"][1], b_scale=w1s, out_dtype=pqm.OUT_BF16, out=u["c"])
        pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, u["d"][0], w2q, u["off"], H, I4,
                             a_scale=u["d"][1], b_scale=w2s, out_dtype=pqm.OUT_BF16, out=u["y"])

    def r_q3_gemm_fp8b(s):
        f = st["fp8b"]
        pqm.moe_grouped_gemm(pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, f["x"][0], f["w1"][0], f["off"],
                             2 * I4, H, a_outer=f["x"][1], b_outer=f["w1"][1],
                             out_dtype=pqm.OUT_BF16, out=f["c"])
        pqm.moe_grouped_gemm(pqm.FMT_FP8_BLOCK, pqm.GEMM_FPROP, f["d"][0], f["w2"][0], f["off"],
                             H, I4, a_outer=f["d"][1], b_outer=f["w2"][1],
                             out_dtype=pqm.OUT_BF16, out=f["y"])

    def r_q3_dequant(s):
        o, (w1q, w1s, w2q, w2s) = st["q3"], st["q3w"]
        prev = st.get("deq", {})
        st["deq"] = dict(w1=pqm.dequantize(pqm.FMT_MXFP8, w1q, w1s, out=prev.get("w1")),
                         w2=pqm.dequantize(pqm.FMT_MXFP8, w2q, w2s, out=prev.get("w2")),
                         a=pqm.dequantize(pqm.FMT_MXFP8, o["qa"], o["sa"], out=prev.get("a")),
                         d=pqm.dequantize(pqm.FMT_MXFP8, o["qd"], o["sd"], out=prev.get("d")))

    def r_q3_bwd(s):
        d, off = st["deq"], st["q3"]["off"]
        # FC2: dD = dY . W2 (W2 [E, H, I], contraction over H); dW2 = dY^T D
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, st["dY"], d["w2"], off, I4, H,
                             out_dtype=pqm.OUT_BF16)
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_WGRAD, st["dY"], d["d"], off, H, I4,
                             out_dtype=pqm.OUT_FP32)
        # FC1: dX = dC . W1 (W1 [E, 2I, H]); dW1 = dC^T A
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, st["dC"], d["w1"], off, H, 2 * I4,
                             out_dtype=pqm.OUT_BF16)
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_WGRAD, st["dC"], d["a"], off, 2 * I4, H,
                             out_dtype=pqm.OUT_FP32)

    def r_q3_bwd_mx(s):
        m = st["bwmx"]
        st["q3_bwd_mx_out"] = moe_layer.mxfp8_expert_backward(st["dY"], st["dC"], m["sx"], m["sd"],
                                                              m["wcol"], m["off"], I4)

    def r_ds_wquant(s):
        st["dsw"] = moe_layer.quantize_expert_weights_nvfp4(st["W1d"], st["W2d"], I5, H5)

    def r_ds_fwd(s):
        st["ds"] = moe_layer.nvfp4_moe_forward(st["x5"], st["ids5"], st["prob5"], *st["dsw"],
                                               E5, I5, keep_intermediates=False)

    def r_ds_gemm(s):
        o, (w1q, w1b, w1g, w2q, w2b, w2g) = st["ds"], st["dsw"]
        pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, o["qa"], w1q, o["off"], 2 * I5, H5,
                             a_scale=o["sba"], a_outer=o["sga"], b_scale=w1b, b_outer=w1g,
                             b_rows_per_scale=2 * I5, out_dtype=pqm.OUT_BF16, out=o["c"])
        pqm.moe_grouped_gemm(pqm.FMT_NVFP4, pqm.GEMM_FPROP, o["qd"], w2q, o["off"], H5, I5,
                             a_scale=o["sbd"], a_outer=o["sgd"], b_scale=w2b, b_outer=w2g,
                             b_rows_per_scale=H5, out_dtype=pqm.OUT_BF16, out=o["y"])

    def r_ds_fc2_online(s):
        o, (w1q, w1b, w1g, w2q, w2b, w2g) = st["ds"], st["dsw"]
        if "p5" not in st:  # made during the warmup steps: the FC2 input, bf16
            st["p5"] = pqm.swiglu_prob(o["c"], st["prob5"], o["src"])
        st["ds_online"] = pqm.moe_fc2_online_nvfp4_split(st["p5"], w2q, w2b, w2g, o["off"], H5,
                                                         w_rows_per_scale=H5)

    def r_ds_reconstruct(s):
        o, (w1q, w1b, w1g, w2q, w2b, w2g) = st["ds"], st["dsw"]
        prev = st.get("dsr", {})
        st["dsr"] = dict(
            a=pqm.dequantize(pqm.FMT_NVFP4, o["qa"], o["sba"], o["sga"], out=prev.get("a")),
            w1=pqm.dequantize(pqm.FMT_NVFP4, w1q, w1b, w1g, rows_per_scale=2 * I5,
                              out=prev.get("w1")),
            w2=pqm.dequantize(pqm.FMT_NVFP4, w2q, w2b, w2g, rows_per_scale=H5,
                              out=prev.get("w2")))

    def r_copy(s):
        st["cp_dst"].copy_(st["cp_src"])

    fns = {"hbm_copy": r_copy, "mxfp8_quant": r_mxfp8, "nvfp4_token": r_nvfp4, "nvfp4_joint_w": r_joint,
           "q3_wquant": r_q3_wquant, "q3_fwd": r_q3_fwd, "q3_gemm": r_q3_gemm,
           "q3_gemm_fp8b": r_q3_gemm_fp8b, "q3_gemm_uniform": r_q3_gemm_uniform,
           "q3_dequant": r_q3_dequant, "q3_bwd": r_q3_bwd, "q3_bwd_mx": r_q3_bwd_mx,
           "ds_wquant": r_ds_wquant,
           "ds_fwd": r_ds_fwd, "ds_gemm": r_ds_gemm, "ds_fc2_online": r_ds_fc2_online,
           "ds_reconstruct": r_ds_reconstruct}
    deps = {"q3_fwd": ["q3_wquant"], "q3_gemm": ["q3_wquant", "q3_fwd"],
            "q3_gemm_uniform": ["q3_wquant"],
            "q3_dequant": ["q3_wquant", "q3_fwd"], "q3_bwd": ["q3_wquant", "q3_fwd", "q3_dequant"],
            "ds_fwd": ["ds_wquant"], "ds_gemm": ["ds_wquant", "ds_fwd"],
            "ds_fc2_online": ["ds_wquant", "ds_fwd"],
            "ds_reconstruct": ["ds_wquant", "ds_fwd"]}
    run = []
    for r in sel:
        for d in deps.get(r, []) + [r]:
            if d not in run:
                run.append(d)
    run = [r for r in order if r in run]

    stream = torch.cuda.current_stream(dev)
    timings = {n: [] for n in run}
    pending = []
    t0 = time.perf_counter()
    for step in range(args.warmup + args.steps):
        if step == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        evs = []
        for n in run:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fns[n](step)
            b.record(stream)
            evs.append((n, a, b))
        if step >= args.warmup:
            pending.append(evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for evs in pending:
        for n, a, b in evs:
            timings[n].append(a.elapsed_time(b) * 1e-3)

    # ------------------------------------------------------ figures
    comp = {}
    R2 = T2 * H
    fl_q3 = 2.0 * M4 * (2 * I4) * H + 2.0 * M4 * H * I4
    fl_ds = 2.0 * M5 * (2 * I5) * H5 + 2.0 * M5 * H5 * I5

    def hbm(c, byt, t):
        c.update(bytes=byt, gbs=byt / t / 1e9, frac_hbm=byt / t / 1e9 / HBM_PEAK_GBS)

    # algorithmic HBM bytes of the two expert GEMMs of a layer (operands and
    # their scales read once, output written once) per encoded byte/element
    def gemm_bytes(M, E_, I_, H_, a_el, w_el, a_row=0.0):
        fc1 = M * H_ * a_el + M * a_row + E_ * 2 * I_ * H_ * w_el + M * 2 * I_ * 2
        fc2 = M * I_ * a_el + M * a_row + E_ * H_ * I_ * w_el + M * H_ * 2
        return fc1 + fc2

    by_q3 = {"q3_gemm": gemm_bytes(M4, E, I4, H, 1 + 1 / 32, 1 + 1 / 32),
             "q3_gemm_uniform": gemm_bytes(M4, E, I4, H, 1 + 1 / 32, 1 + 1 / 32),
             "q3_gemm_fp8b": gemm_bytes(M4, E, I4, H, 1 + 4 / 128, 1 + 4 / 128 ** 2)}
    by_ds = gemm_bytes(M5, E5 + 1, I5, H5, 0.5 + 1 / 16, 0.5 + 1 / 16, a_row=4)

    def floor(c, flop, byt, peak_tflops, t):
        # the larger of the compute and the HBM time at peak: the attainable bound
        fl = max(flop / peak_tflops / 1e12, byt / HBM_PEAK_GBS / 1e9)
        c.update(bytes=byt, floor_us=fl * 1e6, frac_floor=fl / t)

    for n, ts in timings.items():
        if n not in sel:
            continue
        t = float(np.mean(ts)) / (args.reps if n in REPEAT_ROWS else 1)
        c = {"time_us": t * 1e6}
        if n == "mxfp8_quant":
            hbm(c, R2 * (2 + 2 * (1 + 1 / 32)), t)
        elif n == "nvfp4_token":
            hbm(c, R2 * (2 + 0.5 + 1 / 16) + T2 * 4, t)
        elif n == "nvfp4_joint_w":
            hbm(c, E * I2 * H * (2 + 0.5 + 1 / 16) + E * 4, t)
        elif n == "q3_wquant":
            hbm(c, (E * 2 * I4 * H + E * H * I4) * (2 + 1 + 1 / 32), t)
        elif n in ("q3_fwd", "q3_gemm", "q3_gemm_fp8b", "q3_gemm_uniform"):
            c.update(flop=fl_q3, tflops=fl_q3 / t / 1e12, frac_fp8=fl_q3 / t / 1e12 / FP8_PEAK_TFLOPS)
            if n in by_q3:
                floor(c, fl_q3, by_q3[n], FP8_PEAK_TFLOPS, t)
        elif n == "q3_dequant":
            el = E * 2 * I4 * H + E * H * I4 + M4 * H + M4 * I4
            hbm(c, el * (1 + 1 / 32 + 2), t)
        elif n == "q3_bwd":
            fl = 2 * fl_q3
            c.update(flop=fl, tflops=fl / t / 1e12, frac_bf16=fl / t / 1e12 / BF16_PEAK_TFLOPS)
        elif n == "q3_bwd_mx":
            fl = 2 * fl_q3  # algorithmic: routed rows only, padding rows not counted
            c.update(flop=fl, tflops=fl / t / 1e12, frac_fp8=fl / t / 1e12 / FP8_PEAK_TFLOPS)
        elif n == "ds_wquant":
            hbm(c, ((E5 + 1) * (2 * I5 * H5 + H5 * I5)) * (2 + 0.5 + 1 / 16), t)
        elif n in ("ds_fwd", "ds_gemm"):
            c.update(flop=fl_ds, tflops=fl_ds / t / 1e12,
                     frac_bf16=fl_ds / t / 1e12 / BF16_PEAK_TFLOPS)
            if n == "ds_gemm":
                floor(c, fl_ds, by_ds, BF16_PEAK_TFLOPS, t)
        elif n == "ds_fc2_online":
            fl = 2.0 * M5 * H5 * I5
            c.update(flop=fl, tflops=fl / t / 1e12, frac_bf16=fl / t / 1e12 / BF16_PEAK_TFLOPS)
        elif n == "ds_reconstruct":
            el = M5 * H5 + (E5 + 1) * (2 * I5 * H5 + H5 * I5)
            hbm(c, el * (0.5 + 1 / 16 + 2), t)
        elif n == "hbm_copy":
            hbm(c, 2 * COPY_BYTES, t)
        for k, v in list(c.items()):
            if isinstance(v, float):
                c[k] = round(v, 4)
        comp[n] = c
        log(n, c)

    # ------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline and "mxfp8_quant" in sel:
        import oracle
        host = st["sets"][0].view(torch.int16).cpu().numpy().view(np.uint16)
        oracle.build()
        reps, t_cpu, t_start = 0, 0.0, time.perf_counter()
        # about 10 s of oracle work: whole repetitions of the full workload
        while reps < 1 or (reps < 400 and time.perf_counter() - t_start < 10.0):
            t1 = time.perf_counter()
            oracle.quantize_mxfp8(host)
            t_cpu += time.perf_counter() - t1
            reps += 1
        byt = R2 * (2 + 2 * (1 + 1 / 32))
        cpu = {"value": round(byt * reps / t_cpu / 1e9, 4), "unit": "GB/s",
               "cores": oracle.threads(), "kind": "oracle",
               "sample": f"MXFP8 row+col quantize of the full 16384x2048 activation set, "
                         f"{reps} repetitions ({t_cpu:.1f} s)"}
        # the same oracle on one thread, over the first 2048 rows
        n1 = oracle.threads()
        oracle.set_threads(1)
        part = np.ascontiguousarray(host[:2048])
        t1 = time.perf_counter()
        oracle.quantize_mxfp8(part)
        t_one = time.perf_counter() - t1
        oracle.set_threads(n1)
        cpu["single_thread"] = {"value": round(part.size * (2 + 2 * (1 + 1 / 32)) / t_one / 1e9, 4),
                                "unit": "GB/s", "cores": 1,
                                "sample": f"rows 0..2047 of the same set ({t_one:.1f} s)"}
        # the grouped-GEMM oracle (exact decode, binary64 product) on one
        # expert of the Qwen3 gate_up shape: 4096 rows x 2048 -> 1536
        xa = wl.activations(4096, H, seed=31)
        wb = wl.expert_weights(1, 2 * I4, H, 0.02, tag=31).reshape(2 * I4, H)
        qa, sa = oracle.quantize_mxfp8_rowwise(xa)
        qb, sb_ = oracle.quantize_mxfp8_rowwise(wb)
        t1 = time.perf_counter()
        a64, b64 = oracle.decode_mxfp8(qa, sa), oracle.decode_mxfp8(qb, sb_)
        oracle.grouped_gemm(a64, b64[None], np.array([0, 4096]))
        t_g = time.perf_counter() - t1
        cpu["gemm"] = {"value": round(2 * 4096 * 2 * I4 * H / t_g / 1e12, 6), "unit": "TFLOP/s",
                       "cores": oracle.threads(),
                       "sample": f"MXFP8 grouped GEMM oracle, one expert of the Qwen3 gate_up "
                                 f"shape (4096 x 2048 @ 2048 x 1536, {t_g:.2f} s), sampled"}
        log("cpu baseline", cpu)

    head = comp.get("mxfp8_quant", {})
    value = head.get("gbs")
    gem = comp.get("q3_gemm", {})
    out = {
        "metric": "quantize HBM GB/s + MXFP8/NVFP4 MoE grouped-GEMM TFLOPS, 1 MI355X",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "MXFP8 row-wise + column-wise quantize of 16384 x 2048 bf16 "
                               "activations (log-normal token scale, outlier channels); the "
                               "step also runs every other hot-path row (components)",
                   "tokens": T2, "hidden": H},
        "gemm_mxfp8_tflops": gem.get("tflops"),
        "gemm_nvfp4_tflops": comp.get("ds_gemm", {}).get("tflops"),
        "roofline": {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4) if value else None,
                     "traffic": measured_traffic(), "kernel": TRAFFIC["kernel"]},
        "cpu_baseline": cpu,
        "components": comp,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
