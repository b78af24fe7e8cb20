"""Benchmark of the block-scaled quantizer + MoE grouped-GEMM hot path on one
MI355X.

One step is one pass of every hot-path row over one batch of synthetic,
seeded input, with all inputs resident in HBM:

  mxfp8_quant      MXFP8 row-wise + column-wise quantize, 16384 x 2048 bf16
                   activations (Qwen3-30B-A3B hidden size)   <- headline value
  nvfp4_token      per-token NVFP4 quantize of the same-shaped activations
  nvfp4_joint_w    joint gate/up NVFP4 quantize of 128 experts' [1536 x 2048]
  moe_mxfp8_fwd    MXFP8 MoE expert layer forward, 8192 tokens top-8 over 128
                   experts (Zipf 1.1 load): weight quantize, route, token
                   quantize, gather, gate_up grouped GEMM, SwiGLU x prob,
                   quantize, down grouped GEMM, combine
  dequant_bwd      dequantize of the forward operands (dequantized backward)
  bf16_bwd         BF16 dgrad + wgrad grouped GEMMs of both expert GEMMs on
                   the dequantized operands

Quantizer inputs rotate over several buffer sets larger than the 256 MB
Infinity Cache so their rate is HBM's.  Each row is timed with HIP events
on the stream its kernels run on; `value` is the MXFP8 quantizer's HBM
rate (algorithmic bytes / kernel time).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
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
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA BF16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--sets", type=int, default=3, help="rotating quantizer input sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--rows", default="all",
                   help="comma list of rows to run (default all)")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                          "multi-GPU runs are not part of this build",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import precision_quantization_moe_amd as pqm
    from precision_quantization_moe_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs an MI355X GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows_sel = None if args.rows == "all" else set(args.rows.split(","))
    want = lambda r: rows_sel is None or r in rows_sel

    def to_dev_bf16(a: np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(dev)

    # ------------------------------------------------------------ inputs
    T2, H = 16384, 2048
    log("generating inputs")
    sets = [to_dev_bf16(wl.activations(T2, H, seed=100 + i)) for i in range(args.sets)]
    E, I2 = 128, 1536
    w_joint = to_dev_bf16(wl.expert_weights(E, I2, H, 0.02, tag=7).reshape(E * I2, H)) \
        if want("nvfp4_joint_w") else None
    # MXFP8 MoE layer (Qwen3-30B-A3B experts)
    T4, K4, I4 = 8192, 8, 768
    x4 = to_dev_bf16(wl.activations(T4, H, seed=4))
    ids = torch.from_numpy(wl.zipf_routing(T4, E, K4)).to(dev)
    prob = torch.from_numpy(wl.router_probs(T4, K4).reshape(-1)).to(dev)
    W1 = to_dev_bf16(wl.expert_weights(E, 2 * I4, H, 0.02).reshape(E * 2 * I4, H))
    W2 = to_dev_bf16(wl.expert_weights(E, H, I4, 0.02, tag=1).reshape(E * H, I4))
    M4 = T4 * K4
    dY = to_dev_bf16(wl.output_grad(M4, H))
    dC = to_dev_bf16(wl.output_grad(M4, 2 * I4, seed=5))
    torch.cuda.synchronize()
    log("inputs ready")

    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    state = {}

    def row_mxfp8(s):
        pqm.quantize_mxfp8(sets[s % len(sets)])

    def row_nvfp4(s):
        pqm.quantize_nvfp4_per_token(sets[s % len(sets)])

    def row_joint(s):
        pqm.quantize_nvfp4_per_token(w_joint, rows_per_scale=I2)

    def row_layer(s):
        w1q, w1s, _, _ = pqm.quantize_mxfp8(W1, colwise=False)
        w2q, w2s, _, _ = pqm.quantize_mxfp8(W2, colwise=False)
        off, src, slot = pqm.moe_route(ids, E)
        qx, sx, _, _ = pqm.quantize_mxfp8(x4, colwise=False)
        qa = pqm.moe_gather_rows(qx, src, K4)
        sa = pqm.moe_gather_rows(sx, src, K4)
        c = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qa, w1q, off, 2 * I4, H,
                                 a_scale=sa, b_scale=w1s, out_dtype=pqm.OUT_BF16)
        d = pqm.swiglu_prob(c, prob, src)
        qd, sd, _, _ = pqm.quantize_mxfp8(d, colwise=False)
        y = pqm.moe_grouped_gemm(pqm.FMT_MXFP8, pqm.GEMM_FPROP, qd, w2q, off, H, I4,
                                 a_scale=sd, b_scale=w2s, out_dtype=pqm.OUT_BF16)
        out = pqm.moe_combine(y, slot)
        state.update(w1q=w1q, w1s=w1s, w2q=w2q, w2s=w2s, off=off, qa=qa, sa=sa, qd=qd, sd=sd,
                     out=out)

    def row_dequant(s):
        st = state
        state["w1d"] = pqm.dequantize(pqm.FMT_MXFP8, st["w1q"], st["w1s"])
        state["w2d"] = pqm.dequantize(pqm.FMT_MXFP8, st["w2q"], st["w2s"])
        state["ad"] = pqm.dequantize(pqm.FMT_MXFP8, st["qa"], st["sa"])
        state["dd"] = pqm.dequantize(pqm.FMT_MXFP8, st["qd"], st["sd"])

    def row_bwd(s):
        st = state
        off = st["off"]
        # FC2: dD = dY . W2 (W2 [E, H, I]: contraction over H rows); dW2 = dY^T D
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, dY, st["w2d"], off, I4, H,
                             out_dtype=pqm.OUT_BF16)
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_WGRAD, dY, st["dd"], off, H, I4,
                             out_dtype=pqm.OUT_FP32)
        # FC1: dX = dC . W1 (W1 [E, 2I, H]); dW1 = dC^T X
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_DGRAD, dC, st["w1d"], off, H, 2 * I4,
                             out_dtype=pqm.OUT_BF16)
        pqm.moe_grouped_gemm(pqm.FMT_BF16, pqm.GEMM_WGRAD, dC, st["ad"], off, 2 * I4, H,
                             out_dtype=pqm.OUT_FP32)

    rows = [("mxfp8_quant", row_mxfp8), ("nvfp4_token", row_nvfp4),
            ("nvfp4_joint_w", row_joint), ("moe_mxfp8_fwd", row_layer),
            ("dequant_bwd", row_dequant), ("bf16_bwd", row_bwd)]
    rows = [(n, f) for n, f in rows if want(n)]
    if any(n in ("dequant_bwd", "bf16_bwd") for n, _ in rows) and not want("moe_mxfp8_fwd"):
        rows.insert(0, ("moe_mxfp8_fwd", row_layer))

    timings = {n: [] for n, _ in rows}
    for step in range(args.warmup + args.steps):
        if step == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        evs = []
        for n, f in rows:
            a, b = ev(), ev()
            a.record(stream)
            f(step)
            b.record(stream)
            evs.append((n, a, b))
        if step >= args.warmup:
            state.setdefault("_evs", []).append(evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for evs in state["_evs"]:
        for n, a, b in evs:
            timings[n].append(a.elapsed_time(b) * 1e-3)

    comp = {}
    R2 = T2 * H
    fl1 = 2.0 * M4 * (2 * I4) * H
    fl2 = 2.0 * M4 * H * I4
    for n, ts in timings.items():
        t = float(np.mean(ts))
        c = {"time_us": round(t * 1e6, 2)}
        if n == "mxfp8_quant":
            byt = R2 * (2 + 2 * (1 + 1 / 32))
            c.update(bytes=byt, gbs=byt / t / 1e9, frac_hbm=byt / t / 1e9 / HBM_PEAK_GBS)
        elif n == "nvfp4_token":
            byt = R2 * (2 + 0.5 + 1 / 16) + T2 * 4
            c.update(bytes=byt, gbs=byt / t / 1e9, frac_hbm=byt / t / 1e9 / HBM_PEAK_GBS)
        elif n == "nvfp4_joint_w":
            byt = E * I2 * H * (2 + 0.5 + 1 / 16) + E * 4
            c.update(bytes=byt, gbs=byt / t / 1e9, frac_hbm=byt / t / 1e9 / HBM_PEAK_GBS)
        elif n == "moe_mxfp8_fwd":
            c.update(gemm_flop=fl1 + fl2, layer_tflops=(fl1 + fl2) / t / 1e12)
        elif n == "bf16_bwd":
            fl = 2 * (fl1 + fl2)
            c.update(flop=fl, tflops=fl / t / 1e12, frac_bf16=fl / t / 1e12 / BF16_PEAK_TFLOPS)
        for k, v in list(c.items()):
            if isinstance(v, float):
                c[k] = round(v, 4)
        comp[n] = c
        log(n, c)

    # ------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline and want("mxfp8_quant"):
        import oracle
        host = sets[0].view(torch.int16).cpu().numpy().view(np.uint16)
        oracle.build()
        reps, t_cpu, t_start = 0, 0.0, time.perf_counter()
        while reps < 10 and time.perf_counter() - t_start < 10.0:
            t1 = time.perf_counter()
            oracle.quantize_mxfp8(host)
            t_cpu += time.perf_counter() - t1
            reps += 1
        byt = R2 * (2 + 2 * (1 + 1 / 32))
        cpu = {"value": round(byt * reps / t_cpu / 1e9, 4), "unit": "GB/s",
               "cores": int(oracle.lib().pqo_omp_threads()), "kind": "oracle",
               "sample": f"MXFP8 row+col quantize of the full 16384x2048 activation "
                         f"set, {reps} repetitions ({t_cpu:.1f} s)"}
        log("cpu baseline", cpu)

    head = comp.get("mxfp8_quant", {})
    value = head.get("gbs")
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
                               "activations (log-normal token scale, outlier channels); "
                               "step also runs every other hot-path row (components)",
                   "tokens": T2, "hidden": H},
        "roofline": {"bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4) if value else None,
                     "traffic": None, "kernel": "k_quantize_mxfp8<true,true>"},
        "cpu_baseline": cpu,
        "components": comp,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
