#!/usr/bin/env python3
"""Benchmark: one step = forward + backward of the reparameterised LLaMA-style
non-attention block at hidden 2048 (M = 8192 tokens = 4 x 2048, F = 8192,
16 heads x 128) through the GEMM + epilogue library, on one MI355X.

Prints one JSON line with the step throughput (algorithmic TFLOP/s of the
step's GEMMs), the roofline of the dominant kernel (the gate/up GEMM with the
SwiGLU epilogue, timed with HIP events on the stream it runs on), and the CPU
oracle timed on the host on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--hidden 2048|4096]
                       [--precision bf16|fp8] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense MFMA, published


def block_flops(M, D, F):
    """Algorithmic FLOPs (2 M N K per GEMM) of the block forward and backward."""
    fwd = 2 * M * D * (3 * D) + 2 * M * D * D + 2 * M * D * (2 * F) + 2 * M * F * D
    return fwd, 2 * fwd


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--hidden", type=int, default=2048, choices=(2048, 4096))
    ap.add_argument("--precision", default="bf16", choices=("bf16", "fp8"))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="token rows of the CPU-oracle sample")
    return ap.parse_args()


def cpu_baseline(shape_full, seed, rows):
    """The oracle (numpy, contract mode) forward + backward on the first
    `rows` tokens of the same workload, timed on the host cores."""
    import numpy as np
    import coda_inputs as ci
    from oracle import block as ob
    shape = ci.BlockShape(M=rows, D=shape_full.D, F=shape_full.F, seq_len=shape_full.seq_len)
    P = ci.block_inputs(shape, seed)
    t0 = time.perf_counter()
    F = ob.block_forward_contract(P, shape)
    ob.block_backward_contract(P, F, shape)
    dt = time.perf_counter() - t0
    fwd, bwd = block_flops(rows, shape.D, shape.F)
    cores = len(os.sched_getaffinity(0))
    return {"value": (fwd + bwd) / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {shape_full.M} token rows, block fwd+bwd (numpy fp32 contract mode, "
                      f"BLAS threads = {os.environ.get('OMP_NUM_THREADS', 'default')}), {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    cpu = None
    import coda_inputs as ci
    cfg = ci.CFG2 if args.hidden == 2048 else ci.CFG3
    seed = ci.SEEDS["cfg2" if args.hidden == 2048 else "cfg3"]
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, seed, args.cpu_rows)

    import numpy as np
    import torch
    import gemm_epilogue_fp8_amd as coda
    from gemm_epilogue_fp8_amd.block import Block

    dev = "cuda:0"
    torch.cuda.set_device(0)
    P = ci.block_inputs(cfg, seed)
    to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    params = {k: to(v, torch.float32 if k in ("g1", "g2", "gq", "gk") else torch.bfloat16) for k, v in P.items()}
    del P
    prec = coda.PREC_FP8 if args.precision == "fp8" else coda.PREC_BF16
    blk = Block(params, cfg.D, cfg.F, seq_len=cfg.seq_len, theta=cfg.theta, eps=cfg.eps, precision=prec)
    M = cfg.M
    f = blk.alloc_forward(M, dev)
    g = blk.alloc_backward(M, dev)
    for k in ("dWqkv", "dWo", "dWgu", "dWd", "dg1", "dg2", "dgq", "dgk"):
        g[k].zero_()
    x, o = params["x"], params["o"]
    dY, dq, dk, dv = params["dY"], params["dq"], params["dk"], params["dv"]

    # the dominant kernel (gate/up GEMM + SwiGLU epilogue) is bracketed by
    # events on the stream the library launches on (torch's current stream)
    f3_events = []

    def step(record=False):
        f_ = f
        coda.row_sumsq(x, f_["P_x"])
        coda.linear_qknorm_rope_fwd(x, blk.w["qkv"], blk.gq, blk.gk, blk.rope, blk.seq_len, blk.eps,
                                    f_["q"], f_["k"], f_["v"], sumsq_partials=f_["P_x"],
                                    save_qk_pre=f_["qk_pre"], r_out=f_["r1"], precision=prec)
        coda.linear_rmsnorm_residual_fwd(o, blk.w["o"], x, f_["h1"], sumsq_partials_out=f_["P2"], precision=prec)
        if record:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        coda.linear_swiglu_fwd(f_["h1"], blk.w["gu"], blk.eps, f_["a"], sumsq_partials=f_["P2"],
                               save_hgu=f_["hgu"], r_out=f_["r2"], precision=prec)
        if record:
            e1.record()
            f3_events.append((e0, e1))
        coda.linear_rmsnorm_residual_fwd(f_["a"], blk.w["d"], f_["h1"], f_["y"], sumsq_partials_out=f_["P4"],
                                         precision=prec)
        blk.backward(x, o, f_, dY, dq, dk, dv, grads=g, beta=1.0)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step(record=True)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    ms = max(wall * 1e3 / args.steps, gpu_ms)

    fwd, bwd = block_flops(M, cfg.D, cfg.F)
    tflops = (fwd + bwd) / (ms * 1e-3) / 1e12
    f3_ms = sum(a.elapsed_time(b) for a, b in f3_events) / len(f3_events)
    f3_flop = 2 * M * (2 * cfg.F) * cfg.D
    f3_tflops = f3_flop / (f3_ms * 1e-3) / 1e12
    peak = MI355X_PEAK_TFLOPS[args.precision]
    out = {
        "metric": "fused GEMM+epilogue TFLOP/s & % MFMA peak; block fwd+bwd ms, hidden 2048/4096",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.precision,
        "data": "synthetic",
        "config": {"workload": f"LLaMA-style non-attention block forward+backward, hidden {cfg.D}",
                   "tokens": M, "hidden": cfg.D, "mlp": cfg.F, "heads": cfg.heads, "head_dim": 128,
                   "seq_len": cfg.seq_len, "grad_accumulate_beta": 1.0},
        "block_fwd_bwd_ms": round(ms, 4),
        "pct_of_peak": round(100 * tflops / peak, 2),
        "roofline": {"bound": "mfma", "kernel": "gate/up GEMM + SwiGLU epilogue (M x 2F x D)",
                     "achieved": round(f3_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(f3_tflops / peak, 4), "avg_ms": round(f3_ms, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
