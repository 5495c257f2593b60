#!/usr/bin/env python3
"""Benchmark of the GEMM + epilogue library on one MI355X.

One step = forward + backward of the reparameterised LLaMA-style
non-attention block (QKV with delayed RMSNorm + QK-norm + RoPE, O-projection
+ residual + next-norm partials, gate/up + SwiGLU, down-projection +
residual; backward with dSwiGLU, RMSNorm-backward corrections and fp32
weight-gradient accumulation) on synthetic inputs resident in HBM.

Default workload: hidden 2048, MLP 8192, 16 heads x 128, M = 8192 tokens
(4 x 2048).  --config cfg3 runs hidden 4096 (MLP 11008, 32 heads), --config
cfg5 hidden 8192 (MLP 28672, 64 heads, M = 4096) with E4M3 operands.

Prints one JSON line: step throughput (algorithmic TFLOP/s = 2MNK over the
step's GEMMs), block fwd+bwd ms, the unfused baseline (same mainloop with
plain stores + separate elementwise kernels) timed in the same run, a per-call
breakdown, the roofline of the dominant kernel (gate/up GEMM + SwiGLU epilogue,
timed with HIP events on the stream it runs on) and the CPU oracle timed on
the host on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0, "fp6": 10100.0, "fp4": 10100.0}   # MI355X dense MFMA, published
HBM_GBPS = 8000.0


def block_flops(M, D, F):
    """Algorithmic FLOPs (2 M N K per GEMM) of the block forward and backward."""
    fwd = 2 * M * D * (3 * D) + 2 * M * D * D + 2 * M * D * (2 * F) + 2 * M * F * D
    return fwd, 2 * fwd


# The sources the dominant kernel (bf16 gate/up GEMM + SwiGLU epilogue) is built from
DOMINANT_KERNEL_SOURCES = ("coda_device.hpp", "gemm_core.hpp", "epilogues.hpp", "launch.hpp", "gemm_nn.hip")


def kernel_source_hash():
    """Hash of the dominant kernel's HIP sources, to tell whether stored
    counter data is current."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gemm_epilogue_fp8_amd", "csrc")
    for f in DOMINANT_KERNEL_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(config, precision):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, if it was taken on the current sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    e = t.get(f"{config}_{precision}")
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e["bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="cfg2", choices=("cfg2", "cfg3", "cfg5"))
    ap.add_argument("--precision", default=None, choices=("bf16", "fp8", "mxfp8"),
                    help="GEMM operands: bf16, E4M3 with per-row / per-column amax scales (fp8), or E4M3 with "
                         "one E8M0 exponent per 32 values of the contracted axis (mxfp8)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-unfused", action="store_true", help="skip the unfused baseline")
    ap.add_argument("--cpu-rows", type=int, default=0, help="token rows of the CPU-oracle sample (0 = all)")
    ap.add_argument("--no-mx", action="store_true", help="skip the block-scaled (MXFP8) GEMM leg")
    ap.add_argument("--small", action="store_true",
                    help="also time the small SwiGLU layer's latency (opt-in: its launches share the gate/up "
                         "kernel's name, so a profile of the default run keeps that kernel's average clean)")
    ap.add_argument("--ce-only", action="store_true",
                    help="run only the linear + cross-entropy leg and print its JSON object (for per-kernel counters)")
    ap.add_argument("--no-ce", action="store_true", help="skip the linear + cross-entropy leg")
    ap.add_argument("--no-mfma-loop", action="store_true", help="skip the MFMA-only achievable-rate leg")
    ap.add_argument("--no-h4096", action="store_true", help="skip the hidden-4096 block leg of the default run")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the block step")
    ap.add_argument("--no-coresident", action="store_true",
                    help="skip the block step under the co-resident gate/up schedule")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 3 device-to-device copies of 1 GiB (the reference kernel for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    return ap.parse_args()


def copy_calibration():
    """Three copies of exactly 1 GiB between two device buffers: a kernel whose
    HBM traffic is known (1 GiB read + 1 GiB written per launch)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": {"read": n, "write": n}, "launches": 3}))


def small_layer_leg(warmup=20, calls=200):
    """The small SwiGLU layer (x [256, 512], gate and up weights [512, 1024]
    each, RMSNorm over x folded in): one linear_swiglu_fwd call, r computed
    inside the call.  At 0.54 GFLOP it is far below the ridge point, so its
    figure is latency: median and minimum of per-call HIP events."""
    import numpy as np
    import torch
    import coda_inputs as ci
    import gemm_epilogue_fp8_amd as coda

    dev = "cuda:0"
    shape = ci.CFG1
    P = ci.swiglu_inputs(shape, ci.SEEDS["cfg1"])
    to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    x = to(P["x"], torch.bfloat16)
    Wgu = torch.empty((shape.K, 2 * shape.F), dtype=torch.bfloat16, device=dev)
    coda.pack_gate_up(to(P["Wg"], torch.bfloat16), to(P["Wu"], torch.bfloat16), to(P["g"], torch.float32), Wgu)
    out = torch.empty((shape.M, shape.F), dtype=torch.bfloat16, device=dev)
    fn = lambda: coda.linear_swiglu_fwd(x, Wgu, shape.eps, out)
    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return {"workload": f"SwiGLU layer, x [{shape.M}, {shape.K}], gate/up [{shape.K}, {shape.F}] each, bf16",
            "gflop": round(2 * shape.M * 2 * shape.F * shape.K / 1e9, 3),
            "us_median": round(t[len(t) // 2], 2), "us_min": round(t[0], 2)}


def mx_leg(warmup, steps):
    """The block-scaled E4M3 GEMM (one E8M0 scale per 32 K values, applied by
    the scaled MFMA) with the residual epilogue, out = z + a W, at the
    hidden-8192 down-projection shape (M 4096, K 28672, N 8192), against the
    per-token x per-channel amax-scaled E4M3 path of the same layer (which
    includes the quantisation of the activation a), and the same layer with
    MXFP4 (E2M1) and MXFP6 (E2M3) operands.  Synthetic inputs drawn on
    the device from a seeded generator."""
    import torch
    import gemm_epilogue_fp8_amd as coda
    M, K, N = 4096, 28672, 8192
    gen = torch.Generator(device="cuda:0").manual_seed(7)
    a = torch.randn((M, K), generator=gen, device="cuda:0").to(torch.bfloat16)
    W = (torch.randn((K, N), generator=gen, device="cuda:0") * K ** -0.5).to(torch.bfloat16)
    z = torch.randn((M, N), generator=gen, device="cuda:0").to(torch.bfloat16)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    Qw, Sw = coda.quantize_mxfp8(W, 0)
    Qa, Sa = coda.quantize_mxfp8(a, 1)
    wt = coda.Weight(W).prepare_fp8()
    prog = [(coda.EPI_ADD_TILE, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)]

    def ev_ms(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    gemm_ms = ev_ms(lambda: coda.gemm_mx(prog, Qa, Sa, Qw, Sw, out, aux=[z]))
    quant_ms = ev_ms(lambda: coda.quantize_mxfp8(a, 1, Qa, Sa))
    rowcol_ms = ev_ms(lambda: coda.linear_rmsnorm_residual_fwd(a, wt, z, out, precision=coda.PREC_FP8))
    flop = 2 * M * N * K
    tf = flop / (gemm_ms * 1e-3) / 1e12
    del Qw, Sw, Qa, Sa, wt
    # the same layer with MXFP4 (E2M1) operands
    Q4w, S4w = coda.quantize_mxfp4(W, 0)
    Q4a, S4a = coda.quantize_mxfp4(a, 1)
    fp4_ms = ev_ms(lambda: coda.gemm_mx4(prog, Q4a, S4a, Q4w, S4w, out, aux=[z]))
    quant4_ms = ev_ms(lambda: coda.quantize_mxfp4(a, 1, Q4a, S4a))
    tf4 = flop / (fp4_ms * 1e-3) / 1e12
    del Q4w, S4w, Q4a, S4a
    # and with MXFP6 (E2M3) operands
    Q6w, S6w = coda.quantize_mxfp6(W, 0, "e2m3")
    Q6a, S6a = coda.quantize_mxfp6(a, 1, "e2m3")
    fp6_ms = ev_ms(lambda: coda.gemm_mx6(prog, "e2m3", Q6a, S6a, Q6w, S6w, out, aux=[z]))
    tf6 = flop / (fp6_ms * 1e-3) / 1e12
    del a, W, z, out, Q6w, S6w, Q6a, S6a
    torch.cuda.empty_cache()
    return {"workload": f"out = z + a W, M {M}, K {K}, N {N}, MXFP8 operands (E4M3, E8M0 per 32 K)",
            "gemm_ms": round(gemm_ms, 4), "tflops": round(tf, 1), "frac_of_fp8_peak": round(tf / PEAK_TFLOPS["fp8"], 4),
            "quantize_a_ms": round(quant_ms, 4),
            "gemm_plus_quantize_ms": round(gemm_ms + quant_ms, 4),
            "per_row_col_fp8_layer_ms": round(rowcol_ms, 4),
            "mxfp4_gemm_ms": round(fp4_ms, 4), "mxfp4_tflops": round(tf4, 1),
            "mxfp4_frac_of_fp4_peak": round(tf4 / PEAK_TFLOPS["fp4"], 4), "mxfp4_quantize_a_ms": round(quant4_ms, 4),
            "mxfp6_e2m3_gemm_ms": round(fp6_ms, 4), "mxfp6_e2m3_tflops": round(tf6, 1),
            "mxfp6_e2m3_frac_of_fp6_peak": round(tf6 / PEAK_TFLOPS["fp6"], 4)}


OPERANDS = {False: "", True: " with E4M3 operands (per-row / per-column amax scales)",
            "mx": " with MXFP8 operands (E4M3, one E8M0 exponent per 32 values)"}


def mfma_loop_leg(f3_tflops):
    """The achievable matrix-core rate: an MFMA-only loop (no memory traffic,
    no barriers) on every compute unit, timed with HIP events on the current
    stream, with the engine clock it ran at."""
    import torch
    import gemm_epilogue_fp8_amd as coda
    out = {"workload": "MFMA-only loop, 1024 workgroups of 8 waves, 4 independent 32x32 accumulator chains a wave"}
    for name, dt, iters in (("bf16", coda.CODA_BF16, 256), ("fp8", coda.CODA_E4M3, 128),
                            ("fp4", coda.CODA_E2M1X2, 64)):
        blocks = 1024
        buf = torch.zeros(blocks * 3, dtype=torch.float32, device="cuda")
        coda.probe_mfma_loop(dt, blocks, iters, buf)   # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            flops, res = coda.probe_mfma_loop(dt, blocks, iters, buf)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        cyc, ticks = res[:, 1].double(), res[:, 2].double()
        ghz = float(torch.median(cyc / ticks.clamp(min=1.0)) * 0.1)
        tf = flops / (ms * 1e-3) / 1e12
        out[f"{name}_tflops"] = round(tf, 1)
        out[f"{name}_frac_of_published"] = round(tf / PEAK_TFLOPS[name], 4)
        out[f"{name}_engine_clock_ghz"] = round(ghz, 3)
    out["dominant_kernel_frac_of_achievable"] = round(f3_tflops / out["bf16_tflops"], 4)
    return out


def ce_leg(warmup, steps):
    """Linear + cross-entropy forward and backward at h [8192, 2048],
    W_vocab [2048, 128256] with 410 ignored rows (the logits are never
    materialised; the backward recomputes them), plain and with the final
    RMSNorm folded in.  Synthetic inputs drawn on the device from a seeded
    generator: h ~ N(0, 1), W ~ N(0, 1/2048), labels uniform in [0, V)."""
    import torch
    import gemm_epilogue_fp8_amd as coda
    M, D, V = 8192, 2048, 128256
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(11)
    h = torch.randn((M, D), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((D, V), generator=gen, device=dev) * D ** -0.5).to(torch.bfloat16)
    labels = torch.randint(0, V, (M,), generator=gen, device=dev, dtype=torch.int32)
    labels[torch.randperm(M, generator=gen, device=dev)[:410]] = -100
    g = (1 + 0.1 * torch.randn(D, generator=gen, device=dev)).float()
    Wt = coda.fold_gain(W, g, torch.empty_like(W))
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
    loss, lse, nv, r = f32(1), f32(M), torch.empty(1, dtype=torch.int32, device=dev), f32(M)
    dh = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    dW, dg = f32(D, V), f32(D)

    def ev_ms(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    fwd = lambda: coda.linear_cross_entropy_fwd(h, W, labels, loss, lse, nv)
    out = {"workload": f"linear + cross-entropy, h [{M}, {D}], W_vocab [{D}, {V}], 410 ignored rows",
           "model_gflop": round(3 * 2 * M * D * V / 1e9, 1), "with_recompute_gflop": round(4 * 2 * M * D * V / 1e9, 1)}
    out["fwd_ms"] = round(ev_ms(fwd), 4)
    for chunk in (0, 1024):
        bwd = lambda: coda.linear_cross_entropy_bwd(h, W, labels, lse, nv, 1.0, dh, dW, beta=1.0, chunk_rows=chunk)
        ms = ev_ms(bwd)
        out[f"bwd_ms_chunk{chunk}"] = round(ms, 4)
    best = min(out["bwd_ms_chunk0"], out["bwd_ms_chunk1024"])
    tot = out["fwd_ms"] + best
    out["fwd_bwd_ms"] = round(tot, 4)
    out["model_tflops"] = round(3 * 2 * M * D * V / (tot * 1e-3) / 1e12, 1)
    out["hw_tflops"] = round(4 * 2 * M * D * V / (tot * 1e-3) / 1e12, 1)
    nfwd = lambda: coda.linear_rmsnorm_cross_entropy_fwd(h, Wt, 1e-6, labels, loss, lse, nv, r_out=r)
    out["norm_fwd_ms"] = round(ev_ms(nfwd), 4)
    for chunk in (0, 1024):
        nbwd = lambda: coda.linear_rmsnorm_cross_entropy_bwd(h, r, Wt, W, g, labels, lse, nv, 1.0, dh, dW, dg,
                                                            beta=1.0, chunk_rows=chunk)
        out[f"norm_bwd_ms_chunk{chunk}"] = round(ev_ms(nbwd), 4)
    del h, W, Wt, dW, dh
    torch.cuda.empty_cache()
    return out


def cpu_baseline(shape_full, seed, rows, fp8):
    """The oracle (numpy, contract mode) forward + backward on the first
    `rows` tokens of the same workload, timed on the host cores."""
    import coda_inputs as ci
    from oracle import block as ob
    shape = ci.BlockShape(M=rows, D=shape_full.D, F=shape_full.F, seq_len=shape_full.seq_len)
    P = ci.block_inputs(shape, seed)
    t0 = time.perf_counter()
    F = ob.block_forward_contract(P, shape, fp8=fp8)
    ob.block_backward_contract(P, F, shape, fp8=fp8)
    dt = time.perf_counter() - t0
    fwd, bwd = block_flops(rows, shape.D, shape.F)
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OMP_NUM_THREADS") or os.environ.get("OPENBLAS_NUM_THREADS") or str(cores)
    return {"value": round((fwd + bwd) / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {shape_full.M} token rows of the same workload, block fwd+bwd, numpy "
                      f"float32 contract mode{OPERANDS[fp8]}, {dt:.1f} s"}


def partial_bytes(M, D, F):
    """Algorithmic HBM bytes of the cross-N-tile partial-reduction buffers of
    one block step (fp32, each written once by the producing epilogue and read
    once by its finish): the forward's sum-of-squares rows, the backward's T
    rows and the gain-gradient rows."""
    nt = lambda n: (n + 255) // 256
    f = 4
    fwd = {"P_x sumsq(x)": 2 * M * f, "P2 sumsq(h1)": 2 * nt(D) * M * f, "P4 sumsq(y)": 2 * nt(D) * M * f,
           "r1, r2 saves": 2 * M * f}
    bwd = {"T2 partials": 2 * nt(F) * M * f + 2 * M * f, "dg2 partials": 2 * nt(2 * F) * D * f,
           "T1": 2 * M * f, "dg1 partials": 2 * nt(3 * D) * D * f, "dgq, dgk partials": 4 * 128 * f * (M // 256 + 1)}
    return {"fwd": fwd, "bwd": bwd, "total_bytes": sum(fwd.values()) + sum(bwd.values())}


def block_leg(name, precision, args, breakdown=True):
    """One block configuration: fused forward + backward step time (HIP events
    on torch's current stream, which the library launches on), forward time,
    the dominant kernel's (gate/up GEMM + SwiGLU) average duration, the warm
    per-weight-update preparation (fold, pack, RoPE table, fp8 copies), the
    unfused baseline and a per-call breakdown."""
    import numpy as np
    import torch
    import coda_inputs as ci
    import gemm_epilogue_fp8_amd as coda
    from gemm_epilogue_fp8_amd.block import Block
    from gemm_epilogue_fp8_amd.unfused import UnfusedBlock

    dev = "cuda:0"
    cfg = {"cfg2": ci.CFG2, "cfg3": ci.CFG3, "cfg5": ci.CFG5}[name]
    seed = ci.SEEDS[name]
    fp8 = {"bf16": False, "fp8": True, "mxfp8": "mx"}[precision]
    P = ci.block_inputs(cfg, seed)
    to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    params = {k: to(v, torch.float32 if k in ("g1", "g2", "gq", "gk") else torch.bfloat16) for k, v in P.items()}
    del P
    prec = {"bf16": coda.PREC_BF16, "fp8": coda.PREC_FP8, "mxfp8": coda.PREC_MXFP8}[precision]
    torch.cuda.synchronize()
    t_prep = time.perf_counter()
    blk = Block(params, cfg.D, cfg.F, seq_len=cfg.seq_len, theta=cfg.theta, eps=cfg.eps, precision=prec)
    torch.cuda.synchronize()
    prep_cold_ms = (time.perf_counter() - t_prep) * 1e3
    M = cfg.M
    f = blk.alloc_forward(M, dev)
    g = blk.alloc_backward(M, dev)
    for k in ("dWqkv", "dWo", "dWgu", "dWd", "dg1", "dg2", "dgq", "dgk"):
        g[k].zero_()
    x, o = params["x"], params["o"]
    dY, dq, dk, dv = params["dY"], params["dq"], params["dk"], params["dv"]

    # The step as a list of library calls, so each can be bracketed by events
    # on the stream the library launches on (torch's current stream).
    calls = [
        ("aux row_sumsq(x)", lambda: coda.row_sumsq(x, f["P_x"])),
        ("F1 qkv+qknorm+rope", lambda: coda.linear_qknorm_rope_fwd(
            x, blk.w["qkv"], blk.gq, blk.gk, blk.rope, blk.seq_len, blk.eps, f["q"], f["k"], f["v"],
            sumsq_partials=f["P_x"], save_qk_pre=f["qk_pre"], r_out=f["r1"], precision=prec)),
        ("F2 o-proj+residual+sumsq", lambda: coda.linear_rmsnorm_residual_fwd(
            o, blk.w["o"], x, f["h1"], sumsq_partials_out=f["P2"], precision=prec)),
        ("F3 gate/up+swiglu", lambda: coda.linear_swiglu_fwd(
            f["h1"], blk.w["gu"], blk.eps, f["a"], sumsq_partials=f["P2"], save_hgu=f["hgu"], r_out=f["r2"],
            precision=prec)),
        ("F4 down+residual+sumsq", lambda: coda.linear_rmsnorm_residual_fwd(
            f["a"], blk.w["d"], f["h1"], f["y"], sumsq_partials_out=f["P4"], precision=prec)),
        ("B1+B3+B4 swiglu bwd", lambda: coda.linear_swiglu_bwd(
            dY, blk.w["d"], f["hgu"], f["r2"], f["h1"], blk.w["gu"], blk.Wgu, blk.g2, dY, g["dh1"], g["dWgu"],
            g["dg2"], beta=1.0, dh_gu_out=g["dht_gu"], precision=prec)),
        ("B2 dW_down", lambda: coda.linear_rmsnorm_residual_bwd(dY, f["a"], blk.w["d"], g["dWd"], beta=1.0,
                                                                 precision=prec)),
        ("B5+B6 o-proj bwd", lambda: coda.linear_rmsnorm_residual_bwd(g["dh1"], o, blk.w["o"], g["dWo"],
                                                                       da=g["do"], beta=1.0, precision=prec)),
        ("G1+B7+B8 qkv bwd", lambda: coda.linear_qknorm_rope_bwd(
            dq, dk, dv, x, f["r1"], f["qk_pre"], f["v"], blk.w["qkv"], blk.Wqkv, blk.g1, blk.gq, blk.gk,
            blk.rope, blk.seq_len, blk.eps, g["dh1"], g["dx"], g["dWqkv"], g["dg1"], g["dgq"], g["dgk"],
            beta=1.0, dh_qkv_out=g["dht_qkv"], precision=prec)),
    ]
    f3_events = []

    def step(record=None):
        """One step; with a list, the gate/up kernel's events are appended to it."""
        for call, fn in calls:
            if record is not None and call.startswith("F3"):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                record.append((e0, e1))
            else:
                fn()

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return max(wall, a.elapsed_time(b) / steps)

    for _ in range(args.warmup):
        step()
    # an event at the start of each timed step gives K - 1 per-step times
    # (median and minimum beside the mean)
    starts = []

    def step_marked():
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        starts.append(ev)
        step(f3_events)

    ms = timed(step_marked, args.steps)
    per_step = sorted(a.elapsed_time(b) for a, b in zip(starts[:-1], starts[1:]))
    f3_ms = sum(a.elapsed_time(b) for a, b in f3_events) / len(f3_events)
    fwd_ms = timed(lambda: [fn() for n, fn in calls[:5]], max(1, args.steps // 2))
    # The same step captured once as a HIP graph and replayed (the library
    # launches on the caller's stream and allocates nothing, so every kernel
    # of the step is captured; the workspaces were sized by the steps above).
    graph_ms = None
    if not getattr(args, "no_graph", False):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        graph_ms = timed(graph.replay, args.steps)
        del graph
    # The same step with the gate/up GEMM + SwiGLU under the co-resident
    # schedule (two 128 x 256 workgroups a compute unit, one's epilogue
    # overlapping the other's matrix work), and that kernel's own time.
    cores = None
    if precision == "bf16" and not args.no_coresident:
        cev = []
        with coda.schedule(coda.SCHED_CORESIDENT):
            for _ in range(max(1, args.warmup)):
                step()
            cms = timed(lambda: step(cev), args.steps)
        c3 = sum(a.elapsed_time(b) for a, b in cev) / len(cev)
        c3_flop = 2 * cfg.M * (2 * cfg.F) * cfg.D
        cores = {"schedule": "gate/up GEMM + SwiGLU as 128 x 256 tiles, two 4-wave workgroups a compute unit",
                 "block_fwd_bwd_ms": round(cms, 4), "gate_up_swiglu_ms": round(c3, 4),
                 "gate_up_swiglu_tflops": round(c3_flop / (c3 * 1e-3) / 1e12, 2),
                 "pingpong_gate_up_swiglu_ms": round(f3_ms, 4),
                 "speedup_over_pingpong_gate_up": round(f3_ms / c3, 4)}
    # the per-weight-update preparation, warm (no allocation: same buffers)
    blk.prepare(params)
    prep_ms = timed(lambda: blk.prepare(params), 5)

    bd = None
    if breakdown:   # per-call breakdown (one extra, untimed-for-the-metric step)
        evs = []
        torch.cuda.synchronize()
        for call, fn in calls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((call, a, b))
        torch.cuda.synchronize()
        bd = {n: round(a.elapsed_time(b), 4) for n, a, b in evs}

    unfused = None
    if not args.no_unfused and not fp8:
        ub = UnfusedBlock(params, cfg.D, cfg.F, seq_len=cfg.seq_len, theta=cfg.theta, eps=cfg.eps)
        bufs = ub.alloc(M, dev)
        for k in ("dWqkv", "dWo", "dWgu", "dWd", "dg1", "dg2", "dgq", "dgk"):
            bufs[k].zero_()

        def ustep():
            ub.forward(x, o, bufs)
            ub.backward(x, o, bufs, dY, dq, dk, dv, beta=1.0)

        for _ in range(args.warmup):
            ustep()
        ums = timed(ustep, args.steps)
        ufwd = timed(lambda: ub.forward(x, o, bufs), max(1, args.steps // 2))
        unfused = {"block_fwd_bwd_ms": round(ums, 4), "fwd_ms": round(ufwd, 4),
                   "speedup_fused_over_unfused": round(ums / ms, 4),
                   "speedup_with_weight_prep_every_step": round(ums / (ms + prep_ms), 4)}
        del ub, bufs

    fwd_fl, bwd_fl = block_flops(M, cfg.D, cfg.F)
    tflops = (fwd_fl + bwd_fl) / (ms * 1e-3) / 1e12
    f3_flop = 2 * M * (2 * cfg.F) * cfg.D
    f3_tflops = f3_flop / (f3_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[precision]
    out = {
        "workload": f"LLaMA-style non-attention block forward+backward, hidden {cfg.D}, MLP {cfg.F}, "
                    f"{cfg.heads}x128 heads, {M} tokens",
        "block_fwd_bwd_ms": round(ms, 4), "block_fwd_ms": round(fwd_ms, 4),
        "step_ms_median": round(per_step[len(per_step) // 2], 4) if per_step else None,
        "step_ms_min": round(per_step[0], 4) if per_step else None,
        "block_fwd_bwd_graph_ms": None if graph_ms is None else round(graph_ms, 4),
        "tflops": round(tflops, 2), "pct_of_peak": round(100 * tflops / peak, 2),
        "unfused_baseline": unfused,
        "weight_prep_ms": round(prep_ms, 4), "weight_prep_cold_ms": round(prep_cold_ms, 3),
        "breakdown_ms": bd,
        "roofline": {"bound": "mfma", "kernel": "gate/up GEMM + SwiGLU epilogue (M x 2F x D)",
                     "achieved": round(f3_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(f3_tflops / peak, 4), "avg_ms": round(f3_ms, 4),
                     "flop_per_launch": f3_flop, "traffic": stored_traffic(name, precision)},
        "partial_buffers": partial_bytes(M, cfg.D, cfg.F),
        "coresident_schedule": cores,
    }
    del blk, f, g, params, calls
    torch.cuda.empty_cache()
    return out, f3_tflops


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU (asked for --gpus {args.gpus}): the library has no multi-GPU path; "
              f"run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.ce_only:
        print(json.dumps({"cross_entropy": ce_leg(1, max(2, args.steps // 5))}))
        return
    import coda_inputs as ci
    cfg = {"cfg2": ci.CFG2, "cfg3": ci.CFG3, "cfg5": ci.CFG5}[args.config]
    seed = ci.SEEDS[args.config]
    precision = args.precision or ("fp8" if args.config == "cfg5" else "bf16")
    fp8 = {"bf16": False, "fp8": True, "mxfp8": "mx"}[precision]
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, seed, args.cpu_rows or cfg.M, fp8)

    import torch
    import gemm_epilogue_fp8_amd as coda
    from gemm_epilogue_fp8_amd.block import Block
    import numpy as np

    torch.cuda.set_device(0)
    head, f3_tflops = block_leg(args.config, precision, args)
    ms = head["block_fwd_bwd_ms"]
    # hidden 4096 (the size the metric names beside 2048) in the same run
    h4096 = None
    if args.config == "cfg2" and not args.no_h4096:
        h4096, _ = block_leg("cfg3", precision, args)

    small_fwd = {}
    if not args.no_mx and not fp8:
        # the same block forward (inference) with MXFP4 and MXFP6 (E2M3)
        # operands: weights quantised once, activations per call
        dev = "cuda:0"
        P = ci.block_inputs(cfg, seed)
        to = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
        params = {k: to(v, torch.float32 if k in ("g1", "g2", "gq", "gk") else torch.bfloat16) for k, v in P.items()}
        del P
        for key, prec in (("mxfp4_block_forward", coda.PREC_MXFP4), ("mxfp6_e2m3_block_forward", coda.PREC_MXFP6_E2M3)):
            blk = Block(params, cfg.D, cfg.F, seq_len=cfg.seq_len, precision=prec)
            fo = blk.alloc_forward(cfg.M, dev)
            blk.forward(params["x"], params["o"], fo)
            reps = max(1, args.steps // 2)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                blk.forward(params["x"], params["o"], fo)
            b.record()
            torch.cuda.synchronize()
            msq = a.elapsed_time(b) / reps
            small_fwd[key] = {"block_fwd_ms": round(msq, 4),
                              "tflops": round(block_flops(cfg.M, cfg.D, cfg.F)[0] / (msq * 1e-3) / 1e12, 1),
                              f"speedup_over_{precision}_fwd": round(head["block_fwd_ms"] / msq, 4)}
            del blk, fo
        del params
        torch.cuda.empty_cache()
    mx = None if args.no_mx else mx_leg(max(1, args.warmup), max(3, args.steps // 2))
    small = small_layer_leg() if args.small else None
    ce = None if args.no_ce else ce_leg(1, max(2, args.steps // 5))
    peak = PEAK_TFLOPS[precision]
    mloop = None if args.no_mfma_loop else mfma_loop_leg(f3_tflops)
    if mloop is not None and precision != "bf16":
        mloop["dominant_kernel_frac_of_achievable"] = round(f3_tflops / mloop["fp8_tflops"], 4)
    out = {
        "metric": "fused GEMM+epilogue TFLOP/s & % MFMA peak; block fwd+bwd ms, hidden 2048/4096",
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": precision,
        "data": "synthetic",
        "config": {"workload": head["workload"],
                   "tokens": cfg.M, "hidden": cfg.D, "mlp": cfg.F, "heads": cfg.heads, "head_dim": 128,
                   "seq_len": cfg.seq_len, "grad_accumulate_beta": 1.0},
        "block_fwd_bwd_ms": round(ms, 4),
        "block_fwd_ms": head["block_fwd_ms"],
        "step_ms_median": head["step_ms_median"],
        "step_ms_min": head["step_ms_min"],
        "block_fwd_bwd_graph_ms": head["block_fwd_bwd_graph_ms"],
        "pct_of_peak": head["pct_of_peak"],
        "unfused_baseline": head["unfused_baseline"],
        "weight_prep_ms": head["weight_prep_ms"],
        "weight_prep_cold_ms": head["weight_prep_cold_ms"],
        "breakdown_ms": head["breakdown_ms"],
        "roofline": head["roofline"],
        "partial_buffers": head["partial_buffers"],
        "coresident_schedule": head["coresident_schedule"],
        "hidden_4096": h4096,
        "cpu_baseline": cpu,
        "mxfp8_gemm": mx,
        "mxfp4_block_forward": small_fwd.get("mxfp4_block_forward"),
        "mxfp6_e2m3_block_forward": small_fwd.get("mxfp6_e2m3_block_forward"),
        "cross_entropy": ce,
        "mfma_loop": mloop,
        "small_swiglu_layer": small,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
