"""HIP graph capture of the block step through the C ABI.

The library allocates, frees and synchronises nothing and launches every
kernel on the caller's stream, so a whole forward + backward step can be
captured once (torch.cuda.graph) and replayed.  Each replay here runs on new
inputs copied into the captured tensors, with eager work and
synchronisations between replays, and must reproduce the eager step bit for
bit (the kernels reduce in a fixed order); with beta = 1 the weight
gradients accumulate over the replays exactly as over eager steps.
"""
from __future__ import annotations

import numpy as np
import pytest

import coda_inputs as ci

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import gemm_epilogue_fp8_amd as coda  # noqa: E402
from gemm_epilogue_fp8_amd.block import Block  # noqa: E402

DEV = "cuda:0"
GRADS = ("dWqkv", "dWo", "dWgu", "dWd", "dg1", "dg2", "dgq", "dgk")


def _inputs(shape, seed):
    P = ci.block_inputs(shape, seed)
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV).to(
        torch.float32 if k in ("g1", "g2", "gq", "gk") else torch.bfloat16) for k, v in P.items()}


@pytest.mark.parametrize("precision", [coda.PREC_BF16, coda.PREC_FP8])
def test_block_step_graph_replay(precision):
    shape = ci.BlockShape(M=300, D=256, F=352, seq_len=128)
    params = _inputs(shape, 8)
    blk = Block(params, shape.D, shape.F, seq_len=shape.seq_len, theta=shape.theta, eps=shape.eps,
                precision=precision)
    acts = ("x", "o", "dY", "dq", "dk", "dv")
    static = {k: params[k].clone() for k in acts}
    f, g = blk.alloc_forward(shape.M, DEV), blk.alloc_backward(shape.M, DEV)
    prior = {k: torch.randn(g[k].shape, device=DEV) for k in GRADS}
    for k in GRADS:
        g[k].copy_(prior[k])

    def step(ins, fo, go):
        blk.forward(ins["x"], ins["o"], fo)
        blk.backward(ins["x"], ins["o"], fo, ins["dY"], ins["dq"], ins["dk"], ins["dv"], grads=go, beta=1.0)

    # eager warm-up on a side stream (sizes every workspace), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    scratch_f, scratch_g = blk.alloc_forward(shape.M, DEV), blk.alloc_backward(shape.M, DEV)
    with torch.cuda.stream(side):
        step(static, scratch_f, scratch_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(static, f, g)
    torch.cuda.synchronize()
    for k in GRADS:   # capture does not run the kernels
        g[k].copy_(prior[k])

    ref_f, ref_g = blk.alloc_forward(shape.M, DEV), blk.alloc_backward(shape.M, DEV)
    for k in GRADS:
        ref_g[k].copy_(prior[k])
    for rep in range(3):
        new = _inputs(shape, 100 + rep)
        for k in acts:
            static[k].copy_(new[k])
        graph.replay()
        step({k: new[k] for k in acts}, ref_f, ref_g)        # eager, same stream, same inputs
        torch.cuda.synchronize()
        for k in ref_f:
            assert torch.equal(f[k], ref_f[k]), (rep, k)
        for k in ("dh1", "dx", "do", "dht_gu", "dht_qkv") + GRADS:
            assert torch.equal(g[k], ref_g[k]), (rep, k)
