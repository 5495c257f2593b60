"""The reparameterised LLaMA-style non-attention block as a sequence of
GEMM + epilogue calls (CODA paper, arXiv 2605.19269, §3.2 and §3.2.1).

Forward (per block):
  aux   P_x = row sum-of-squares of x (stands in for the previous block's
        down-projection partials)
  F1    q, k, v = RoPE(QKnorm(r1 * (x W~qkv)))           linear_qknorm_rope_fwd
  F2    h1 = x + o Wo,  sum-of-squares partials of h1     linear_rmsnorm_residual_fwd
  F3    a = SwiGLU(r2 * (h1 W~gu))                        linear_swiglu_fwd
  F4    y = h1 + a Wd,  partials for the next norm        linear_rmsnorm_residual_fwd
Backward, given dY and the attention gradients dq, dk, dv:
  B1+B3+B4  dh1, dW_gu, dg2 (dSwiGLU fused behind dY Wd^T)  linear_swiglu_bwd
  B2        dWd                                            linear_rmsnorm_residual_bwd
  B5+B6     do, dWo                                        linear_rmsnorm_residual_bwd
  G1+B7+B8  dx, dWqkv, dg1, dgq, dgk                       linear_qknorm_rope_bwd

This module only allocates tensors and orders the library calls; every
arithmetic step runs in the HIP kernels of libcoda.so.
"""
from __future__ import annotations

from typing import Dict

import torch

from . import (PREC_BF16, PREC_FP8, PREC_MXFP4, PREC_MXFP6_E2M3, PREC_MXFP6_E3M2, PREC_MXFP8, Weight, fold_gain, linear_qknorm_rope_bwd, linear_qknorm_rope_fwd,
               linear_rmsnorm_residual_bwd, linear_rmsnorm_residual_fwd, linear_swiglu_bwd, linear_swiglu_fwd,
               pack_gate_up, partials_cols, rope_table, row_sumsq)


class Block:
    """Device weights of one block (folded, packed and, for fp8, quantised)
    and the forward / backward call sequences."""

    def __init__(self, params: Dict[str, torch.Tensor], D: int, F: int, seq_len: int = 2048,
                 theta: float = 5e5, eps: float = 1e-6, precision: int = PREC_BF16):
        dev = params["Wqkv"].device
        self.D, self.F, self.seq_len, self.eps, self.precision = D, F, seq_len, eps, precision
        bf = torch.bfloat16
        self.g1, self.g2 = params["g1"], params["g2"]
        self.gq, self.gk = params["gq"], params["gk"]
        self.Wqkv = params["Wqkv"]                        # unfolded, for the gain gradient
        self.Wqkv_t = torch.empty_like(self.Wqkv)
        self.Wgu_t = torch.empty((D, 2 * F), dtype=bf, device=dev)
        self.Wgu = torch.empty((D, 2 * F), dtype=bf, device=dev)
        self.Wo, self.Wd = params["Wo"], params["Wd"]
        self.rope = torch.empty((seq_len, 128), dtype=torch.float32, device=dev)
        self.w = {}
        self.prepare(params)

    def prepare(self, params):
        """Once per weight update: fold gains, pack gate/up, RoPE table and,
        for fp8, the two E4M3 copies of every weight."""
        fold_gain(self.Wqkv, self.g1, self.Wqkv_t)
        pack_gate_up(params["Wg"], params["Wu"], self.g2, self.Wgu_t)
        pack_gate_up(params["Wg"], params["Wu"], None, self.Wgu)
        rope_table(self.seq_len, self.rope)
        self.w = {"qkv": Weight(self.Wqkv_t), "o": Weight(self.Wo), "gu": Weight(self.Wgu_t),
                  "d": Weight(self.Wd)}
        if self.precision == PREC_FP8:
            for w in self.w.values():
                w.prepare_fp8()
        elif self.precision == PREC_MXFP8:
            for w in self.w.values():
                w.prepare_mxfp8()
        elif self.precision == PREC_MXFP4:
            for w in self.w.values():
                w.prepare_mxfp4()
        elif self.precision in (PREC_MXFP6_E2M3, PREC_MXFP6_E3M2):
            fmt = "e2m3" if self.precision == PREC_MXFP6_E2M3 else "e3m2"
            for w in self.w.values():
                w.prepare_mxfp6(fmt)

    def alloc_forward(self, M: int, device) -> Dict[str, torch.Tensor]:
        D, F = self.D, self.F
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device=device)
        return dict(P_x=e(1, M, dt=f32), q=e(M, D), k=e(M, D), v=e(M, D), qk_pre=e(M, 2 * D), r1=e(M, dt=f32),
                    h1=e(M, D), P2=e(partials_cols(D), M, dt=f32), a=e(M, F), hgu=e(M, 2 * F),
                    r2=e(M, dt=f32), y=e(M, D), P4=e(partials_cols(D), M, dt=f32))

    def forward(self, x, o, out=None):
        M = x.shape[0]
        f = out if out is not None else self.alloc_forward(M, x.device)
        p = self.precision
        row_sumsq(x, f["P_x"])
        linear_qknorm_rope_fwd(x, self.w["qkv"], self.gq, self.gk, self.rope, self.seq_len, self.eps,
                               f["q"], f["k"], f["v"], sumsq_partials=f["P_x"], save_qk_pre=f["qk_pre"],
                               r_out=f["r1"], precision=p)
        linear_rmsnorm_residual_fwd(o, self.w["o"], x, f["h1"], sumsq_partials_out=f["P2"], precision=p)
        linear_swiglu_fwd(f["h1"], self.w["gu"], self.eps, f["a"], sumsq_partials=f["P2"], save_hgu=f["hgu"],
                          r_out=f["r2"], precision=p)
        linear_rmsnorm_residual_fwd(f["a"], self.w["d"], f["h1"], f["y"], sumsq_partials_out=f["P4"], precision=p)
        return f

    def alloc_backward(self, M: int, device) -> Dict[str, torch.Tensor]:
        D, F = self.D, self.F
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device=device)
        return dict(dh1=e(M, D), dht_gu=e(M, 2 * F), dht_qkv=e(M, 3 * D), do=e(M, D), dx=e(M, D),
                    dWqkv=e(D, 3 * D, dt=f32), dWo=e(D, D, dt=f32), dWgu=e(D, 2 * F, dt=f32),
                    dWd=e(F, D, dt=f32), dg1=e(D, dt=f32), dg2=e(D, dt=f32), dgq=e(128, dt=f32),
                    dgk=e(128, dt=f32))

    def backward(self, x, o, f, dY, dq, dk, dv, grads=None, beta: float = 0.0):
        M = x.shape[0]
        b = grads if grads is not None else self.alloc_backward(M, x.device)
        p = self.precision
        linear_swiglu_bwd(dY, self.w["d"], f["hgu"], f["r2"], f["h1"], self.w["gu"], self.Wgu, self.g2,
                          dY, b["dh1"], b["dWgu"], b["dg2"], beta=beta, dh_gu_out=b["dht_gu"], precision=p)
        linear_rmsnorm_residual_bwd(dY, f["a"], self.w["d"], b["dWd"], beta=beta, precision=p)
        linear_rmsnorm_residual_bwd(b["dh1"], o, self.w["o"], b["dWo"], da=b["do"], beta=beta, precision=p)
        linear_qknorm_rope_bwd(dq, dk, dv, x, f["r1"], f["qk_pre"], f["v"], self.w["qkv"], self.Wqkv, self.g1,
                               self.gq, self.gk, self.rope, self.seq_len, self.eps, b["dh1"], b["dx"], b["dWqkv"],
                               b["dg1"], b["dgq"], b["dgk"], beta=beta, dh_qkv_out=b["dht_qkv"], precision=p)
        return b


def unpack_gate_up(t: torch.Tensor):
    """Split a packed [.., 2F] tensor (64-column blocks of 32 gate, 32 up)
    into its gate and up halves [.., F] (a view reshuffle, no arithmetic)."""
    *lead, n2 = t.shape
    v = t.reshape(*lead, n2 // 64, 2, 32)
    return v[..., 0, :].reshape(*lead, n2 // 2), v[..., 1, :].reshape(*lead, n2 // 2)
