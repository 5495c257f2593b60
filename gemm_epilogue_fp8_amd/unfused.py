"""The unfused baseline block: the same GEMM mainloop with plain-store
epilogues, plus separate memory-bound kernels for every RMSNorm, residual
add, SwiGLU and QK-norm + RoPE (include/coda_unfused.h).  This is the
operator-by-operator sequence that the CODA paper (arXiv 2605.19269, §1,
§2.1) contrasts with GEMM + epilogue programs; it exists to be timed
against the fused block on the same GPU.

Only argument marshalling and call ordering here; every step runs in
libcoda.so.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict

import torch

from . import (EPI_ACCUM_F32, EPI_STORE_BF16, _check, _p, _stream, _ws_call, gemm_epi, lib,
               linear_rmsnorm_residual_bwd, pack_gate_up, rope_table)


def rmsnorm_fwd(x, g, eps, out, r_out=None):
    _check(lib().coda_unfused_rmsnorm_fwd(_p(x), _p(g), eps, _p(out), _p(r_out), _stream()))
    return out


def rmsnorm_bwd(u, g, r, dy, du, dg, dres=None, beta=0.0):
    ws, n = _ws_call(lib().coda_unfused_rmsnorm_bwd_workspace, (u.shape[0], u.shape[1]), u.device)
    _check(lib().coda_unfused_rmsnorm_bwd(_p(u), _p(g), _p(r), _p(dy), _p(dres), _p(du), _p(dg), beta, ws, n,
                                          _stream()))
    return du, dg


def add(a, b, out):
    _check(lib().coda_unfused_add(_p(a), _p(b), _p(out), _stream()))
    return out


def swiglu_fwd(h, out):
    _check(lib().coda_unfused_swiglu_fwd(_p(h), _p(out), _stream()))
    return out


def swiglu_bwd(da, h, dh):
    _check(lib().coda_unfused_swiglu_bwd(_p(da), _p(h), _p(dh), _stream()))
    return dh


def qknorm_rope_fwd(qkv, gq, gk, rope, seq_len, eps, q, k):
    _check(lib().coda_unfused_qknorm_rope_fwd(_p(qkv), _p(gq), _p(gk), _p(rope), seq_len, eps, _p(q), _p(k),
                                              _stream()))
    return q, k


def qknorm_rope_bwd(dq, dk, dv, qkv, gq, gk, rope, seq_len, eps, dqkv, dgq, dgk, beta=0.0):
    M, D3 = qkv.shape
    ws, n = _ws_call(lib().coda_unfused_qknorm_rope_bwd_workspace, (M, D3 // 3), qkv.device)
    _check(lib().coda_unfused_qknorm_rope_bwd(_p(dq), _p(dk), _p(dv), _p(qkv), _p(gq), _p(gk), _p(rope), seq_len,
                                              eps, _p(dqkv), _p(dgq), _p(dgk), beta, ws, n, _stream()))
    return dqkv, dgq, dgk


STORE = [(EPI_STORE_BF16, 0, 0.0)]


def _wgrad(a, dout, W, dW, beta):
    """dW = beta dW + a^T dout: the plain fp32-accumulate weight-gradient GEMM
    (the same kernel, token-axis split included, that the fused path uses)."""
    linear_rmsnorm_residual_bwd(dout, a, W, dW, beta=beta)


def _acc(beta):
    return [(EPI_ACCUM_F32, 0, float(beta))]


class UnfusedBlock:
    """The canonical block: RMSNorm -> GEMM -> QK-norm/RoPE, GEMM + residual
    add, RMSNorm -> GEMM -> SwiGLU, GEMM + residual add, and its backward,
    each operator a kernel of its own."""

    def __init__(self, params: Dict[str, torch.Tensor], D: int, F: int, seq_len: int = 2048, theta: float = 5e5,
                 eps: float = 1e-6):
        dev = params["Wqkv"].device
        self.D, self.F, self.seq_len, self.eps = D, F, seq_len, eps
        self.g1, self.g2, self.gq, self.gk = params["g1"], params["g2"], params["gq"], params["gk"]
        self.Wqkv, self.Wo, self.Wd = params["Wqkv"], params["Wo"], params["Wd"]
        self.Wgu = torch.empty((D, 2 * F), dtype=torch.bfloat16, device=dev)
        pack_gate_up(params["Wg"], params["Wu"], None, self.Wgu)
        self.rope = torch.empty((seq_len, 128), dtype=torch.float32, device=dev)
        rope_table(seq_len, self.rope, theta=theta)

    def alloc(self, M, device):
        D, F = self.D, self.F
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=bf: torch.empty(s, dtype=dt, device=device)
        return dict(xn1=e(M, D), r1=e(M, dt=f32), qkv=e(M, 3 * D), q=e(M, D), k=e(M, D), t=e(M, D), h1=e(M, D),
                    xn2=e(M, D), r2=e(M, dt=f32), hgu=e(M, 2 * F), a=e(M, F), y=e(M, D),
                    da=e(M, F), dhgu=e(M, 2 * F), dxn2=e(M, D), dh1=e(M, D), do=e(M, D), dqkv=e(M, 3 * D),
                    dxn1=e(M, D), dx=e(M, D),
                    dWqkv=e(D, 3 * D, dt=f32), dWo=e(D, D, dt=f32), dWgu=e(D, 2 * F, dt=f32), dWd=e(F, D, dt=f32),
                    dg1=e(D, dt=f32), dg2=e(D, dt=f32), dgq=e(128, dt=f32), dgk=e(128, dt=f32))

    def forward(self, x, o, b):
        D = self.D
        rmsnorm_fwd(x, self.g1, self.eps, b["xn1"], b["r1"])
        gemm_epi(STORE, b["xn1"], 0, self.Wqkv, 0, b["qkv"])
        qknorm_rope_fwd(b["qkv"], self.gq, self.gk, self.rope, self.seq_len, self.eps, b["q"], b["k"])
        gemm_epi(STORE, o, 0, self.Wo, 0, b["t"])
        add(x, b["t"], b["h1"])
        rmsnorm_fwd(b["h1"], self.g2, self.eps, b["xn2"], b["r2"])
        gemm_epi(STORE, b["xn2"], 0, self.Wgu, 0, b["hgu"])
        swiglu_fwd(b["hgu"], b["a"])
        gemm_epi(STORE, b["a"], 0, self.Wd, 0, b["t"])
        add(b["h1"], b["t"], b["y"])
        return b

    def backward(self, x, o, b, dY, dq, dk, dv, beta=0.0):
        D = self.D
        gemm_epi(STORE, dY, 0, self.Wd, 1, b["da"])                    # da = dY Wd^T
        _wgrad(b["a"], dY, self.Wd, b["dWd"], beta)                      # dWd = a^T dY
        swiglu_bwd(b["da"], b["hgu"], b["dhgu"])
        gemm_epi(STORE, b["dhgu"], 0, self.Wgu, 1, b["dxn2"])          # dxn2 = dh Wgu^T
        _wgrad(b["xn2"], b["dhgu"], self.Wgu, b["dWgu"], beta)           # dWgu = xn2^T dh
        rmsnorm_bwd(b["h1"], self.g2, b["r2"], b["dxn2"], b["dh1"], b["dg2"], dres=dY, beta=beta)
        gemm_epi(STORE, b["dh1"], 0, self.Wo, 1, b["do"])              # do = dh1 Wo^T
        _wgrad(o, b["dh1"], self.Wo, b["dWo"], beta)                     # dWo = o^T dh1
        qknorm_rope_bwd(dq, dk, dv, b["qkv"], self.gq, self.gk, self.rope, self.seq_len, self.eps, b["dqkv"],
                        b["dgq"], b["dgk"], beta=beta)
        gemm_epi(STORE, b["dqkv"], 0, self.Wqkv, 1, b["dxn1"])        # dxn1 = dqkv Wqkv^T
        _wgrad(b["xn1"], b["dqkv"], self.Wqkv, b["dWqkv"], beta)         # dWqkv = xn1^T dqkv
        rmsnorm_bwd(x, self.g1, b["r1"], b["dxn1"], b["dx"], b["dg1"], dres=b["dh1"], beta=beta)
        return b
