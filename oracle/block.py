"""Oracle for the LLaMA-style non-attention block, the fused RMSNorm -> Linear ->
SwiGLU op, and linear + cross-entropy.

Test infrastructure only (imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path).

Two evaluations of every path:

* ``*_canonical``: the unfused textbook sequence (RMSNorm, then GEMM, then
  SwiGLU, residual, QK-norm, RoPE, softmax cross-entropy) and its analytic
  gradients.  Run in float64 without rounding this is the "ideal" result;
  with bf16 rounding of every operator output it is the operator-by-operator
  pipeline that the unfused baseline implements.

* ``*_contract``: the reparameterised sequence of the CODA paper, §3.2.1: the
  identity RMSNorm(xW0 + z, g) W1 = (r (xW0 + z) * g) W1, with the per-row
  factor r moved behind the second GEMM (the "delayed r" of the KuCoin news
  summary of CODA, section on the epilogue) and the gain g folded into the
  weight, W~ = diag(g) W.  It rounds to bf16 (or quantises to E4M3) exactly at
  the tensors that the fused GPU path materialises, and keeps everything
  else in float32 with float32 GEMM accumulation.  With the rounding
  functions replaced by the identity and float64 data it must agree with the
  canonical evaluation to rounding level; the tests pin that.

The backward of the reparameterised form (the paper, §3.2, states that a
tile-local forward keeps the GEMM-epilogue structure in the backward; the
formulas themselves are derived here) with dh~ = r * dh and h = r (u W~):
    dW  = g * (u^T dh~)          (row scale of the weight-gradient tile)
    dg  = sum_n W * (u^T dh~)    (row reduction of the same tile)
    du  = dh~ W~^T - (r T / D) u,  T = sum_j dh~_j h_j   (per-row)
"""
from __future__ import annotations

from typing import Callable, Dict, Optional

import numpy as np

from . import mx
from . import mx_small
from . import numerics as nm
from . import ops


def _ident(x):
    return x


# --------------------------------------------------------------------------- GEMM
def mm(A, B, fp8=False):
    """A @ B with float32 (or float64) accumulation.

    With fp8 = True, each operand is quantised to E4M3 with one scale per index
    of its non-contracted axis (per row of A, per column of B) and the product
    is dequantised as (QA @ QB) * s_A[m] * s_B[n].

    With fp8 = "mx", each operand is quantised to MXFP8 (E4M3 elements, one
    E8M0 scale per 32 consecutive values of the contracted axis K: along the
    rows of A and down the columns of B; OCP Microscaling Formats v1.0) and the
    product of the dequantised operands is taken in float64, then float32.

    With fp8 = "mx4", the same with MXFP4 operands (E2M1 elements,
    oracle/mx_small.py), and with fp8 = "mx6_e2m3" / "mx6_e3m2" with MXFP6
    operands of that element format.
    """
    small = {"mx4": "e2m1", "mx6_e2m3": "e2m3", "mx6_e3m2": "e3m2"}
    if fp8 in small:
        fmt = small[fp8]
        PA, eA = mx_small.quantize(np.asarray(A, np.float32), fmt)
        PB, eB = mx_small.quantize(np.ascontiguousarray(np.asarray(B, np.float32).T), fmt)
        return mx_small.matmul_nt(PA, eA, PB, eB).astype(np.float32)
    if fp8 == "mx":
        PA, eA = mx.quantize(np.asarray(A, np.float32))
        PB, eB = mx.quantize(np.ascontiguousarray(np.asarray(B, np.float32).T))
        return mx.matmul_nt(PA, eA, PB, eB).astype(np.float32)
    if not fp8:
        return np.matmul(A, B)
    QA, sA = nm.quantize_e4m3(A, axis=1)
    QB, sB = nm.quantize_e4m3(B, axis=0)
    acc = np.matmul(QA, QB).astype(np.float32)
    return (acc * sA[:, None]).astype(np.float32) * sB[None, :]


# --------------------------------------------------------------------------- config 1
def swiglu_forward_canonical(x, g, Wg, Wu, eps):
    xn = ops.rms_norm(x, g, eps)
    return ops.swiglu(xn @ Wg, xn @ Wu)


def swiglu_forward_contract(x, g, Wg, Wu, eps, rnd: Callable = nm.bf16):
    """r (x W~g), r (x W~u) then SiLU(gate) * up, output rounded once."""
    x = np.asarray(x)
    Wg_t = rnd(g[:, None] * Wg)
    Wu_t = rnd(g[:, None] * Wu)
    r = ops.inv_rms(x, eps)[:, None]
    hg = r * mm(x, Wg_t)
    hu = r * mm(x, Wu_t)
    return rnd(ops.swiglu(hg, hu))


# --------------------------------------------------------------------------- block
def _positions(M, seq_len):
    return np.arange(M) % seq_len


def block_forward_canonical(P: Dict[str, np.ndarray], shape, dt=np.float64, rnd: Callable = _ident):
    """Unfused block forward: pre-norm QKV (with QK-norm and RoPE on q, k),
    O-projection with residual, pre-norm gate/up with SwiGLU, down-projection
    with residual.  ``o`` stands in for the attention output.

    ``rnd`` rounds the output of every operator (identity: the ideal
    evaluation; bf16 with float32 data: the operator-by-operator bf16
    pipeline, where each norm, GEMM, activation and residual add writes its
    result to memory)."""
    c = {k: np.asarray(v, dtype=dt) for k, v in P.items() if k != "labels"}
    D, hd, eps = shape.D, shape.head_dim, shape.eps
    cos, sin = ops.rope_tables(shape.seq_len, hd, shape.theta)
    pos = _positions(c["x"].shape[0], shape.seq_len)
    xn1 = rnd(ops.rms_norm(c["x"], c["g1"], eps))
    qkv = rnd(xn1 @ c["Wqkv"])
    q_pre, k_pre, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
    q = rnd(ops.rope(ops.qk_norm(q_pre, c["gq"], eps, hd), pos, cos, sin, hd))
    k = rnd(ops.rope(ops.qk_norm(k_pre, c["gk"], eps, hd), pos, cos, sin, hd))
    h1 = rnd(c["x"] + rnd(c["o"] @ c["Wo"]))
    xn2 = rnd(ops.rms_norm(h1, c["g2"], eps))
    hg, hu = rnd(xn2 @ c["Wg"]), rnd(xn2 @ c["Wu"])
    a = rnd(ops.swiglu(hg, hu))
    y = rnd(h1 + rnd(a @ c["Wd"]))
    return dict(q=q, k=k, v=v, q_pre=q_pre, k_pre=k_pre, h1=h1, xn1=xn1, xn2=xn2,
                hg=hg, hu=hu, a=a, y=y, sumsq_y=np.sum(y * y, axis=1))


def block_backward_canonical(P, F, shape, dt=np.float64, rnd: Callable = _ident):
    """Analytic gradients of block_forward_canonical given dY (for y) and
    dq, dk, dv (for the post-RoPE q, k and for v).  ``rnd`` rounds every
    activation gradient an operator writes (weight and gain gradients are
    never rounded)."""
    c = {k: np.asarray(v, dtype=dt) for k, v in P.items()}
    D, hd, eps = shape.D, shape.head_dim, shape.eps
    cos, sin = ops.rope_tables(shape.seq_len, hd, shape.theta)
    pos = _positions(c["x"].shape[0], shape.seq_len)
    dY = c["dY"]
    da = rnd(dY @ c["Wd"].T)
    dWd = F["a"].T @ dY
    dhg, dhu = ops.swiglu_bwd(F["hg"], F["hu"], da)
    dhg, dhu = rnd(dhg), rnd(dhu)
    dxn2 = rnd(dhg @ c["Wg"].T + dhu @ c["Wu"].T)
    dWg, dWu = F["xn2"].T @ dhg, F["xn2"].T @ dhu
    du2, dg2 = ops.rms_norm_bwd(F["h1"], c["g2"], eps, dxn2)
    dh1 = rnd(dY + du2)
    do = rnd(dh1 @ c["Wo"].T)
    dWo = c["o"].T @ dh1
    dqn = ops.rope(c["dq"], pos, cos, sin, hd, inverse=True)
    dkn = ops.rope(c["dk"], pos, cos, sin, hd, inverse=True)
    dq_pre, dgq = ops.qk_norm_bwd(F["q_pre"], c["gq"], eps, dqn, hd)
    dk_pre, dgk = ops.qk_norm_bwd(F["k_pre"], c["gk"], eps, dkn, hd)
    dqkv = rnd(np.concatenate([dq_pre, dk_pre, c["dv"]], axis=1))
    dxn1 = rnd(dqkv @ c["Wqkv"].T)
    dWqkv = F["xn1"].T @ dqkv
    du1, dg1 = ops.rms_norm_bwd(c["x"], c["g1"], eps, dxn1)
    dx = rnd(dh1 + du1)
    return dict(dx=dx, do=do, dWqkv=dWqkv, dWo=dWo, dWg=dWg, dWu=dWu, dWd=dWd,
                dg1=dg1, dg2=dg2, dgq=dgq, dgk=dgk)


def block_forward_contract(P, shape, fp8: bool = False, rnd: Callable = nm.bf16,
                           dt=np.float32):
    """Reparameterised block forward with the fused path's rounding points.

    Materialised (rounded) tensors: the folded weights W~, q, k, v, the saved
    pre-norm q_pre/k_pre, h1, the saved SwiGLU inputs hg/hu, a and y.  The
    QK-norm statistics come from the unrounded q_pre/k_pre of the same
    epilogue; r2 comes from the stored h1; the next-norm sum of squares from
    the stored y.
    """
    c = {k: np.asarray(v, dtype=dt) for k, v in P.items()}
    D, hd, eps = shape.D, shape.head_dim, shape.eps
    M = c["x"].shape[0]
    cos, sin = ops.rope_tables(shape.seq_len, hd, shape.theta)
    pos = _positions(M, shape.seq_len)
    W = fold_weights(c, rnd)
    x, o = c["x"], c["o"]
    r1 = ops.inv_rms(x, eps)
    t = r1[:, None] * mm(x, W["Wqkv_t"], fp8)
    q32, k32, v32 = t[:, :D], t[:, D:2 * D], t[:, 2 * D:]
    q = rnd(ops.rope(ops.qk_norm(q32, c["gq"], eps, hd), pos, cos, sin, hd))
    k = rnd(ops.rope(ops.qk_norm(k32, c["gk"], eps, hd), pos, cos, sin, hd))
    h1 = rnd(x + mm(o, c["Wo"], fp8))
    r2 = ops.inv_rms(h1, eps)
    hg = r2[:, None] * mm(h1, W["Wg_t"], fp8)
    hu = r2[:, None] * mm(h1, W["Wu_t"], fp8)
    a = rnd(ops.swiglu(hg, hu))
    y = rnd(h1 + mm(a, c["Wd"], fp8))
    return dict(q=q, k=k, v=rnd(v32), q_pre=rnd(q32), k_pre=rnd(k32), h1=h1,
                hg=rnd(hg), hu=rnd(hu), a=a, y=y, r1=r1, r2=r2,
                sumsq_y=np.sum(y * y, axis=1, dtype=dt), **W)


def fold_weights(c, rnd: Callable = nm.bf16):
    """W~ = diag(g) W rounded once, for every GEMM that consumes an RMSNorm."""
    return dict(Wqkv_t=rnd(c["g1"][:, None] * c["Wqkv"]),
                Wg_t=rnd(c["g2"][:, None] * c["Wg"]),
                Wu_t=rnd(c["g2"][:, None] * c["Wu"]))


def block_backward_contract(P, F, shape, fp8: bool = False, rnd: Callable = nm.bf16,
                            dt=np.float32, priors: Optional[Dict[str, np.ndarray]] = None,
                            beta: float = 0.0):
    """Reparameterised block backward with the fused path's rounding points.

    Materialised (rounded) tensors: dh~_gu = r2 [dhg, dhu], dh1, do,
    dh~_qkv = r1 [dq_pre, dk_pre, dv] and dx.  Statistics T2 and T1 use the
    rounded dh~ and the saved (rounded) pre-activations.  Gradients are never
    rounded; with ``priors`` the weight and gain gradients are accumulated as
    beta * prior + new.
    """
    c = {k: np.asarray(v, dtype=dt) for k, v in P.items()}
    D, hd, eps = shape.D, shape.head_dim, shape.eps
    M = c["x"].shape[0]
    cos, sin = ops.rope_tables(shape.seq_len, hd, shape.theta)
    pos = _positions(M, shape.seq_len)
    x, o, dY = c["x"], c["o"], c["dY"]
    r1, r2 = F["r1"][:, None], F["r2"][:, None]
    # down-projection and SwiGLU backward
    da = mm(dY, c["Wd"].T, fp8)
    dWd = mm(F["a"].T, dY, fp8)
    dhg, dhu = ops.swiglu_bwd(F["hg"], F["hu"], da)
    dht_gu = rnd(r2 * np.concatenate([dhg, dhu], axis=1))
    h_gu = np.concatenate([F["hg"], F["hu"]], axis=1)
    T2 = np.sum(dht_gu * h_gu, axis=1, dtype=dt)[:, None]
    c2 = r2 * T2 / dt(D)
    W_gu_t = np.concatenate([F["Wg_t"], F["Wu_t"]], axis=1)
    dh1 = rnd(mm(dht_gu, W_gu_t.T, fp8) - c2 * F["h1"] + dY)
    acc_gu = mm(F["h1"].T, dht_gu, fp8)
    Fw = c["Wg"].shape[1]
    acc_g, acc_u = acc_gu[:, :Fw], acc_gu[:, Fw:]
    g2 = c["g2"][:, None]
    dWg, dWu = g2 * acc_g, g2 * acc_u
    dg2 = np.sum(c["Wg"] * acc_g, axis=1, dtype=dt) + np.sum(c["Wu"] * acc_u, axis=1, dtype=dt)
    # O-projection backward
    do = rnd(mm(dh1, c["Wo"].T, fp8))
    dWo = mm(o.T, dh1, fp8)
    # glue: inverse RoPE, QK-norm backward, r1 scale
    dqn = ops.rope(c["dq"], pos, cos, sin, hd, inverse=True)
    dkn = ops.rope(c["dk"], pos, cos, sin, hd, inverse=True)
    dq_pre, dgq = ops.qk_norm_bwd(F["q_pre"], c["gq"], eps, dqn, hd)
    dk_pre, dgk = ops.qk_norm_bwd(F["k_pre"], c["gk"], eps, dkn, hd)
    dht_qkv = rnd(r1 * np.concatenate([dq_pre, dk_pre, c["dv"]], axis=1))
    h_qkv = np.concatenate([F["q_pre"], F["k_pre"], F["v"]], axis=1)
    T1 = np.sum(dht_qkv * h_qkv, axis=1, dtype=dt)[:, None]
    c1 = r1 * T1 / dt(D)
    dx = rnd(mm(dht_qkv, F["Wqkv_t"].T, fp8) - c1 * x + dh1)
    acc_qkv = mm(x.T, dht_qkv, fp8)
    dWqkv = c["g1"][:, None] * acc_qkv
    dg1 = np.sum(c["Wqkv"] * acc_qkv, axis=1, dtype=dt)
    out = dict(dx=dx, do=do, dWqkv=dWqkv, dWo=dWo, dWg=dWg, dWu=dWu, dWd=dWd,
               dg1=dg1, dg2=dg2, dgq=dgq, dgk=dgk,
               dht_gu=dht_gu, dh1=dh1, dht_qkv=dht_qkv, T1=T1[:, 0], T2=T2[:, 0])
    if priors:
        for key, prior in priors.items():
            out[key] = dt(beta) * np.asarray(prior, dtype=dt) + out[key]
    return out


# --------------------------------------------------------------------------- CE
def ce_forward_contract(h, W, labels, ignore_index=-100, fp8: bool = False):
    """z = h W in float32; lse, per-row loss and the mean over valid rows are
    reduced in float64 from the float32 logits and returned as float32."""
    z = mm(np.asarray(h, np.float32), np.asarray(W, np.float32), fp8)
    loss, per_row, lse, n_valid, _ = ops.cross_entropy(z.astype(np.float64), labels, ignore_index)
    return dict(loss=np.float32(loss), per_row=per_row.astype(np.float32),
                lse=lse.astype(np.float32), n_valid=n_valid, z=z)


def ce_backward_contract(h, W, labels, lse, n_valid, dloss=1.0, ignore_index=-100,
                         rnd: Callable = nm.bf16, fp8: bool = False,
                         dW_prior=None, beta: float = 0.0):
    """G = bf16(exp(z - lse) - onehot(label)) on valid rows, those whose label
    lies in [0, V) (0 on ignored rows and on rows with a label out of range,
    which the forward leaves out of the mean), then dh = rnd(s * G W^T) and
    dW = beta * prior + s * h^T G with the float32 scale s = dloss / n_valid."""
    h = np.asarray(h, np.float32)
    W = np.asarray(W, np.float32)
    labels = np.asarray(labels)
    z = mm(h, W, fp8)
    valid = (labels >= 0) & (labels < W.shape[1])
    p = np.exp(z - np.asarray(lse, np.float32)[:, None]).astype(np.float32)
    rows = np.nonzero(valid)[0]
    p[rows, labels[rows]] -= np.float32(1.0)
    p[~valid] = 0
    G = rnd(p)
    s = np.float32(dloss) / np.float32(max(n_valid, 1)) if n_valid > 0 else np.float32(0)
    dh = rnd(s * mm(G, W.T, fp8))
    dW = s * mm(h.T, G, fp8)
    if dW_prior is not None:
        dW = np.float32(beta) * dW_prior + dW
    return dict(G=G, dh=dh, dW=dW, scale=s)


# --------------------------------------------------------------------------- RMSNorm -> Linear -> sigmoid
# A pre-norm sigmoid layer h = RMSNorm(x, g) W, a = sigmoid(h), read by a
# consumer linear a Wn whose output joins the residual stream: the elementwise
# map of the CODA paper's §3.1 item 1 in place of SwiGLU.  The same layer with
# a = GELU(h) (act="gelu") is the second elementwise activation.
_ACTS = {"sigmoid": (ops.sigmoid, ops.sigmoid_grad), "gelu": (ops.gelu, ops.gelu_grad)}


def sigmoid_layer_canonical(x, g, W, Wn, dY, eps, dres=None, dt=np.float64, act: str = "sigmoid"):
    """Canonical evaluation and gradients: given dY = dL/d(a Wn), da = dY Wn^T,
    dh = da act'(h), dxn = dh W^T, dW = xn^T dh, then the RMSNorm backward
    for (dx, dg); dx also receives dres.  act is "sigmoid" or "gelu"."""
    x, g, W, Wn, dY = (np.asarray(t, dt) for t in (x, g, W, Wn, dY))
    f, df = _ACTS[act]
    xn = ops.rms_norm(x, g, eps)
    h = xn @ W
    a = f(h)
    da = dY @ Wn.T
    dh = da * a * (dt(1) - a) if act == "sigmoid" else da * df(h)
    dx, dg = ops.rms_norm_bwd(x, g, eps, dh @ W.T)
    if dres is not None:
        dx = dx + np.asarray(dres, dt)
    return dict(h=h, a=a, dx=dx, dW=xn.T @ dh, dg=dg)


def sigmoid_forward_contract(x, g, W, eps, fp8: bool = False, rnd: Callable = nm.bf16, dt=np.float32,
                             act: str = "sigmoid"):
    """W~ = rnd(g W), r = inv_rms(x), h = r (x W~); stored a = rnd(act(h))
    and the saved pre-activation rnd(h)."""
    x = np.asarray(x, dt)
    Wt = rnd(np.asarray(g, dt)[:, None] * np.asarray(W, dt))
    r = ops.inv_rms(x, eps)
    h = r[:, None] * mm(x, Wt, fp8)
    return dict(a=rnd(_ACTS[act][0](h)), h=rnd(h), r=r, Wt=Wt)


def sigmoid_backward_contract(x, g, W, Wn, dY, F, eps, dres=None, fp8: bool = False, rnd: Callable = nm.bf16,
                              priors=None, beta: float = 0.0, dt=np.float32, act: str = "sigmoid"):
    """With the saved h: dh~ = rnd(r (dY Wn^T) act'(h)) (for the sigmoid
    act'(h) = s (1 - s), s = sigmoid(h)), T = sum_j dh~ h,
    dx = rnd(dh~ W~^T - (r T / D) x + dres),
    dW = beta prior + g (x^T dh~), dg = beta prior + sum_n W (x^T dh~)."""
    x, g, W, Wn, dY = (np.asarray(t, dt) for t in (x, g, W, Wn, dY))
    r = np.asarray(F["r"], dt)[:, None]
    h = np.asarray(F["h"], dt)
    if act == "sigmoid":
        s = ops.sigmoid(h)
        dht = rnd(r * mm(dY, Wn.T, fp8) * s * (dt(1) - s))
    else:
        dht = rnd(r * mm(dY, Wn.T, fp8) * _ACTS[act][1](h))
    T = np.sum(dht * h, axis=1, dtype=dt)[:, None]
    dx = mm(dht, F["Wt"].T, fp8) - r * T / dt(x.shape[1]) * x
    if dres is not None:
        dx = dx + np.asarray(dres, dt)
    acc = mm(x.T, dht, fp8)
    dW = g[:, None] * acc
    dg = np.sum(W * acc, axis=1, dtype=dt)
    if priors is not None:
        dW = dt(beta) * priors["dW"] + dW
        dg = dt(beta) * priors["dg"] + dg
    return dict(dht=dht, dx=rnd(dx), dW=dW, dg=dg, T=T[:, 0])


# --------------------------------------------------------------------------- final RMSNorm -> LM head -> CE
# The third occurrence of the GEMM-residual-RMSNorm-GEMM pattern in the CODA
# paper (§3.2.1, final down-projection -> residual -> final RMSNorm -> LM
# head): the norm's r becomes a row scale of the logits, the gain folds into
# W_vocab, and the loss is the cross-entropy above.
def norm_ce_canonical(y, g, W, labels, eps, ignore_index=-100, dres=None, dt=np.float64):
    """Canonical evaluation: xn = RMSNorm(y, g), z = xn W, mean cross-entropy
    over the rows whose label is not ignored, and the analytic gradients
    dz (softmax - onehot) / n_valid, dxn = dz W^T, dW = xn^T dz, then the
    RMSNorm backward for (dy, dg); dy also receives the residual-stream
    gradient dres when given."""
    y = np.asarray(y, dt)
    g = np.asarray(g, dt)
    W = np.asarray(W, dt)
    xn = ops.rms_norm(y, g, eps)
    z = xn @ W
    loss, per_row, lse, n_valid, dz = ops.cross_entropy(z, labels, ignore_index)
    dxn = dz @ W.T
    dW = xn.T @ dz
    dy, dg = ops.rms_norm_bwd(y, g, eps, dxn)
    if dres is not None:
        dy = dy + np.asarray(dres, dt)
    return dict(loss=loss, per_row=per_row, lse=lse, n_valid=n_valid, z=z, dy=dy, dW=dW, dg=dg)


def norm_ce_forward_contract(y, g, W, labels, eps, ignore_index=-100, rnd: Callable = nm.bf16, dt=np.float32):
    """Reparameterised forward: W~ = rnd(g W), r = inv_rms(y), z = r (y W~);
    lse, per-row loss and the mean are reduced in float64 from z."""
    y = np.asarray(y, dt)
    Wt = rnd(np.asarray(g, dt)[:, None] * np.asarray(W, dt))
    r = ops.inv_rms(y, eps)
    z = r[:, None] * mm(y, Wt)
    loss, per_row, lse, n_valid, _ = ops.cross_entropy(z.astype(np.float64), labels, ignore_index)
    return dict(loss=np.float32(loss) if dt == np.float32 else loss, per_row=per_row.astype(dt),
                lse=lse.astype(dt), n_valid=n_valid, z=z, r=r, Wt=Wt)


def norm_ce_backward_contract(y, g, W, labels, lse, r, n_valid, eps, dloss=1.0, ignore_index=-100,
                              rnd: Callable = nm.bf16, dres=None, priors=None, beta: float = 0.0, dt=np.float32):
    """Reparameterised backward with the fused path's rounding points.

    z is recomputed as r (y W~).  The stored gradient tile is
    G~ = rnd(r (exp(z - lse) - onehot)) on valid rows (label in [0, V); 0 on
    every other row);
    with s = dloss / n_valid (float32) and T = s sum_v G~ z (from the stored
    G~), dy = rnd(s G~ W~^T - (r T / D) y + dres), dW = beta prior +
    s g (y^T G~) and dg = beta prior + s sum_v W (y^T G~).
    """
    y = np.asarray(y, dt)
    g = np.asarray(g, dt)
    W = np.asarray(W, dt)
    Wt = rnd(g[:, None] * W)
    labels = np.asarray(labels)
    r = np.asarray(r, dt)
    z = r[:, None] * mm(y, Wt)
    valid = (labels >= 0) & (labels < W.shape[1])     # ignored and out-of-range rows get 0
    p = np.exp(z - np.asarray(lse, dt)[:, None]).astype(dt)
    rows = np.nonzero(valid)[0]
    p[rows, labels[rows]] -= dt(1.0)
    p[~valid] = 0
    Gt = rnd(r[:, None] * p)
    s = dt(dloss) / dt(max(n_valid, 1)) if n_valid > 0 else dt(0)
    T = s * np.sum(Gt * z, axis=1, dtype=dt)
    D = y.shape[1]
    dy = s * mm(Gt, Wt.T) - (r * T / dt(D))[:, None] * y
    if dres is not None:
        dy = dy + np.asarray(dres, dt)
    dy = rnd(dy)
    acc = mm(y.T, Gt)
    dW = s * (g[:, None] * acc)
    dg = s * np.sum(W * acc, axis=1, dtype=dt)
    if priors is not None:
        dW = dt(beta) * priors["dW"] + dW
        dg = dt(beta) * priors["dg"] + dg
    return dict(G=Gt, dy=dy, dW=dW, dg=dg, T=T, scale=s)


def tile_partials(values, BN: int, reduce: Callable = np.sum):
    """Per-(column tile, row) partial reductions P[t, i] over columns
    [t BN, (t+1) BN) of ``values`` (the ragged last tile is shorter)."""
    M, N = values.shape
    nt = (N + BN - 1) // BN
    return np.stack([reduce(values[:, t * BN:(t + 1) * BN], axis=1) for t in range(nt)])
