"""Canonical (unfused) Transformer operations and their analytic gradients.

Test infrastructure only.  Every function is the plain textbook definition,
written for any float dtype (the oracle runs them in float64 for its "ideal"
mode and float32 for its "contract" mode).

Sources: the CODA paper (arXiv 2605.19269), §3.1 (the five epilogue primitive
classes: maps, vector loads, tile loads, tile reductions, state transitions)
and §3.2.1 (RMSNorm written as the per-row inverse RMS factor r times the
gain); the RMSNorm, SwiGLU, RoPE and softmax cross-entropy definitions are the
standard ones that the paper's reparameterisations start from, and GELU is
the exact (error-function) form of Hendrycks and Gimpel's definition, the
second elementwise activation map beside the sigmoid.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------- RMSNorm
def inv_rms(u, eps: float):
    """r = (mean over the last axis of u^2 + eps)^(-1/2); eps sits inside the
    square root and the mean divides by the full row length."""
    u = np.asarray(u)
    ms = np.mean(u * u, axis=-1)
    return (1.0 / np.sqrt(ms + u.dtype.type(eps))).astype(u.dtype)


def rms_norm(u, g, eps: float):
    """RMSNorm(u, g) = r * u * g with r = inv_rms(u) per row."""
    r = inv_rms(u, eps)
    return u * r[..., None] * g


def rms_norm_bwd(u, g, eps: float, dy):
    """Gradients of RMSNorm given the upstream gradient dy.

    With t = g * dy and r = inv_rms(u):  du = r t - (r^3 / n) u sum(u t), and
    dg = sum over rows of r u dy.
    """
    n = u.shape[-1]
    r = inv_rms(u, eps)[..., None]
    t = g * dy
    s = np.sum(u * t, axis=-1, keepdims=True)
    du = r * t - (r ** 3 / n) * u * s
    dg = np.sum(r * u * dy, axis=tuple(range(u.ndim - 1)))
    return du, dg


# ----------------------------------------------------------------- SwiGLU
def sigmoid(t):
    one = t.dtype.type(1.0)
    return one / (one + np.exp(-t))


def sigmoid_grad(t):
    """sigmoid'(t) = s (1 - s) with s = sigmoid(t)."""
    s = sigmoid(t)
    return s * (t.dtype.type(1.0) - s)


# ----------------------------------------------------------------- GELU
def gelu(t):
    """GELU(t) = t Phi(t), Phi the standard normal CDF written through the
    error function: Phi(t) = (1 + erf(t / sqrt 2)) / 2 (the exact form, not
    the tanh approximation)."""
    t = np.asarray(t)
    half = t.dtype.type(0.5)
    return half * t * (t.dtype.type(1.0) + _erf(t / t.dtype.type(np.sqrt(2.0))))


def gelu_grad(t):
    """GELU'(t) = Phi(t) + t phi(t), phi(t) = exp(-t^2 / 2) / sqrt(2 pi)."""
    t = np.asarray(t)
    one, half = t.dtype.type(1.0), t.dtype.type(0.5)
    cdf = half * (one + _erf(t / t.dtype.type(np.sqrt(2.0))))
    pdf = np.exp(-half * t * t) / t.dtype.type(np.sqrt(2.0 * np.pi))
    return cdf + t * pdf


def _erf(t):
    from scipy.special import erf
    return erf(t).astype(t.dtype)


def silu(t):
    """SiLU(t) = t * sigmoid(t)."""
    return t * sigmoid(t)


def swiglu(hg, hu):
    """SwiGLU gating with the SiLU on the gate half: SiLU(hg) * hu."""
    return silu(hg) * hu


def swiglu_bwd(hg, hu, da):
    """d/dhg = da hu s (1 + hg (1 - s)),  d/dhu = da hg s,  with s = sigmoid(hg)."""
    one = hg.dtype.type(1.0)
    s = sigmoid(hg)
    dhg = da * hu * s * (one + hg * (one - s))
    dhu = da * hg * s
    return dhg, dhu


# ----------------------------------------------------------------- RoPE
def rope_tables(seq_len: int, head_dim: int, theta: float):
    """cos/sin tables [seq_len, head_dim/2]: angle p * theta^(-2i/head_dim) for
    position p and pair i, evaluated in float64 and stored as float32."""
    p = np.arange(seq_len, dtype=np.float64)[:, None]
    i = np.arange(head_dim // 2, dtype=np.float64)[None, :]
    ang = p * theta ** (-2.0 * i / head_dim)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope(t, positions, cos, sin, head_dim: int = 128, inverse: bool = False):
    """Rotate adjacent column pairs (2i, 2i+1) of every head by the angle of
    the row's position: (a, b) -> (a cos - b sin, a sin + b cos).  The inverse
    rotation uses the negated angle (the rotation's transpose)."""
    M, N = t.shape
    H = N // head_dim
    c = cos[positions].astype(t.dtype)[:, None, :]      # [M, 1, hd/2]
    s = sin[positions].astype(t.dtype)[:, None, :]
    if inverse:
        s = -s
    v = t.reshape(M, H, head_dim // 2, 2)
    a, b = v[..., 0], v[..., 1]
    out = np.empty_like(v)
    out[..., 0] = a * c - b * s
    out[..., 1] = a * s + b * c
    return out.reshape(M, N)


# ----------------------------------------------------------------- QK-norm
def qk_norm(t, g, eps: float, head_dim: int = 128):
    """RMSNorm over every head's head_dim columns, one gain shared by heads."""
    M, N = t.shape
    v = t.reshape(M, N // head_dim, head_dim)
    return rms_norm(v, g, eps).reshape(M, N)


def qk_norm_bwd(t, g, eps: float, dy, head_dim: int = 128):
    M, N = t.shape
    v = t.reshape(M, N // head_dim, head_dim)
    du, dg = rms_norm_bwd(v, g, eps, dy.reshape(v.shape))
    return du.reshape(M, N), dg


# ----------------------------------------------------------------- cross-entropy
def logsumexp_rows(z):
    m = np.max(z, axis=1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=1, keepdims=True)))[:, 0]


def cross_entropy(z, labels, ignore_index: int = -100):
    """Mean softmax cross-entropy over the rows whose label is not ignored.

    Returns (loss, per-row loss (0 on ignored rows), lse, n_valid, dz) where
    dz = (softmax(z) - onehot(label)) / n_valid on valid rows and 0 elsewhere.
    With n_valid = 0 the loss is 0/0 = NaN and dz is 0.  A label outside
    [0, V) that is not the ignore index raises ValueError.
    """
    M, V = z.shape
    labels = np.asarray(labels)
    valid = labels != ignore_index
    if np.any(valid & ((labels < 0) | (labels >= V))):
        raise ValueError("label outside [0, V) that is not the ignore index")
    lse = logsumexp_rows(z)
    rows = np.nonzero(valid)[0]
    zy = np.zeros(M, dtype=z.dtype)
    zy[rows] = z[rows, labels[rows]]
    per_row = np.where(valid, lse - zy, z.dtype.type(0))
    n_valid = int(valid.sum())
    with np.errstate(invalid="ignore", divide="ignore"):
        loss = z.dtype.type(np.sum(per_row[valid])) / z.dtype.type(n_valid)
    dz = np.exp(z - lse[:, None])
    dz[rows, labels[rows]] -= 1
    dz[~valid] = 0
    if n_valid > 0:
        dz = dz / z.dtype.type(n_valid)
    return loss, per_row, lse, n_valid, dz
