"""Shared test helpers: tolerance checks and host/device transfers."""
from __future__ import annotations

import numpy as np

# Tolerances of the parity bar
BF16_TOL = 2e-2        # |d| <= tol (1 + |ref|) for bf16 outputs
FP8_TOL = 6e-2         # same rule for every tensor of an fp8 run
GRAD_REL = 1e-3        # norm-wise relative error of fp32 reductions / gradients
LOSS_REL = 1e-4        # relative error of the loss
# Extra, stricter check: both sides round the same fp32 values to bf16, so
# only accumulation-order ties can flip a rounding; norm-wise error stays small.
BF16_NORM_REL = 3e-3


def to_dev(a, dtype=None, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def to_np(t):
    import torch
    if t.dtype in (torch.bfloat16, torch.float8_e4m3fn):
        t = t.float()
    return t.detach().cpu().numpy()


def rel_norm(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_bf16(name, got, ref, tol=BF16_TOL, norm_rel=BF16_NORM_REL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - ref) / (1.0 + np.abs(ref))
    assert d.max() <= tol, f"{name}: max |d|/(1+|ref|) = {d.max():.3e} > {tol}"
    if norm_rel is not None:
        r = rel_norm(got, ref)
        assert r <= norm_rel, f"{name}: norm-wise relative error {r:.3e} > {norm_rel}"


def assert_grad(name, got, ref, rel=GRAD_REL):
    got = np.asarray(got, np.float64)
    assert got.shape == np.shape(ref), (name, got.shape, np.shape(ref))
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r = rel_norm(got, ref)
    assert r <= rel, f"{name}: norm-wise relative error {r:.3e} > {rel}"


def unpack_gu(a):
    """Packed [.., 2F] (64-column blocks: 32 gate, 32 up) -> (gate, up)."""
    a = np.asarray(a)
    *lead, n2 = a.shape
    v = a.reshape(*lead, n2 // 64, 2, 32)
    return v[..., 0, :].reshape(*lead, n2 // 2), v[..., 1, :].reshape(*lead, n2 // 2)
