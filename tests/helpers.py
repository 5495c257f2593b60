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


def amax_flip_rows(pairs):
    """Rows where the row amax of a tensor that feeds an E4M3 row quantiser
    differs between the two sides.  Both sides materialise that tensor in
    bf16 from fp32 sums taken in different orders, so a rare element moves by
    one ulp; when it is the row's amax, every code of the row moves with it."""
    rows = set()
    for got, ref in pairs:
        g = np.abs(np.asarray(got, np.float64)).max(axis=1)
        r = np.abs(np.asarray(ref, np.float64)).max(axis=1)
        rows |= set(np.nonzero(g != r)[0].tolist())
    return np.array(sorted(rows), dtype=np.int64)


def assert_fp8_rows(name, got, ref, flagged, tol=FP8_TOL, flagged_tol=0.25, norm_rel=2e-2):
    """The elementwise fp8 bound on every row whose quantiser inputs agree on
    both sides; rows in `flagged` (an upstream amax moved by one ulp) only
    need |d| <= flagged_tol (1 + |ref|)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - ref) / (1.0 + np.abs(ref))
    keep = np.ones(got.shape[0], bool)
    keep[flagged] = False
    if keep.any():
        assert d[keep].max() <= tol, f"{name}: max |d|/(1+|ref|) = {d[keep].max():.3e} > {tol} on unflagged rows"
    if not keep.all():
        assert d[~keep].max() <= flagged_tol, f"{name}: flagged rows reach {d[~keep].max():.3e}"
    r = rel_norm(got, ref)
    assert r <= norm_rel, f"{name}: norm-wise relative error {r:.3e} > {norm_rel}"


def amax_flip_cols(pairs):
    """Columns where the column amax (over rows) differs between the two
    sides: the E4M3 column quantisers of a weight-gradient GEMM's operands."""
    return amax_flip_rows([(np.asarray(g).T, np.asarray(r).T) for g, r in pairs])


def assert_fp8_grad(name, got, ref, flag_rows, flag_cols, tol=FP8_TOL, flagged_tol=0.5, norm_rel=2e-2):
    """The fp8 bound on every gradient element whose row and column quantisers
    saw the same amax on both sides; elements in a flagged row or column only
    need |d| <= flagged_tol (1 + |ref|).  A vector gradient is one row."""
    got = np.atleast_2d(np.asarray(got, np.float64))
    ref = np.atleast_2d(np.asarray(ref, np.float64))
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - ref) / (1.0 + np.abs(ref))
    keep = np.ones(got.shape, bool)
    keep[np.asarray(flag_rows, np.int64), :] = False
    keep[:, np.asarray(flag_cols, np.int64)] = False
    if keep.any():
        assert d[keep].max() <= tol, f"{name}: max |d|/(1+|ref|) = {d[keep].max():.3e} > {tol} on unflagged elements"
    if not keep.all():
        assert d[~keep].max() <= flagged_tol, f"{name}: flagged elements reach {d[~keep].max():.3e}"
    r = rel_norm(got, ref)
    assert r <= norm_rel, f"{name}: norm-wise relative error {r:.3e} > {norm_rel}"


def unpack_gu(a):
    """Packed [.., 2F] (64-column blocks: 32 gate, 32 up) -> (gate, up)."""
    a = np.asarray(a)
    *lead, n2 = a.shape
    v = a.reshape(*lead, n2 // 64, 2, 32)
    return v[..., 0, :].reshape(*lead, n2 // 2), v[..., 1, :].reshape(*lead, n2 // 2)
