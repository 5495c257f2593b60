"""Pins for the oracle's canonical operations (CPU only): brute-force loops on
tiny shapes, closed forms, invariants, central finite differences and torch's
CPU float64 routines."""
import math

import numpy as np
import pytest
import torch

from oracle import ops
from oracle.block import mm, tile_partials


def _fd(f, x, eps=1e-6):
    """Central finite-difference gradient of a scalar function."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f(x)
        x[i] = old - eps
        fm = f(x)
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_matmul_against_triple_loop():
    rng = np.random.default_rng(0)
    A = rng.standard_normal((5, 7)).astype(np.float32)
    B = rng.standard_normal((7, 3)).astype(np.float32)
    ref = [[sum(float(A[i, k]) * float(B[k, j]) for k in range(7)) for j in range(3)] for i in range(5)]
    got = mm(A, B)
    assert got.shape == (5, 3)
    np.testing.assert_allclose(got, np.array(ref), rtol=7 * 2 ** -23 * 4, atol=1e-6)


def test_rms_norm_closed_forms():
    c, eps = 3.0, 1e-6
    u = np.full((1, 16), c)
    g = np.linspace(0.5, 2.0, 16)
    np.testing.assert_allclose(ops.rms_norm(u, g, eps), c / math.sqrt(c * c + eps) * g[None], rtol=1e-14)
    rng = np.random.default_rng(1)
    u = rng.standard_normal((4, 32))
    xn = ops.rms_norm(u, np.ones(32), 0.0)
    np.testing.assert_allclose(np.mean(xn * xn, axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(ops.rms_norm(7.5 * u, g[:1].repeat(32), 0.0),
                               ops.rms_norm(u, g[:1].repeat(32), 0.0), rtol=1e-13)
    r = ops.inv_rms(u, eps)
    for i in range(4):
        ms = sum(float(v) ** 2 for v in u[i]) / 32
        assert abs(r[i] - 1 / math.sqrt(ms + eps)) < 1e-14


def test_rms_norm_bwd_fd_and_torch():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((3, 8))
    g = 1 + 0.1 * rng.standard_normal(8)
    dy = rng.standard_normal((3, 8))
    eps = 1e-6
    du, dg = ops.rms_norm_bwd(u, g, eps, dy)
    np.testing.assert_allclose(du, _fd(lambda v: np.sum(ops.rms_norm(v, g, eps) * dy), u.copy()), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dg, _fd(lambda w: np.sum(ops.rms_norm(u, w, eps) * dy), g.copy()), rtol=1e-6, atol=1e-8)
    tu = torch.tensor(u, requires_grad=True)
    tg = torch.tensor(g, requires_grad=True)
    y = torch.nn.functional.rms_norm(tu, (8,), tg, eps)
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(du, tu.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ops.rms_norm(u, g, eps), y.detach().numpy(), rtol=1e-13)


def test_silu_swiglu():
    t = np.array([0.0, 50.0, -50.0, 1.0])
    s = ops.silu(t)
    assert s[0] == 0 and abs(s[1] - 50) < 1e-12 and abs(s[2]) < 1e-18
    assert abs(s[3] - 1 / (1 + math.exp(-1))) < 1e-15
    # SiLU'(0) = 1/2
    d = (ops.silu(np.array([1e-6])) - ops.silu(np.array([-1e-6]))) / 2e-6
    assert abs(d[0] - 0.5) < 1e-9
    rng = np.random.default_rng(4)
    hg, hu, da = rng.standard_normal((3, 2, 5)) * 2
    dhg, dhu = ops.swiglu_bwd(hg, hu, da)
    np.testing.assert_allclose(dhg, _fd(lambda v: np.sum(ops.swiglu(v, hu) * da), hg.copy()), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(dhu, _fd(lambda v: np.sum(ops.swiglu(hg, v) * da), hu.copy()), rtol=1e-6, atol=1e-9)
    th = torch.tensor(hg)
    np.testing.assert_allclose(ops.swiglu(hg, hu), (torch.nn.functional.silu(th) * torch.tensor(hu)).numpy(), rtol=1e-14)


def test_rope_tables_values():
    cos, sin = ops.rope_tables(2048, 128, 5e5)
    assert cos.shape == (2048, 64) and cos.dtype == np.float32
    assert np.all(cos[0] == 1) and np.all(sin[0] == 0)
    assert cos[1, 0] == np.float32(math.cos(1.0))
    assert sin[5, 1] == np.float32(math.sin(5 * 5e5 ** (-2 / 128)))
    assert sin[2047, 63] == np.float32(math.sin(2047 * 5e5 ** (-126 / 128)))


def test_rope_properties():
    rng = np.random.default_rng(5)
    cos, sin = ops.rope_tables(64, 8, 10.0)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((1, 16))
    cos64, sin64 = cos.astype(np.float64), sin.astype(np.float64)
    # identity at position 0
    assert np.array_equal(ops.rope(q, np.array([0]), cos64, sin64, 8), q)
    # pair norms are preserved
    p = np.array([37])
    rq = ops.rope(q, p, cos64, sin64, 8)
    np.testing.assert_allclose(np.hypot(rq[0, 0::2], rq[0, 1::2]), np.hypot(q[0, 0::2], q[0, 1::2]), rtol=1e-6)
    # inverse undoes the rotation
    np.testing.assert_allclose(ops.rope(rq, p, cos64, sin64, 8, inverse=True), q, rtol=1e-6, atol=1e-7)
    # relative position: <R_a q, R_b k> = <q, R_{b-a} k> per head (exact tables here)
    ca, sa = ops.rope_tables(64, 8, 10.0)
    c64 = np.cos(np.arange(64)[:, None] * 10.0 ** (-2.0 * np.arange(4)[None] / 8))
    s64 = np.sin(np.arange(64)[:, None] * 10.0 ** (-2.0 * np.arange(4)[None] / 8))
    lhs = np.sum(ops.rope(q, np.array([9]), c64, s64, 8) * ops.rope(k, np.array([30]), c64, s64, 8))
    rhs = np.sum(q * ops.rope(k, np.array([21]), c64, s64, 8))
    assert abs(lhs - rhs) < 1e-12
    # pair layout: column 2i pairs with 2i+1 and pair i uses frequency i
    e = np.zeros((1, 8)); e[0, 2] = 1.0
    out = ops.rope(e, np.array([3]), c64, s64, 8)
    assert abs(out[0, 2] - c64[3, 1]) < 1e-15 and abs(out[0, 3] - s64[3, 1]) < 1e-15
    assert np.count_nonzero(out) == 2


def test_qk_norm_per_head_loops():
    rng = np.random.default_rng(6)
    t = rng.standard_normal((2, 12))
    g = 1 + 0.1 * rng.standard_normal(4)
    out = ops.qk_norm(t, g, 1e-6, head_dim=4)
    for i in range(2):
        for h in range(3):
            seg = t[i, 4 * h:4 * h + 4]
            r = 1 / math.sqrt(sum(v * v for v in seg) / 4 + 1e-6)
            np.testing.assert_allclose(out[i, 4 * h:4 * h + 4], seg * r * g, rtol=1e-14)
    dy = rng.standard_normal((2, 12))
    du, dg = ops.qk_norm_bwd(t, g, 1e-6, dy, head_dim=4)
    np.testing.assert_allclose(du, _fd(lambda v: np.sum(ops.qk_norm(v, g, 1e-6, 4) * dy), t.copy()), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dg, _fd(lambda w: np.sum(ops.qk_norm(t, w, 1e-6, 4) * dy), g.copy()), rtol=1e-6, atol=1e-8)


def test_cross_entropy_closed_forms():
    V = 128256
    z = np.zeros((3, V))
    loss, per_row, lse, n, dz = ops.cross_entropy(z, np.array([0, 5, V - 1]))
    assert abs(loss - math.log(V)) < 1e-12 and abs(loss - 11.7617835456) < 1e-9
    rng = np.random.default_rng(8)
    z = rng.standard_normal((6, 50)) * 3
    labels = np.array([0, 49, -100, 7, 7, 25])
    loss, per_row, lse, n, dz = ops.cross_entropy(z, labels)
    assert n == 5 and per_row[2] == 0 and np.all(dz[2] == 0)
    np.testing.assert_allclose(dz.sum(axis=1), 0, atol=1e-15)
    # a per-row shift of the logits changes nothing
    loss2, _, lse2, _, dz2 = ops.cross_entropy(z + rng.standard_normal((6, 1)) * 10, labels)
    assert abs(loss2 - loss) < 1e-12 and np.allclose(dz2, dz, atol=1e-15)
    tz = torch.tensor(z, requires_grad=True)
    tl = torch.nn.functional.cross_entropy(tz, torch.tensor(labels), ignore_index=-100)
    tl.backward()
    assert abs(tl.item() - loss) < 1e-13
    np.testing.assert_allclose(dz, tz.grad.numpy(), atol=1e-16)
    # brute force for one row
    i = 3
    ref = -math.log(math.exp(z[i, 7]) / sum(math.exp(v) for v in z[i]))
    assert abs(per_row[i] - ref) < 1e-12


def test_cross_entropy_degenerate():
    z = np.random.default_rng(9).standard_normal((3, 10))
    loss, _, _, n, dz = ops.cross_entropy(z, np.array([-100, -100, -100]))
    assert n == 0 and math.isnan(loss) and np.all(dz == 0)
    with pytest.raises(ValueError):
        ops.cross_entropy(z, np.array([0, 10, 1]))
    with pytest.raises(ValueError):
        ops.cross_entropy(z, np.array([0, -5, 1]))


def test_tile_partials():
    u = np.arange(2 * 10, dtype=np.float64).reshape(2, 10)
    P = tile_partials(u * u, 4)
    assert P.shape == (3, 2)
    assert P[2, 1] == sum(v * v for v in u[1, 8:10])
    np.testing.assert_allclose(P.sum(axis=0), (u * u).sum(axis=1))
