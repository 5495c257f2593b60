"""Pins for the oracle's block, config-1 and cross-entropy evaluations (CPU).

* The reparameterised (contract) evaluation with rounding switched off, in
  float64, equals the canonical unfused evaluation (the CODA paper, §3.2.1
  identity and the delayed-r rewrite) - forward and every gradient.
* The canonical backward equals central finite differences of the canonical
  forward and torch's float64 autograd.
* Special cases reduce the block to its parts; brute-force scalar loops
  evaluate a two-token block.
"""
import math

import numpy as np
import pytest
import torch

import coda_inputs as ci
from oracle import block as ob
from oracle import numerics as nm
from oracle import ops

TINY = ci.BlockShape(M=6, D=16, F=24, head_dim=8, seq_len=4, theta=10.0, eps=1e-6)


def tiny_inputs(seed=0, shape=TINY):
    rng = np.random.default_rng(seed)
    M, D, F, hd = shape.M, shape.D, shape.F, shape.head_dim
    n = lambda *s: rng.standard_normal(s)
    return dict(x=n(M, D), o=n(M, D), g1=1 + 0.1 * n(D), g2=1 + 0.1 * n(D),
                gq=1 + 0.1 * n(hd), gk=1 + 0.1 * n(hd),
                Wqkv=n(D, 3 * D) / math.sqrt(D), Wo=n(D, D) / math.sqrt(D),
                Wg=n(D, F) / math.sqrt(D), Wu=n(D, F) / math.sqrt(D), Wd=n(F, D) / math.sqrt(F),
                dY=0.1 * n(M, D), dq=0.1 * n(M, D), dk=0.1 * n(M, D), dv=0.1 * n(M, D))


def _ident(x):
    return x


def test_reparameterised_forward_equals_canonical():
    P = tiny_inputs(1)
    can = ob.block_forward_canonical(P, TINY)
    rep = ob.block_forward_contract(P, TINY, rnd=_ident, dt=np.float64)
    for k in ("q", "k", "v", "q_pre", "k_pre", "h1", "hg", "hu", "a", "y", "sumsq_y"):
        np.testing.assert_allclose(rep[k], can[k], rtol=1e-12, atol=1e-12, err_msg=k)


def test_reparameterised_backward_equals_canonical():
    P = tiny_inputs(2)
    can_f = ob.block_forward_canonical(P, TINY)
    can_b = ob.block_backward_canonical(P, can_f, TINY)
    rep_f = ob.block_forward_contract(P, TINY, rnd=_ident, dt=np.float64)
    rep_b = ob.block_backward_contract(P, rep_f, TINY, rnd=_ident, dt=np.float64)
    for k in can_b:
        np.testing.assert_allclose(rep_b[k], can_b[k], rtol=1e-11, atol=1e-12, err_msg=k)


def _loss(P):
    f = ob.block_forward_canonical(P, TINY)
    return (np.sum(f["y"] * P["dY"]) + np.sum(f["q"] * P["dq"]) + np.sum(f["k"] * P["dk"])
            + np.sum(f["v"] * P["dv"]))


@pytest.mark.parametrize("name,grad", [("x", "dx"), ("o", "do"), ("Wqkv", "dWqkv"), ("Wo", "dWo"),
                                       ("Wg", "dWg"), ("Wu", "dWu"), ("Wd", "dWd"), ("g1", "dg1"),
                                       ("g2", "dg2"), ("gq", "dgq"), ("gk", "dgk")])
def test_canonical_backward_finite_differences(name, grad):
    P = tiny_inputs(3)
    B = ob.block_backward_canonical(P, ob.block_forward_canonical(P, TINY), TINY)
    rng = np.random.default_rng(11)
    flat = P[name].reshape(-1)
    idx = rng.choice(flat.size, size=min(flat.size, 24), replace=False)
    h = 1e-6
    for i in idx:
        old = flat[i]
        flat[i] = old + h
        lp = _loss(P)
        flat[i] = old - h
        lm = _loss(P)
        flat[i] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - B[grad].reshape(-1)[i]) <= 1e-6 * (1 + abs(fd)), (name, i)


def _torch_block(T, shape):
    D, hd, eps = shape.D, shape.head_dim, shape.eps
    M = T["x"].shape[0]
    cos, sin = ops.rope_tables(shape.seq_len, hd, shape.theta)
    pos = np.arange(M) % shape.seq_len
    c = torch.tensor(cos[pos], dtype=torch.float64)
    s = torch.tensor(sin[pos], dtype=torch.float64)

    def rope(t):
        v = t.reshape(M, -1, hd // 2, 2)
        a, b = v[..., 0], v[..., 1]
        cc, ss = c[:, None, :], s[:, None, :]
        return torch.stack([a * cc - b * ss, a * ss + b * cc], dim=-1).reshape(M, -1)

    def qkn(t, g):
        return torch.nn.functional.rms_norm(t.reshape(M, -1, hd), (hd,), g, eps).reshape(M, -1)

    rms = torch.nn.functional.rms_norm
    qkv = rms(T["x"], (D,), T["g1"], eps) @ T["Wqkv"]
    q = rope(qkn(qkv[:, :D], T["gq"]))
    k = rope(qkn(qkv[:, D:2 * D], T["gk"]))
    v = qkv[:, 2 * D:]
    h1 = T["x"] + T["o"] @ T["Wo"]
    xn2 = rms(h1, (D,), T["g2"], eps)
    a = torch.nn.functional.silu(xn2 @ T["Wg"]) * (xn2 @ T["Wu"])
    y = h1 + a @ T["Wd"]
    return q, k, v, y


def test_canonical_backward_matches_torch_autograd():
    P = tiny_inputs(4)
    B = ob.block_backward_canonical(P, ob.block_forward_canonical(P, TINY), TINY)
    T = {k: torch.tensor(v, requires_grad=True) for k, v in P.items()}
    q, k, v, y = _torch_block(T, TINY)
    loss = (y * T["dY"]).sum() + (q * T["dq"]).sum() + (k * T["dk"]).sum() + (v * T["dv"]).sum()
    loss.backward()
    pairs = dict(dx="x", do="o", dWqkv="Wqkv", dWo="Wo", dWg="Wg", dWu="Wu", dWd="Wd",
                 dg1="g1", dg2="g2", dgq="gq", dgk="gk")
    for g, n in pairs.items():
        np.testing.assert_allclose(B[g], T[n].grad.numpy(), rtol=1e-10, atol=1e-13, err_msg=g)


def test_block_special_cases():
    P = tiny_inputs(5)
    P0 = dict(P, Wo=np.zeros_like(P["Wo"]))
    f = ob.block_forward_canonical(P0, TINY)
    assert np.array_equal(f["h1"], P["x"])
    P1 = dict(P, Wu=np.zeros_like(P["Wu"]))
    f = ob.block_forward_canonical(P1, TINY)
    assert np.all(f["a"] == 0) and np.array_equal(f["y"], f["h1"])
    f = ob.block_forward_canonical(P, TINY)
    # rows at position 0 (rows 0 and 4 with seq_len 4) are not rotated
    qn = ops.qk_norm(f["q_pre"], P["gq"], TINY.eps, TINY.head_dim)
    np.testing.assert_array_equal(f["q"][[0, 4]], qn[[0, 4]])
    assert not np.allclose(f["q"][1], qn[1])


def test_block_brute_force_two_tokens():
    shape = ci.BlockShape(M=2, D=4, F=3, head_dim=2, seq_len=2, theta=10.0, eps=1e-6)
    P = tiny_inputs(6, shape)
    f = ob.block_forward_canonical(P, shape)
    D, F, hd, eps = 4, 3, 2, 1e-6
    for i in range(2):
        x = [float(v) for v in P["x"][i]]
        r = 1 / math.sqrt(sum(v * v for v in x) / D + eps)
        xn = [x[k] * r * P["g1"][k] for k in range(D)]
        qkv = [sum(xn[k] * P["Wqkv"][k, j] for k in range(D)) for j in range(3 * D)]
        out_q = []
        for hh in range(D // hd):
            seg = qkv[hh * hd:(hh + 1) * hd]
            rr = 1 / math.sqrt(sum(v * v for v in seg) / hd + eps)
            n = [seg[j] * rr * P["gq"][j] for j in range(hd)]
            ang = i * 10.0 ** 0.0     # one pair per head: frequency theta^0 = 1
            cs, sn = float(np.float32(math.cos(ang))), float(np.float32(math.sin(ang)))
            out_q += [n[0] * cs - n[1] * sn, n[0] * sn + n[1] * cs]
        np.testing.assert_allclose(f["q"][i], out_q, rtol=1e-12)
        np.testing.assert_allclose(f["v"][i], qkv[2 * D:], rtol=1e-12)
        h1 = [x[j] + sum(P["o"][i, k] * P["Wo"][k, j] for k in range(D)) for j in range(D)]
        r2 = 1 / math.sqrt(sum(v * v for v in h1) / D + eps)
        xn2 = [h1[k] * r2 * P["g2"][k] for k in range(D)]
        hg = [sum(xn2[k] * P["Wg"][k, j] for k in range(D)) for j in range(F)]
        hu = [sum(xn2[k] * P["Wu"][k, j] for k in range(D)) for j in range(F)]
        a = [hg[j] / (1 + math.exp(-hg[j])) * hu[j] for j in range(F)]
        y = [h1[j] + sum(a[k] * P["Wd"][k, j] for k in range(F)) for j in range(D)]
        np.testing.assert_allclose(f["y"][i], y, rtol=1e-12)


def test_contract_bf16_close_to_ideal():
    shape = ci.BlockShape(M=64, D=256, F=320, head_dim=128, seq_len=32)
    P = ci.block_inputs(shape, seed=0)
    ideal_f = ob.block_forward_canonical(P, shape)
    ideal_b = ob.block_backward_canonical(P, ideal_f, shape)
    con_f = ob.block_forward_contract(P, shape)
    con_b = ob.block_backward_contract(P, con_f, shape)
    for k in ("q", "k", "v", "h1", "a", "y"):
        d = np.abs(con_f[k] - ideal_f[k]) / (1 + np.abs(ideal_f[k]))
        assert d.max() < 2e-2, k
    for k in ("dWqkv", "dWo", "dWg", "dWu", "dWd", "dg1", "dg2", "dgq", "dgk", "dx", "do"):
        rel = np.linalg.norm(con_b[k] - ideal_b[k]) / np.linalg.norm(ideal_b[k])
        assert rel < 2e-2, (k, rel)


def test_swiglu_config1_forms_agree():
    s = ci.SwiGLUShape(M=8, K=64, F=32)
    P = ci.swiglu_inputs(s, 0)
    P64 = {k: v.astype(np.float64) for k, v in P.items()}
    can = ob.swiglu_forward_canonical(P64["x"], P64["g"], P64["Wg"], P64["Wu"], s.eps)
    rep = ob.swiglu_forward_contract(P64["x"], P64["g"], P64["Wg"], P64["Wu"], s.eps, rnd=_ident)
    np.testing.assert_allclose(rep, can, rtol=1e-12, atol=1e-13)
    con = ob.swiglu_forward_contract(P["x"], P["g"], P["Wg"], P["Wu"], s.eps)
    assert np.all(nm.bf16(con) == con)
    assert (np.abs(con - can) / (1 + np.abs(can))).max() < 2e-2


def test_fp8_mm_error_bound_and_axes():
    rng = np.random.default_rng(12)
    A = rng.standard_normal((16, 64)).astype(np.float32)
    A[3] *= 1e-6                       # a tiny row keeps its own scale
    B = rng.standard_normal((64, 24)).astype(np.float32)
    B[:, 5] *= 1e3                     # a huge column keeps its own scale
    got = ob.mm(A, B, fp8=True)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    bound = 2 * 2.0 ** -4 * (np.abs(A).astype(np.float64) @ np.abs(B)) + 1e-30
    assert np.all(np.abs(got - exact) <= bound * 1.01)
    # one scale for the whole of A flushes the tiny row to zero: the bound fails
    QA, sA = nm.quantize_e4m3(A.reshape(1, -1), axis=1)
    QB, sB = nm.quantize_e4m3(B, axis=0)
    whole = (QA.reshape(A.shape) @ QB) * sA[0] * sB[None, :]
    assert np.all(whole[3] == 0) and np.any(np.abs(whole - exact) > bound * 1.01)


def test_ce_contract_matches_canonical():
    rng = np.random.default_rng(13)
    h = ci.to_bf16_values(rng.standard_normal((40, 32)).astype(np.float32))
    W = ci.to_bf16_values((rng.standard_normal((32, 300)) / math.sqrt(32)).astype(np.float32))
    labels = rng.integers(0, 300, 40).astype(np.int32)
    labels[[3, 17]] = -100
    f = ob.ce_forward_contract(h, W, labels)
    loss, per_row, lse, n, dz = ops.cross_entropy(h.astype(np.float64) @ W.astype(np.float64), labels)
    assert f["n_valid"] == n == 38
    assert abs(f["loss"] - loss) / loss < 1e-6
    b = ob.ce_backward_contract(h, W, labels, f["lse"], f["n_valid"], rnd=_ident)
    np.testing.assert_allclose(b["G"] * b["scale"], dz, atol=1e-7)
    np.testing.assert_allclose(b["dh"], dz @ W.T.astype(np.float64), rtol=1e-4, atol=1e-7)
    np.testing.assert_allclose(b["dW"], h.T.astype(np.float64) @ dz, rtol=1e-4, atol=1e-7)
    assert np.all(b["dh"][[3, 17]] == 0)
    # the tile-wise online (max, sum-exp) combine gives the same lse
    z = f["z"].astype(np.float64)
    m_t = ob.tile_partials(z, 64, np.max)
    s_t = np.stack([np.sum(np.exp(z[:, t * 64:(t + 1) * 64] - m_t[t][:, None]), axis=1)
                    for t in range(m_t.shape[0])])
    mstar = m_t.max(axis=0)
    lse_c = mstar + np.log(np.sum(s_t * np.exp(m_t - mstar), axis=0))
    np.testing.assert_allclose(lse_c, ops.logsumexp_rows(z), rtol=1e-13)


def test_ce_backward_out_of_range_labels_are_skipped():
    """A label outside [0, V) that is not the ignore index is a data error:
    the forward raises on it (the device path counts it instead) and leaves
    the row out of the mean, and the backward treats the row like an ignored
    one - its G row and dh row are exactly 0 and it adds nothing to dW.  So
    the backward with bad labels equals the backward with those rows set to
    the ignore index, which torch's float64 cross-entropy (ignore_index=-100)
    pins: dz and dW match its autograd with the rows masked."""
    rng = np.random.default_rng(14)
    M, D, V = 24, 16, 50
    h = ci.to_bf16_values(rng.standard_normal((M, D)).astype(np.float32))
    W = ci.to_bf16_values((rng.standard_normal((D, V)) / math.sqrt(D)).astype(np.float32))
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[[1, 5]] = -100
    bad = labels.copy()
    bad[[3, 8, 9]] = [V, -3, 2 ** 30]
    with pytest.raises(ValueError):
        ob.ce_forward_contract(h, W, bad)
    masked = bad.copy()
    masked[[3, 8, 9]] = -100
    f = ob.ce_forward_contract(h, W, masked)
    assert f["n_valid"] == M - 5
    b_bad = ob.ce_backward_contract(h, W, bad, f["lse"], f["n_valid"], rnd=_ident)
    b_msk = ob.ce_backward_contract(h, W, masked, f["lse"], f["n_valid"], rnd=_ident)
    for k in ("G", "dh", "dW"):
        assert np.array_equal(b_bad[k], b_msk[k]), k
    assert np.all(b_bad["G"][[1, 3, 5, 8, 9]] == 0) and np.all(b_bad["dh"][[1, 3, 5, 8, 9]] == 0)
    H, Wt = torch.tensor(h.astype(np.float64), requires_grad=True), torch.tensor(W.astype(np.float64),
                                                                                  requires_grad=True)
    torch.nn.functional.cross_entropy(H @ Wt, torch.tensor(masked.astype(np.int64)), ignore_index=-100).backward()
    np.testing.assert_allclose(b_bad["dW"], Wt.grad.numpy(), rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(b_bad["dh"], H.grad.numpy(), rtol=1e-4, atol=1e-6)
    # the final-norm form skips them the same way
    g = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    F = ob.norm_ce_forward_contract(h, g, W, masked, 1e-6, rnd=_ident)
    n_bad = ob.norm_ce_backward_contract(h, g, W, bad, F["lse"], F["r"], F["n_valid"], 1e-6, rnd=_ident)
    n_msk = ob.norm_ce_backward_contract(h, g, W, masked, F["lse"], F["r"], F["n_valid"], 1e-6, rnd=_ident)
    for k in ("G", "dy", "dW", "dg"):
        assert np.array_equal(n_bad[k], n_msk[k]), k


# ------------------------------------------------------------------ final RMSNorm -> LM head -> CE
def _norm_ce_tiny(seed=21, M=12, D=16, V=40):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((M, D))
    g = 1 + 0.1 * rng.standard_normal(D)
    W = rng.standard_normal((D, V)) / math.sqrt(D)
    labels = rng.integers(0, V, M)
    labels[[2, 7]] = -100
    dres = 0.1 * rng.standard_normal((M, D))
    return y, g, W, labels, dres


def test_norm_ce_canonical_matches_torch_autograd():
    y, g, W, labels, dres = _norm_ce_tiny()
    C = ob.norm_ce_canonical(y, g, W, labels, 1e-6, dres=dres)
    Y, G_, W_ = (torch.tensor(a, requires_grad=True) for a in (y, g, W))
    r = torch.rsqrt((Y * Y).mean(dim=1, keepdim=True) + 1e-6)
    z = (Y * r * G_) @ W_
    loss = torch.nn.functional.cross_entropy(z, torch.tensor(labels), ignore_index=-100)
    (loss + (Y * torch.tensor(dres)).sum()).backward()
    assert abs(C["loss"] - loss.item()) <= 1e-12 * abs(loss.item())
    np.testing.assert_allclose(C["dy"], Y.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(C["dW"], W_.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(C["dg"], G_.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_norm_ce_reparameterised_equals_canonical():
    """With rounding off, in float64, the delayed-r form (z = r (y W~), the
    stored gradient r (p - onehot), the T correction, dW and dg through the
    fold) equals the canonical RMSNorm -> linear -> CE and its autograd."""
    y, g, W, labels, dres = _norm_ce_tiny(22)
    eps = 1e-6
    C = ob.norm_ce_canonical(y, g, W, labels, eps, dres=dres)
    F = ob.norm_ce_forward_contract(y, g, W, labels, eps, rnd=_ident, dt=np.float64)
    assert abs(F["loss"] - C["loss"]) <= 1e-12 * abs(C["loss"]) and F["n_valid"] == C["n_valid"] == 10
    np.testing.assert_allclose(F["z"], C["z"], rtol=1e-12, atol=1e-14)
    B = ob.norm_ce_backward_contract(y, g, W, labels, F["lse"], F["r"], F["n_valid"], eps, rnd=_ident,
                                     dres=dres, dt=np.float64)
    for k in ("dy", "dW", "dg"):
        np.testing.assert_allclose(B[k], C[k], rtol=1e-10, atol=1e-14, err_msg=k)
    assert np.all(B["G"][[2, 7]] == 0)


def test_norm_ce_reduces_to_plain_ce():
    """Rows of unit mean square with g = 1 and eps = 0 make the norm an
    identity: the loss, lse and dW equal the plain cross-entropy's, and with
    every row on the unit sphere dy is the plain dh minus its radial part."""
    rng = np.random.default_rng(23)
    M, D, V = 9, 8, 30
    y = rng.standard_normal((M, D))
    y /= np.sqrt(np.mean(y * y, axis=1, keepdims=True))
    W = rng.standard_normal((D, V)) / math.sqrt(D)
    labels = rng.integers(0, V, M)
    C = ob.norm_ce_canonical(y, np.ones(D), W, labels, 0.0)
    loss, per_row, lse, n, dz = ops.cross_entropy(y @ W, labels)
    assert abs(C["loss"] - loss) <= 1e-13 * abs(loss)
    np.testing.assert_allclose(C["dW"], y.T @ dz, rtol=1e-12, atol=1e-15)
    dh = dz @ W.T
    radial = np.sum(dh * y, axis=1, keepdims=True) / D * y
    np.testing.assert_allclose(C["dy"], dh - radial, rtol=1e-10, atol=1e-14)


# ------------------------------------------------------------------ RMSNorm -> Linear -> sigmoid
def _sigmoid_tiny(seed=31, M=10, D=16, N=24):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, D)), 1 + 0.1 * rng.standard_normal(D),
            rng.standard_normal((D, N)) / math.sqrt(D), rng.standard_normal((N, D)) / math.sqrt(N),
            0.1 * rng.standard_normal((M, D)), 0.1 * rng.standard_normal((M, D)))


def test_sigmoid_layer_canonical_matches_torch_autograd():
    x, g, W, Wn, dY, dres = _sigmoid_tiny()
    C = ob.sigmoid_layer_canonical(x, g, W, Wn, dY, 1e-6, dres=dres)
    X, G_, W_ = (torch.tensor(a, requires_grad=True) for a in (x, g, W))
    r = torch.rsqrt((X * X).mean(dim=1, keepdim=True) + 1e-6)
    y = torch.sigmoid((X * r * G_) @ W_) @ torch.tensor(Wn)
    ((y * torch.tensor(dY)).sum() + (X * torch.tensor(dres)).sum()).backward()
    np.testing.assert_allclose(C["dx"], X.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(C["dW"], W_.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(C["dg"], G_.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_sigmoid_reparameterised_equals_canonical():
    x, g, W, Wn, dY, dres = _sigmoid_tiny(32)
    C = ob.sigmoid_layer_canonical(x, g, W, Wn, dY, 1e-6, dres=dres)
    F = ob.sigmoid_forward_contract(x, g, W, 1e-6, rnd=_ident, dt=np.float64)
    np.testing.assert_allclose(F["a"], C["a"], rtol=1e-13)
    B = ob.sigmoid_backward_contract(x, g, W, Wn, dY, F, 1e-6, dres=dres, rnd=_ident, dt=np.float64)
    for k in ("dx", "dW", "dg"):
        np.testing.assert_allclose(B[k], C[k], rtol=1e-10, atol=1e-14, err_msg=k)


def test_sigmoid_special_values():
    """sigmoid(0) = 1/2 with slope 1/4; symmetric: s(-t) = 1 - s(t)."""
    t = np.linspace(-30, 30, 61)
    s = ops.sigmoid(t)
    assert s[30] == 0.5
    np.testing.assert_allclose(s[::-1], 1 - s, atol=1e-15)
    h = 1e-6
    assert abs((ops.sigmoid(np.array(h)) - ops.sigmoid(np.array(-h))) / (2 * h) - 0.25) < 1e-9


# ------------------------------------------------------------------ RMSNorm -> Linear -> GELU
def test_gelu_layer_canonical_matches_torch_autograd():
    """The GELU layer against torch's exact (erf) GELU under float64 autograd."""
    x, g, W, Wn, dY, dres = _sigmoid_tiny(33)
    C = ob.sigmoid_layer_canonical(x, g, W, Wn, dY, 1e-6, dres=dres, act="gelu")
    X, G_, W_ = (torch.tensor(a, requires_grad=True) for a in (x, g, W))
    r = torch.rsqrt((X * X).mean(dim=1, keepdim=True) + 1e-6)
    h = (X * r * G_) @ W_
    a = torch.nn.functional.gelu(h, approximate="none")
    np.testing.assert_allclose(C["a"], a.detach().numpy(), rtol=1e-13, atol=1e-15)
    ((a @ torch.tensor(Wn) * torch.tensor(dY)).sum() + (X * torch.tensor(dres)).sum()).backward()
    np.testing.assert_allclose(C["dx"], X.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(C["dW"], W_.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(C["dg"], G_.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_gelu_reparameterised_equals_canonical():
    x, g, W, Wn, dY, dres = _sigmoid_tiny(34)
    C = ob.sigmoid_layer_canonical(x, g, W, Wn, dY, 1e-6, dres=dres, act="gelu")
    F = ob.sigmoid_forward_contract(x, g, W, 1e-6, rnd=_ident, dt=np.float64, act="gelu")
    np.testing.assert_allclose(F["a"], C["a"], rtol=1e-13, atol=1e-15)
    B = ob.sigmoid_backward_contract(x, g, W, Wn, dY, F, 1e-6, dres=dres, rnd=_ident, dt=np.float64, act="gelu")
    for k in ("dx", "dW", "dg"):
        np.testing.assert_allclose(B[k], C[k], rtol=1e-10, atol=1e-14, err_msg=k)


def test_gelu_special_values():
    """GELU(t) = t Phi(t): GELU(0) = 0 with slope 1/2; GELU(1) = Phi(1) and
    GELU(-1) = Phi(1) - 1 from the normal table; GELU(t) - GELU(-t) = t, so
    GELU'(t) + GELU'(-t) = 1; GELU(t) -> t for large t and -> 0 for large -t."""
    phi1 = 0.8413447460685429     # standard normal CDF at 1
    assert ops.gelu(np.array(0.0)) == 0.0
    assert abs(ops.gelu_grad(np.array(0.0)) - 0.5) < 1e-16
    assert abs(ops.gelu(np.array(1.0)) - phi1) < 1e-15
    assert abs(ops.gelu(np.array(-1.0)) - (phi1 - 1.0)) < 1e-15
    t = np.linspace(-6, 6, 121)
    np.testing.assert_allclose(ops.gelu(t) - ops.gelu(-t), t, atol=1e-14)
    np.testing.assert_allclose(ops.gelu_grad(t) + ops.gelu_grad(-t), 1.0, atol=1e-14)
    assert abs(ops.gelu(np.array(10.0)) - 10.0) < 1e-12 and abs(ops.gelu(np.array(-10.0))) < 1e-12
    e = 1e-6    # the derivative against central differences of the function
    np.testing.assert_allclose(ops.gelu_grad(t), (ops.gelu(t + e) - ops.gelu(t - e)) / (2 * e), atol=1e-8)
    assert ops.gelu(np.float32([1.5])).dtype == np.float32


def test_sigmoid_grad_matches_differences():
    t = np.linspace(-8, 8, 81)
    e = 1e-6
    np.testing.assert_allclose(ops.sigmoid_grad(t), (ops.sigmoid(t + e) - ops.sigmoid(t - e)) / (2 * e), atol=1e-9)
