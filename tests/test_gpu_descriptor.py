"""GPU parity of the generic entry point: one epilogue program per compiled
chain, built from the primitive ops of the descriptor (coda_gemm_epi,
coda_gemm_mx), against the CPU oracle on the same seeded inputs, at sizes
with ragged M and N tails and several tiles."""
import numpy as np
import pytest

from oracle import block as ob
from oracle import numerics as nm
from oracle import ops
from tests.helpers import FP8_TOL, assert_bf16, assert_grad, to_dev, to_np, unpack_gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gemm_epilogue_fp8_amd as coda  # noqa: E402
from coda_inputs import to_bf16_values  # noqa: E402

BF = torch.bfloat16
DEV = "cuda"


def rnd(rng, *shape, std=1.0):
    return to_bf16_values(rng.standard_normal(shape).astype(np.float32) * np.float32(std))


def bf(a):
    return to_dev(np.asarray(a, np.float32), BF)


def f32(a):
    return to_dev(np.asarray(a, np.float32))


def empty(*shape, dt=torch.float32):
    return torch.empty(shape, dtype=dt, device=DEV)


def split_partials(x2, parts):
    """Row sums of squares of x split over `parts` column slices (as producer
    epilogues would hand them over): fp32 [parts, M]."""
    b = np.linspace(0, x2.shape[1], parts + 1).astype(int)
    return np.stack([x2[:, i:j].sum(axis=1) for i, j in zip(b[:-1], b[1:])]).astype(np.float32)


def test_chain_rms_swiglu_with_saves():
    """ROW_RMS_FROM_PARTIALS (12 partial rows, merged in the workspace)
    STORE_ROW_VEC SAVE_PRE SWIGLU STORE_BF16: the config-1 layer."""
    rng = np.random.default_rng(101)
    M, K, F = 332, 256, 352          # multi-row partials [n, M] need M % 4 == 0
    x, g = rnd(rng, M, K), (1 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    Wg, Wu = rnd(rng, K, F, std=K ** -0.5), rnd(rng, K, F, std=K ** -0.5)
    Wgu = empty(K, 2 * F, dt=BF)
    coda.pack_gate_up(bf(Wg), bf(Wu), f32(g), Wgu)
    P = f32(split_partials(x.astype(np.float64) ** 2, 12))
    a, r, save = empty(M, F, dt=BF), empty(M), empty(M, 2 * F, dt=BF)
    E = coda
    coda.gemm_epi([(E.EPI_ROW_RMS_FROM_PARTIALS, 0, 1e-6), (E.EPI_STORE_ROW_VEC, 1, 0.0), (E.EPI_SAVE_PRE, 2, 0.0),
                   (E.EPI_SWIGLU, 0, 0.0), (E.EPI_STORE_BF16, 0, 0.0)], bf(x), 0, Wgu, 0, a, aux=[P, r, save])
    torch.cuda.synchronize()
    assert_bf16("a", to_np(a), ob.swiglu_forward_contract(x, g, Wg, Wu, 1e-6))
    rr = ops.inv_rms(x, 1e-6)
    assert_grad("r", to_np(r), rr)
    hg, hu = unpack_gu(to_np(save))
    assert_bf16("saved hg", hg, nm.bf16(rr[:, None] * ob.mm(x, nm.bf16(g[:, None] * Wg))))
    assert_bf16("saved hu", hu, nm.bf16(rr[:, None] * ob.mm(x, nm.bf16(g[:, None] * Wu))))


@pytest.mark.parametrize("act", ["sigmoid", "gelu"])
def test_chain_row_scale_sigmoid(act):
    """ROW_SCALE SAVE_PRE SIGMOID|GELU STORE_BF16 with a given row factor."""
    rng = np.random.default_rng(102)
    M, K, N = 300, 264, 352
    x, W = rnd(rng, M, K), rnd(rng, K, N, std=K ** -0.5)
    r = rng.uniform(0.5, 2.0, M).astype(np.float32)
    out, h = empty(M, N, dt=BF), empty(M, N, dt=BF)
    op, f = (coda.EPI_SIGMOID, ops.sigmoid) if act == "sigmoid" else (coda.EPI_GELU, ops.gelu)
    coda.gemm_epi([(coda.EPI_ROW_SCALE, 0, 0.0), (coda.EPI_SAVE_PRE, 1, 0.0), (op, 0, 0.0),
                   (coda.EPI_STORE_BF16, 0, 0.0)], bf(x), 0, bf(W), 0, out, aux=[f32(r), h])
    torch.cuda.synchronize()
    hh = r[:, None] * ob.mm(x, W)
    assert_bf16("h", to_np(h), nm.bf16(hh))
    assert_bf16(act, to_np(out), nm.bf16(f(hh)))


def test_chain_rms_qknorm_rope():
    """ROW_RMS_FROM_PARTIALS STORE_ROW_VEC SAVE_PRE QKNORM_ROPE STORE_BF16: the
    QKV layer, D = q | k | v, two heads of 128, positions m mod 100."""
    rng = np.random.default_rng(103)
    M, K, Dh, seq = 300, 256, 256, 100
    x, W = rnd(rng, M, K), rnd(rng, K, 3 * Dh, std=K ** -0.5)
    gains = (1 + 0.1 * rng.standard_normal((2, 128))).astype(np.float32)
    table = empty(seq, 128)
    coda.rope_table(seq, table)
    P = f32(split_partials(x.astype(np.float64) ** 2, 3))
    D, r, save = empty(M, 3 * Dh, dt=BF), empty(M), empty(M, 2 * Dh, dt=BF)
    E = coda
    coda.gemm_epi([(E.EPI_ROW_RMS_FROM_PARTIALS, 0, 1e-6), (E.EPI_STORE_ROW_VEC, 1, 0.0), (E.EPI_SAVE_PRE, 2, 0.0),
                   (E.EPI_QKNORM_ROPE, (3, 4), 1e-6), (E.EPI_STORE_BF16, 0, 0.0)], bf(x), 0, bf(W), 0, D,
                  aux=[P, r, save, f32(gains), table])
    torch.cuda.synchronize()
    rr = ops.inv_rms(x, 1e-6)
    t = rr[:, None] * ob.mm(x, W)
    cos, sin = ops.rope_tables(seq, 128, 5e5)
    pos = np.arange(M) % seq
    q = ops.rope(ops.qk_norm(t[:, :Dh], gains[0], 1e-6), pos, cos, sin)
    k = ops.rope(ops.qk_norm(t[:, Dh:2 * Dh], gains[1], 1e-6), pos, cos, sin)
    got = to_np(D)
    assert_bf16("q", got[:, :Dh], nm.bf16(q))
    assert_bf16("k", got[:, Dh:2 * Dh], nm.bf16(k))
    assert_bf16("v", got[:, 2 * Dh:], nm.bf16(t[:, 2 * Dh:]))
    assert_bf16("q_pre|k_pre", to_np(save), nm.bf16(t[:, :2 * Dh]))
    assert_grad("r", to_np(r), rr)


@pytest.mark.parametrize("which", ["dswiglu", "dsigmoid", "dgelu"])
def test_chain_activation_backward(which):
    """DSWIGLU|DSIGMOID|DGELU ROW_SCALE STORE_BF16 ROW_DOT_PARTIAL behind
    da = dY Wn^T (B stored [N, K]): dh~ = bf16(r dact(da, saved)), and the
    partials T[t, m] = sum over tile t of dh~ * saved."""
    rng = np.random.default_rng(104)
    M, Dm, N = 300, 256, 352
    dY, Wn = rnd(rng, M, Dm, std=0.1), rnd(rng, N, Dm, std=Dm ** -0.5)
    r = rng.uniform(0.5, 2.0, M).astype(np.float32)
    sw = which == "dswiglu"
    saved = rnd(rng, M, 2 * N if sw else N, std=2.0)
    tn = coda.partials_cols(N)
    out, T = empty(M, 2 * N if sw else N, dt=BF), empty(tn, M)
    op = dict(dswiglu=coda.EPI_DSWIGLU, dsigmoid=coda.EPI_DSIGMOID, dgelu=coda.EPI_DGELU)[which]
    coda.gemm_epi([(op, 0, 0.0), (coda.EPI_ROW_SCALE, 1, 0.0), (coda.EPI_STORE_BF16, 0, 0.0),
                   (coda.EPI_ROW_DOT_PARTIAL, 2, 0.0)], bf(dY), 0, bf(Wn), 1, out, aux=[bf(saved), f32(r), T])
    torch.cuda.synchronize()
    da = ob.mm(dY, Wn.T.copy())
    if sw:
        hg, hu = unpack_gu(saved)
        dhg, dhu = ops.swiglu_bwd(hg, hu, da)
        ref = nm.bf16(r[:, None] * np.concatenate([dhg, dhu], axis=1))
        gg, gu = unpack_gu(to_np(out))
        got = np.concatenate([gg, gu], axis=1)
        # each 256-column tile of da covers the packed columns [512 t, 512 t + 512)
        Tref = ob.tile_partials(to_np(out).astype(np.float64) * saved.astype(np.float64), 512)
    else:
        if which == "dsigmoid":
            s = ops.sigmoid(saved)
            ref = nm.bf16(r[:, None] * (da * s * (1 - s)))
        else:
            ref = nm.bf16(r[:, None] * (da * ops.gelu_grad(saved)))
        got = to_np(out)
        Tref = ob.tile_partials(ref.astype(np.float64) * saved.astype(np.float64), 256)
    assert_bf16("dh~", got, ref)
    assert_grad("T partials", to_np(T), Tref)


def test_chain_norm_correction_scale_and_residual():
    """NORM_CORRECTION SCALE_DEV ADD_TILE STORE_BF16 (B stored [N, K]) with 10
    partial rows of T, merged in the workspace:
    out = bf16(s (acc - (r T / N) u) + res)."""
    rng = np.random.default_rng(105)
    M, K, N = 300, 384, 264
    A, B = rnd(rng, M, K, std=0.1), rnd(rng, N, K, std=K ** -0.5)
    u, res = rnd(rng, M, N), rnd(rng, M, N, std=0.1)
    r = rng.uniform(0.5, 2.0, M).astype(np.float32)
    Tp = (0.1 * rng.standard_normal((10, M))).astype(np.float32)
    s = np.float32(0.75)
    out = empty(M, N, dt=BF)
    coda.gemm_epi([(coda.EPI_NORM_CORRECTION, (0, 1, 2), 0.0), (coda.EPI_SCALE_DEV, 3, 0.0),
                   (coda.EPI_ADD_TILE, 4, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)], bf(A), 0, bf(B), 1, out,
                  aux=[bf(u), f32(r), f32(Tp), f32([s]), bf(res)])
    torch.cuda.synchronize()
    c = r * Tp.sum(axis=0, dtype=np.float32) / np.float32(N)
    ref = nm.bf16(s * (ob.mm(A, B.T.copy()) - c[:, None] * u) + res)
    assert_bf16("out", to_np(out), ref)


def test_chain_wgrad_gain_accumulate():
    """SCALE_DEV WGRAD_GAIN(beta = 1) on a transposed A (the weight-gradient
    form X^T G): D = D + s g acc, partials P[t, k] = s sum over tile t of W acc."""
    rng = np.random.default_rng(106)
    Mt, Kin, N = 520, 264, 600
    X, G = rnd(rng, Mt, Kin), rnd(rng, Mt, N, std=0.1)
    W = rnd(rng, Kin, N, std=Kin ** -0.5)
    g = (1 + 0.1 * rng.standard_normal(Kin)).astype(np.float32)
    prior = rng.standard_normal((Kin, N)).astype(np.float32)
    s = np.float32(0.5)
    tn = coda.partials_cols(N)
    D, P = f32(prior), empty(tn, Kin)
    coda.gemm_epi([(coda.EPI_SCALE_DEV, 0, 0.0), (coda.EPI_WGRAD_GAIN, (1, 2, 3), 1.0)], bf(X), 1, bf(G), 0, D,
                  aux=[f32([s]), bf(W), f32(g), P])
    torch.cuda.synchronize()
    acc = ob.mm(X.T.copy(), G)
    assert_grad("dW", to_np(D), prior + s * (g[:, None] * acc))
    assert_grad("gain partials", to_np(P), ob.tile_partials(s * (W.astype(np.float64) * acc), 256))


@pytest.mark.parametrize("norm", [False, True])
def test_chain_cross_entropy_partials(norm):
    """[ROW_RMS_FROM_PARTIALS STORE_ROW_VEC] CE_LSE_PARTIAL: per (N tile, row)
    online max and sum-exp over the valid columns and the gathered label
    logit; nothing is stored to D.  The host combines the partials into lse."""
    rng = np.random.default_rng(107 + norm)
    M, K, V = 300, 256, 1000
    h, W = rnd(rng, M, K), rnd(rng, K, V, std=K ** -0.5)
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[[0, 1, 2]] = [0, V - 1, 255]
    tn = coda.partials_cols(V)
    P, zy, r = empty(2 * tn, M), empty(M).fill_(-7.0), empty(M)
    E = coda
    if norm:
        S = f32(split_partials(h.astype(np.float64) ** 2, 2))
        prog = [(E.EPI_ROW_RMS_FROM_PARTIALS, 0, 1e-6), (E.EPI_STORE_ROW_VEC, 1, 0.0),
                (E.EPI_CE_LSE_PARTIAL, (2, 3, 4), 0.0)]
        aux = [S, r, to_dev(labels), P, zy]
    else:
        prog, aux = [(E.EPI_CE_LSE_PARTIAL, (0, 1, 2), 0.0)], [to_dev(labels), P, zy]
    coda.gemm_epi(prog, bf(h), 0, bf(W), 0, None, aux=aux)
    torch.cuda.synchronize()
    z = ob.mm(h, W).astype(np.float64)
    if norm:
        rr = ops.inv_rms(h, 1e-6)
        assert_grad("r", to_np(r), rr)
        z = rr[:, None].astype(np.float64) * z
    Pg = to_np(P).astype(np.float64)
    m_t, s_t = Pg[:tn], Pg[tn:]
    mstar = m_t.max(axis=0)
    lse = mstar + np.log(np.sum(s_t * np.exp(m_t - mstar), axis=0))
    assert_grad("lse", lse, ops.logsumexp_rows(z))
    assert_grad("tile max", m_t, ob.tile_partials(z, 256, np.max))
    assert_grad("label logit", to_np(zy), z[np.arange(M), labels])


@pytest.mark.parametrize("norm", [False, True])
def test_chain_cross_entropy_grad(norm):
    """CE_GRAD STORE_BF16, and ROW_SCALE CE_GRAD STORE_BF16 ROW_DOT_PARTIAL:
    G = bf16([r] (exp(z - lse) - onehot)) on rows with a label in [0, V),
    exactly 0 elsewhere (ignored and out-of-range labels); z = [r] acc; the
    partials sum G * z per tile."""
    rng = np.random.default_rng(109 + norm)
    M, K, V = 300, 256, 1000
    h, W = rnd(rng, M, K), rnd(rng, K, V, std=K ** -0.5)
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[[3, 4, 5]] = [-100, V, -2]
    r = rng.uniform(0.5, 2.0, M).astype(np.float32) if norm else np.ones(M, np.float32)
    z = r[:, None] * ob.mm(h, W)
    lse = ops.logsumexp_rows(z.astype(np.float64)).astype(np.float32)
    G = empty(M, V, dt=BF)
    E = coda
    if norm:
        T = empty(coda.partials_cols(V), M)
        coda.gemm_epi([(E.EPI_ROW_SCALE, 0, 0.0), (E.EPI_CE_GRAD, (1, 2), 0.0), (E.EPI_STORE_BF16, 0, 0.0),
                       (E.EPI_ROW_DOT_PARTIAL, 3, 0.0)], bf(h), 0, bf(W), 0, G,
                      aux=[f32(r), to_dev(labels), f32(lse), T])
    else:
        coda.gemm_epi([(E.EPI_CE_GRAD, (0, 1), 0.0), (E.EPI_STORE_BF16, 0, 0.0)], bf(h), 0, bf(W), 0, G,
                      aux=[to_dev(labels), f32(lse)])
    torch.cuda.synchronize()
    p = np.exp(z - lse[:, None]).astype(np.float32)
    valid = (labels >= 0) & (labels < V)
    rows = np.nonzero(valid)[0]
    p[rows, labels[rows]] -= 1
    p[~valid] = 0
    ref = nm.bf16(r[:, None] * p)
    got = to_np(G)
    assert np.all(got[~valid] == 0)
    assert_bf16("G", got, ref)
    if norm:
        assert_grad("T partials", to_np(T), ob.tile_partials(got.astype(np.float64) * z, 256))


def test_chains_device_scale():
    """SCALE_DEV STORE_BF16 (B stored [N, K]) and SCALE_DEV ACCUM_F32 on a
    transposed A with beta = 1."""
    rng = np.random.default_rng(111)
    M, K, N = 304, 264, 352          # the transposed A [K, M] needs M % 8 == 0
    A, B = rnd(rng, M, K), rnd(rng, N, K, std=K ** -0.5)
    s = np.float32(1.0 / 37.0)
    out = empty(M, N, dt=BF)
    coda.gemm_epi([(coda.EPI_SCALE_DEV, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)], bf(A), 0, bf(B), 1, out,
                  aux=[f32([s])])
    prior = rng.standard_normal((M, N)).astype(np.float32)
    D = f32(prior)
    coda.gemm_epi([(coda.EPI_SCALE_DEV, 0, 0.0), (coda.EPI_ACCUM_F32, 0, 1.0)], bf(A.T.copy()), 1,
                  bf(B.T.copy()), 0, D, aux=[f32([s])])
    torch.cuda.synchronize()
    acc = ob.mm(A, B.T.copy())
    assert_bf16("s acc", to_np(out), nm.bf16(s * acc))
    assert_grad("prior + s acc", to_np(D), prior + s * acc)


def _e4m3(X, axis):
    """Library E4M3 copy of X along `axis` (1: per row, [R, C]; 0: per column,
    written transposed [C, R])."""
    R, Cc = X.shape
    Q = torch.empty((R, Cc) if axis == 1 else (Cc, R), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty(R if axis == 1 else Cc, dtype=torch.float32, device=DEV)
    coda.quantize_e4m3(bf(X), axis, Q, s)
    return Q, s


def test_chains_e4m3_operands():
    """DEQUANT_E4M3 first: E4M3 operands A [M, K], B [N, K] with per-row and
    per-column amax scales, then ADD_TILE STORE_BF16 ROW_SUMSQ_PARTIAL and
    ROW_SCALE SWIGLU STORE_BF16; against the oracle's E4M3 product of the
    same bf16 inputs (the quantiser is bit-exact, so only accumulation
    differs)."""
    rng = np.random.default_rng(112)
    M, K, N = 304, 256, 384
    a, W = rnd(rng, M, K), rnd(rng, K, N, std=K ** -0.5)
    z = rnd(rng, M, N)
    Qa, sa = _e4m3(a, 1)
    Qw, sw = _e4m3(W, 0)
    tn = coda.partials_cols(N)
    out, P = empty(M, N, dt=BF), empty(tn, M)
    E = coda
    coda.gemm_epi([(E.EPI_DEQUANT_E4M3, (0, 1), 0.0), (E.EPI_ADD_TILE, 2, 0.0), (E.EPI_STORE_BF16, 0, 0.0),
                   (E.EPI_ROW_SUMSQ_PARTIAL, 3, 0.0)], Qa, 0, Qw, 1, out, aux=[sa, sw, bf(z), P])
    r = rng.uniform(0.5, 2.0, M).astype(np.float32)
    a2 = empty(M, N // 2, dt=BF)
    coda.gemm_epi([(E.EPI_DEQUANT_E4M3, (0, 1), 0.0), (E.EPI_ROW_SCALE, 2, 0.0), (E.EPI_SWIGLU, 0, 0.0),
                   (E.EPI_STORE_BF16, 0, 0.0)], Qa, 0, Qw, 1, a2, aux=[sa, sw, f32(r)])
    torch.cuda.synchronize()
    acc = ob.mm(a, W, fp8=True)
    y = nm.bf16(z + acc)
    assert_bf16("residual", to_np(out), y, tol=FP8_TOL)
    assert_grad("sumsq partials", to_np(P), ob.tile_partials(to_np(out).astype(np.float64) ** 2, 256))
    hg, hu = unpack_gu(r[:, None] * acc)
    assert_bf16("swiglu", to_np(a2), nm.bf16(ops.swiglu(hg, hu)), tol=FP8_TOL)


def test_chain_mxfp8_norm_correction():
    """A chain the block-scaled entry point now reaches through the
    descriptor: NORM_CORRECTION ADD_TILE STORE_BF16 on MXFP8 operands."""
    rng = np.random.default_rng(113)
    M, K, N = 300, 384, 264
    A, B = rnd(rng, M, K, std=0.1), rnd(rng, K, N, std=K ** -0.5)
    u, res = rnd(rng, M, N), rnd(rng, M, N, std=0.1)
    r = rng.uniform(0.5, 2.0, M).astype(np.float32)
    Tp = (0.1 * rng.standard_normal((3, M))).astype(np.float32)
    QA, SA = coda.quantize_mxfp8(bf(A), 1)
    QB, SB = coda.quantize_mxfp8(bf(B), 0)
    out = empty(M, N, dt=BF)
    coda.gemm_mx([(coda.EPI_NORM_CORRECTION, (0, 1, 2), 0.0), (coda.EPI_ADD_TILE, 3, 0.0),
                  (coda.EPI_STORE_BF16, 0, 0.0)], QA, SA, QB, SB, out, aux=[bf(u), f32(r), f32(Tp), bf(res)])
    torch.cuda.synchronize()
    c = r * Tp.sum(axis=0, dtype=np.float32) / np.float32(N)
    ref = nm.bf16(ob.mm(A, B, "mx") - c[:, None] * u + res)
    assert_bf16("out", to_np(out), ref, tol=FP8_TOL)


@pytest.mark.parametrize("fmt", ["e2m1", "e2m3", "e3m2"])
def test_chain_mx_small_backward_chains(fmt):
    """Two backward chains of the MX column on MXFP4 and MXFP6 operands
    through the descriptor: NORM_CORRECTION ADD_TILE STORE_BF16, and
    SCALE_DEV WGRAD_GAIN accumulating onto a prior (both operands quantised
    along the contracted axis), against the oracle's product in the same
    format."""
    rng = np.random.default_rng(117)
    mode = {"e2m1": "mx4", "e2m3": "mx6_e2m3", "e3m2": "mx6_e3m2"}[fmt]

    def q(X, axis):
        return coda.quantize_mxfp4(bf(X), axis) if fmt == "e2m1" else coda.quantize_mxfp6(bf(X), axis, fmt)

    def gemm(prog, QA, SA, QB, SB, D, aux):
        if fmt == "e2m1":
            return coda.gemm_mx4(prog, QA, SA, QB, SB, D, aux=aux)
        return coda.gemm_mx6(prog, fmt, QA, SA, QB, SB, D, aux=aux)

    M, K, N = 300, 384, 264
    A, B = rnd(rng, M, K, std=0.1), rnd(rng, K, N, std=K ** -0.5)
    u, res = rnd(rng, M, N), rnd(rng, M, N, std=0.1)
    r = rng.uniform(0.5, 2.0, M).astype(np.float32)
    Tp = (0.1 * rng.standard_normal((3, M))).astype(np.float32)
    QA, SA = q(A, 1)
    QB, SB = q(B, 0)
    out = empty(M, N, dt=BF)
    gemm([(coda.EPI_NORM_CORRECTION, (0, 1, 2), 0.0), (coda.EPI_ADD_TILE, 3, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)],
         QA, SA, QB, SB, out, [bf(u), f32(r), f32(Tp), bf(res)])
    # weight-gradient form: D[Kin, N] += s g[k] (X^T G)[k, n] over Mt tokens
    Mt, Kin = 256, 264
    X, G = rnd(rng, Mt, Kin), rnd(rng, Mt, N, std=0.1)
    W = rnd(rng, Kin, N, std=Kin ** -0.5)
    g = (1 + 0.1 * rng.standard_normal(Kin)).astype(np.float32)
    prior = rng.standard_normal((Kin, N)).astype(np.float32)
    s = np.float32(0.5)
    QX, SX = q(X, 0)          # [Kin, Mt]: blocks along the tokens
    QG, SG = q(G, 0)          # [N, Mt]
    Dw, P = f32(prior), empty(coda.partials_cols(N), Kin)
    gemm([(coda.EPI_SCALE_DEV, 0, 0.0), (coda.EPI_WGRAD_GAIN, (1, 2, 3), 1.0)], QX, SX, QG, SG, Dw,
         [f32([s]), bf(W), f32(g), P])
    torch.cuda.synchronize()
    c = r * Tp.sum(axis=0, dtype=np.float32) / np.float32(N)
    assert_bf16("norm correction", to_np(out), nm.bf16(ob.mm(A, B, mode) - c[:, None] * u + res), tol=FP8_TOL)
    acc = ob.mm(X.T.copy(), G, mode)
    assert_grad("dW", to_np(Dw), prior + s * (g[:, None] * acc), rel=2e-3)
    assert_grad("gain partials", to_np(P), ob.tile_partials(s * (W.astype(np.float64) * acc), 256), rel=2e-3)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e2m3", "e3m2"])
def test_chain_mx_gelu(fmt):
    """GELU forward (ROW_SCALE SAVE_PRE GELU STORE_BF16) and backward (DGELU
    ROW_SCALE STORE_BF16 ROW_DOT_PARTIAL behind da = dY Wn^T) on MXFP8, MXFP4
    and both MXFP6 operands the library quantised, against the oracle's
    product in the same format."""
    rng = np.random.default_rng(118)
    mode = {"e4m3": "mx", "e2m1": "mx4", "e2m3": "mx6_e2m3", "e3m2": "mx6_e3m2"}[fmt]

    def q(X, axis):
        if fmt == "e4m3":
            return coda.quantize_mxfp8(bf(X), axis)
        return coda.quantize_mxfp4(bf(X), axis) if fmt == "e2m1" else coda.quantize_mxfp6(bf(X), axis, fmt)

    def gemm(prog, QA, SA, QB, SB, D, aux):
        if fmt == "e4m3":
            return coda.gemm_mx(prog, QA, SA, QB, SB, D, aux=aux)
        if fmt == "e2m1":
            return coda.gemm_mx4(prog, QA, SA, QB, SB, D, aux=aux)
        return coda.gemm_mx6(prog, fmt, QA, SA, QB, SB, D, aux=aux)

    M, K, N = 300, 384, 264
    x, W = rnd(rng, M, K), rnd(rng, K, N, std=K ** -0.5)
    r = rng.uniform(0.5, 2.0, M).astype(np.float32)
    QA, SA = q(x, 1)
    QB, SB = q(W, 0)
    out, h = empty(M, N, dt=BF), empty(M, N, dt=BF)
    gemm([(coda.EPI_ROW_SCALE, 0, 0.0), (coda.EPI_SAVE_PRE, 1, 0.0), (coda.EPI_GELU, 0, 0.0),
          (coda.EPI_STORE_BF16, 0, 0.0)], QA, SA, QB, SB, out, [f32(r), h])
    Dm = 256
    dY, Wn = rnd(rng, M, Dm, std=0.1), rnd(rng, N, Dm, std=Dm ** -0.5)
    saved = rnd(rng, M, N, std=2.0)
    QY, SY = q(dY, 1)
    QW, SW = q(Wn, 1)          # [N, Dm]: blocks along the contracted axis
    dh, T = empty(M, N, dt=BF), empty(coda.partials_cols(N), M)
    gemm([(coda.EPI_DGELU, 0, 0.0), (coda.EPI_ROW_SCALE, 1, 0.0), (coda.EPI_STORE_BF16, 0, 0.0),
          (coda.EPI_ROW_DOT_PARTIAL, 2, 0.0)], QY, SY, QW, SW, dh, [bf(saved), f32(r), T])
    torch.cuda.synchronize()
    hh = r[:, None] * ob.mm(x, W, mode)
    assert_bf16("h", to_np(h), nm.bf16(hh), tol=FP8_TOL)
    assert_bf16("gelu", to_np(out), nm.bf16(ops.gelu(hh)), tol=FP8_TOL)
    ref = nm.bf16(r[:, None] * (ob.mm(dY, Wn.T.copy(), mode) * ops.gelu_grad(saved)))
    assert_bf16("dh~", to_np(dh), ref, tol=FP8_TOL)
    assert_grad("T partials", to_np(T), ob.tile_partials(ref.astype(np.float64) * saved.astype(np.float64), 256),
                rel=2e-3)
