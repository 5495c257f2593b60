"""GPU parity of the MXFP8 path (E4M3 elements with one E8M0 scale per 32
values of the contracted axis, OCP Microscaling v1.0) through the C ABI:
the quantiser bit for bit against oracle/mx.py, and the block-scaled GEMM
with each compiled epilogue against the oracle's float64 product of the
dequantised operands."""
import numpy as np
import pytest

import coda_inputs as ci
from oracle import block as ob
from oracle import mx
from oracle import numerics as nm
from oracle import ops
from tests.helpers import assert_bf16, assert_grad, to_dev, to_np, unpack_gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gemm_epilogue_fp8_amd as coda  # noqa: E402

BF = torch.bfloat16
DEV = "cuda"
FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def bf(a):
    return to_dev(np.asarray(a, np.float32), BF)


def f32(a):
    return to_dev(np.asarray(a, np.float32))


def u8(a):
    return to_dev(np.ascontiguousarray(a, dtype=np.uint8))


def e4m3_dev(codes):
    return u8(codes).view(torch.float8_e4m3fn)


def to_words(e8):
    """[rows, nblocks] exponent bytes -> the library's word layout
    [ceil(nblocks / 4), 4 rows]: byte (g, 4 r + j) = block 4 g + j of row r."""
    rows, nb = e8.shape
    G = (nb + 3) // 4
    full = np.zeros((rows, 4 * G), np.uint8)
    full[:, :nb] = e8
    return np.ascontiguousarray(full.reshape(rows, G, 4).transpose(1, 0, 2).reshape(G, 4 * rows))


def from_words(S, rows, nb):
    """Inverse of to_words, keeping the nb blocks that exist."""
    S = np.asarray(S)
    G = S.shape[0]
    return S.reshape(G, rows, 4).transpose(1, 0, 2).reshape(rows, 4 * G)[:, :nb]


def varied_bf16(rng, R, C, axis):
    """bf16 values whose magnitude changes by powers of two from block to
    block along `axis`, with one all-zero block and one block of large values,
    so that the shared exponents cover a wide range."""
    X = rng.standard_normal((R, C)).astype(np.float32)
    if axis == 1:
        X *= np.exp2(rng.integers(-24, 24, size=(R, C // 32))).repeat(32, axis=1).astype(np.float32)
        X[0, :32] = 0.0
        X[-1, -32:] *= np.float32(2.0 ** 60)
    else:
        X *= np.exp2(rng.integers(-24, 24, size=(R // 32, C))).repeat(32, axis=0).astype(np.float32)
        X[:32, 0] = 0.0
        X[-32:, -1] *= np.float32(2.0 ** 60)
    return ci.to_bf16_values(X)


# ------------------------------------------------------------------ quantiser
@pytest.mark.parametrize("axis,R,C", [(1, 37, 320), (1, 1, 32), (0, 320, 72), (0, 96, 200)])
def test_quantize_mxfp8_bit_exact(axis, R, C):
    rng = np.random.default_rng(R * 7 + C + axis)
    X = varied_bf16(rng, R, C, axis)
    Q, S = coda.quantize_mxfp8(bf(X), axis)
    torch.cuda.synchronize()
    P, e = mx.quantize(X if axis == 1 else X.T.copy())
    assert np.array_equal(Q.view(torch.uint8).cpu().numpy(), mx.codes(P))
    assert S.shape == ((e.shape[1] + 3) // 4, 4 * e.shape[0])
    assert np.array_equal(from_words(S.cpu().numpy(), *e.shape), mx.e8m0_codes(e))


def test_quantize_mxfp8_rejects_ragged_blocks():
    X = torch.zeros((40, 48), dtype=BF, device=DEV)
    with pytest.raises(coda.CodaError):
        coda.quantize_mxfp8(X, 1)
    with pytest.raises(coda.CodaError):
        coda.quantize_mxfp8(X, 0)


# ------------------------------------------------------------------ GEMM
def random_mx(rng, rows, K, emin=117, emax=137):
    """An MXFP8 operand drawn directly: uniform finite E4M3 codes and E8M0
    codes uniform in [emin, emax] (2^-10 .. 2^10), independent per block."""
    codes = rng.choice(FINITE_CODES, size=(rows, K))
    scales = rng.integers(emin, emax + 1, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


def mx_values(codes, scales):
    """float64 values an MXFP8 operand stands for (oracle decode)."""
    return mx.dequantize(nm.e4m3_decode(codes), scales.astype(np.int64) - 127)


def mfma_fp8_bound(A, B):
    """Bound on the difference between the matrix core's sum of
    sum_k A[m,k] B[n,k] and the exact sum: 2^-10 sum_k |A B|.  The E4M3
    MFMA does not round like a sequence of fp32 additions: on MI355X its
    error, with unit scales and with block scales alike, reaches about
    5000 u sum_k |A B| (u = 2^-24, K = 384), i.e. 3e-4 sum_k |A B|, and
    5e-5 norm-wise; products of two E4M3 values times powers of two are
    exact, so only the accumulation contributes."""
    return 2.0 ** -10 * (np.abs(A) @ np.abs(B).T)


@pytest.mark.parametrize("M,N,K", [(300, 264, 384), (517, 520, 1024), (64, 8, 128)])
def test_gemm_mx_accum_and_store(M, N, K):
    rng = np.random.default_rng(M + N + K)
    ca, sa = random_mx(rng, M, K)
    cb, sb = random_mx(rng, N, K)
    A, B = mx_values(ca, sa), mx_values(cb, sb)
    ref = A @ B.T
    prior = ci.fp32_prior((M, N), 4)
    D32 = f32(prior)
    coda.gemm_mx([(coda.EPI_ACCUM_F32, 0, 1.0)], e4m3_dev(ca), u8(to_words(sa)), e4m3_dev(cb), u8(to_words(sb)), D32)
    D16 = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx([(coda.EPI_STORE_BF16, 0, 0.0)], e4m3_dev(ca), u8(to_words(sa)), e4m3_dev(cb), u8(to_words(sb)), D16)
    torch.cuda.synchronize()
    bound = mfma_fp8_bound(A, B)
    got32 = to_np(D32).astype(np.float64) - prior
    # the prior add is one more fp32 rounding
    assert np.all(np.abs(got32 - ref) <= bound + 2.0 ** -23 * (np.abs(ref) + np.abs(prior))), \
        float(np.max(np.abs(got32 - ref) - bound))
    got16 = to_np(D16).astype(np.float64)
    assert np.all(np.abs(got16 - ref) <= 1.01 * bound + 2.0 ** -8 * np.abs(ref)), \
        float(np.max(np.abs(got16 - ref) - bound))
    assert np.linalg.norm(got32 - ref) <= 1e-3 * np.linalg.norm(ref)
    # elementwise |d| / (1 + |ref|) means little at these magnitudes (block
    # scales 2^-10 .. 2^10 and cancelling sums); the bound above is per element
    assert np.linalg.norm(got16 - nm.bf16(ref)) <= 3e-3 * np.linalg.norm(ref)


def test_gemm_mx_one_scale_per_block():
    """Scales that differ only between the four blocks of one 128-K word and
    between rows: a scale taken from the wrong block, stage or row moves the
    result by a power of two."""
    rng = np.random.default_rng(17)
    M, N, K = 256, 256, 256
    ca, _ = random_mx(rng, M, K)
    cb, _ = random_mx(rng, N, K)
    sa = (120 + (np.arange(K // 32)[None, :] * 3 + np.arange(M)[:, None]) % 15).astype(np.uint8)
    sb = (121 + (np.arange(K // 32)[None, :] * 5 + 2 * np.arange(N)[:, None]) % 13).astype(np.uint8)
    A, B = mx_values(ca, sa), mx_values(cb, sb)
    D32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    coda.gemm_mx([(coda.EPI_ACCUM_F32, 0, 0.0)], e4m3_dev(ca), u8(to_words(sa)), e4m3_dev(cb), u8(to_words(sb)), D32)
    torch.cuda.synchronize()
    ref = A @ B.T
    assert np.all(np.abs(to_np(D32) - ref) <= mfma_fp8_bound(A, B))
    assert np.linalg.norm(to_np(D32) - ref) <= 1e-3 * np.linalg.norm(ref)


def test_gemm_mx_epilogues_from_bf16():
    """bf16 inputs quantised by the library and by the oracle (bit-exact, as
    tested above), then the row/column-scale, residual + sum-of-squares and
    SwiGLU programs on the block-scaled product."""
    rng = np.random.default_rng(23)
    M, N, K = 300, 576, 384
    a = ci.to_bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    W = ci.to_bf16_values((rng.standard_normal((K, N)) * K ** -0.5).astype(np.float32))
    Qa, Sa = coda.quantize_mxfp8(bf(a), 1)
    Qw, Sw = coda.quantize_mxfp8(bf(W), 0)          # [N, K]: K contiguous
    Pa, ea = mx.quantize(a)
    Pw, ew = mx.quantize(W.T.copy())
    acc = mx.matmul_nt(Pa, ea, Pw, ew)
    bound = mfma_fp8_bound(mx.dequantize(Pa, ea), mx.dequantize(Pw, ew))

    rv = rng.uniform(0.5, 2, M).astype(np.float32)
    cv = rng.uniform(0.5, 2, N).astype(np.float32)
    D1 = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx([(coda.EPI_ROW_SCALE, 0, 0.0), (coda.EPI_COL_SCALE, 1, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)],
                 Qa, Sa, Qw, Sw, D1, aux=[f32(rv), f32(cv)])
    Z = ci.to_bf16_values(rng.standard_normal((M, N)).astype(np.float32))
    nT = coda.partials_cols(N)
    P = torch.empty((nT, M), dtype=torch.float32, device=DEV)
    D2 = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx([(coda.EPI_ADD_TILE, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0), (coda.EPI_ROW_SUMSQ_PARTIAL, 1, 0.0)],
                 Qa, Sa, Qw, Sw, D2, aux=[bf(Z), P])
    r = rng.uniform(0.5, 2, M).astype(np.float32)
    D3 = torch.empty((M, N // 2), dtype=BF, device=DEV)
    coda.gemm_mx([(coda.EPI_ROW_SCALE, 0, 0.0), (coda.EPI_SWIGLU, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)],
                 Qa, Sa, Qw, Sw, D3, aux=[f32(r)])
    torch.cuda.synchronize()

    # codes on both sides agree, so what is left is the matrix core's
    # accumulation and the epilogue's fp32 roundings before the bf16 store
    sref = (acc * rv[:, None]) * cv[None, :]
    sbound = bound * rv[:, None] * cv[None, :]
    assert np.all(np.abs(to_np(D1).astype(np.float64) - sref) <= 1.01 * sbound + 2.0 ** -8 * np.abs(sref))
    assert_bf16("scaled", to_np(D1), nm.bf16((acc * rv[:, None]) * cv[None, :]))
    y = nm.bf16(Z + acc)
    assert_bf16("residual", to_np(D2), y)
    assert_grad("sumsq partials", to_np(P), ob.tile_partials(y.astype(np.float64) ** 2, 256))
    hg, hu = unpack_gu(r[:, None] * acc)
    assert_bf16("swiglu", to_np(D3), nm.bf16(ops.swiglu(hg, hu)))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_gemm_mx_full_size_sampled():
    """The hidden-8192 down-projection shape (M 4096, K 28672, N 8192) with
    residual: the library quantises a and W; 128 sampled outputs are
    recomputed by the oracle from its own MXFP8 copies of the sampled rows of
    a and columns of W (whose codes must equal the library's bit for bit)."""
    M, K, N = 4096, 28672, 8192
    rng = np.random.default_rng(71)
    a = ci.to_bf16_values(rng.standard_normal((M, K), dtype=np.float32))
    W = ci.to_bf16_values(rng.standard_normal((K, N), dtype=np.float32) * np.float32(K ** -0.5))
    z = ci.to_bf16_values(rng.standard_normal((M, N), dtype=np.float32))
    ag, Wg, zg = bf(a), bf(W), bf(z)
    Qa, Sa = coda.quantize_mxfp8(ag, 1)
    Qw, Sw = coda.quantize_mxfp8(Wg, 0)
    out = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx([(coda.EPI_ADD_TILE, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)], Qa, Sa, Qw, Sw, out, aux=[zg])
    torch.cuda.synchronize()
    ms = rng.integers(0, M, 128)
    ns = rng.integers(0, N, 128)
    um, un = np.unique(ms), np.unique(ns)
    Pa, ea = mx.quantize(a[um])
    Pw, ew = mx.quantize(W[:, un].T.copy())
    assert np.array_equal(Qa.view(torch.uint8)[torch.from_numpy(um).to(DEV)].cpu().numpy(), mx.codes(Pa))
    assert np.array_equal(from_words(Sa.cpu().numpy(), M, K // 32)[um], mx.e8m0_codes(ea))
    assert np.array_equal(Qw.view(torch.uint8)[torch.from_numpy(un).to(DEV)].cpu().numpy(), mx.codes(Pw))
    assert np.array_equal(from_words(Sw.cpu().numpy(), N, K // 32)[un], mx.e8m0_codes(ew))
    Ad, Bd = mx.dequantize(Pa, ea), mx.dequantize(Pw, ew)
    im, jn = np.searchsorted(um, ms), np.searchsorted(un, ns)
    acc = np.einsum("ik,ik->i", Ad[im], Bd[jn])
    bound = 2.0 ** -10 * np.einsum("ik,ik->i", np.abs(Ad[im]), np.abs(Bd[jn]))
    ref = z[ms, ns].astype(np.float64) + acc
    got = out[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1.01 * bound + 2.0 ** -8 * np.abs(ref)), float(np.max(np.abs(got - ref) - bound))
    assert_bf16("sampled out", got, nm.bf16(ref))


def test_gemm_mx_degenerate_shapes():
    """Empty M or N (empty views of allocated buffers: the C ABI takes a NULL
    pointer as an absent argument) is a no-op that leaves D untouched; a single
    row and the smallest K (one 128-value word of exponents) still match the
    oracle."""
    rng = np.random.default_rng(29)
    K = 128
    sentinel = torch.full((64, 64), 3.0, dtype=BF, device=DEV)
    for M, N in ((0, 64), (64, 0)):
        A = torch.empty((max(M, 1), K), dtype=torch.float8_e4m3fn, device=DEV)[:M]
        B = torch.empty((max(N, 1), K), dtype=torch.float8_e4m3fn, device=DEV)[:N]
        SA = torch.empty((1, 4 * max(M, 1)), dtype=torch.uint8, device=DEV)[:, :4 * M]
        SB = torch.empty((1, 4 * max(N, 1)), dtype=torch.uint8, device=DEV)[:, :4 * N]
        coda.gemm_mx([(coda.EPI_STORE_BF16, 0, 0.0)], A, SA, B, SB, sentinel[:M, :N])
    torch.cuda.synchronize()
    assert bool((sentinel == 3.0).all())
    ca, sa = random_mx(rng, 1, K)
    cb, sb = random_mx(rng, 40, K)
    D = torch.empty((1, 40), dtype=torch.float32, device=DEV)
    coda.gemm_mx([(coda.EPI_ACCUM_F32, 0, 0.0)], e4m3_dev(ca), u8(to_words(sa)), e4m3_dev(cb), u8(to_words(sb)), D)
    torch.cuda.synchronize()
    A, B = mx_values(ca, sa), mx_values(cb, sb)
    assert np.all(np.abs(to_np(D) - A @ B.T) <= mfma_fp8_bound(A, B))


# ---------------------------------------------------------------- MXFP4 quantiser
def fp4_ladder_bf16(rng, R, C, axis):
    """varied_bf16 plus, in every fourth block along `axis`, the E2M1 ties:
    a block maximum of exactly 4 (so e = 0 after scaling by the block's power
    of two) and elements on every midpoint of the value ladder, both signs,
    and small negatives that round to zero."""
    X = varied_bf16(rng, R, C, axis)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                     -0.1, -0.2, 4.0, 0.0], np.float32)
    Xt = X if axis == 1 else X.T
    nb = Xt.shape[1] // 32
    for r in range(0, Xt.shape[0], 3):
        for b in range(0, nb, 4):
            s = np.float32(2.0 ** int(rng.integers(-10, 10)))
            blk = np.resize(ties, 32) * s
            blk[rng.integers(0, 32)] = 4.0 * s
            Xt[r, 32 * b:32 * b + 32] = blk
    return ci.to_bf16_values(X if axis == 1 else Xt.T)


@pytest.mark.parametrize("axis,R,C", [(1, 300, 480), (1, 5, 32), (0, 480, 296), (0, 64, 7 * 8)])
def test_mxfp4_quantiser_bit_exact(axis, R, C):
    """Packed E2M1 codes and E8M0 exponents equal the oracle's (oracle/mx_small.py)
    bit for bit, in both orientations, with ragged tiles, an all-zero block,
    a block of very large values and every rounding tie of the E2M1 ladder."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(40 + axis)
    X = fp4_ladder_bf16(rng, R, C, axis)
    Q, S = coda.quantize_mxfp4(bf(X), axis)
    torch.cuda.synchronize()
    Xr = X if axis == 1 else np.ascontiguousarray(X.T)       # blocks along the rows of Xr
    P, e = ms.quantize(Xr, "e2m1")
    want_q = ms.pack_fp4(ms.encode(P, "e2m1"))
    got_q = to_np(Q).astype(np.uint8)
    rows, L = Xr.shape
    assert got_q.shape == (rows, L // 2)
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, (bad[:5], got_q[tuple(bad[0])], want_q[tuple(bad[0])])
    got_e = from_words(to_np(S), rows, L // 32)
    np.testing.assert_array_equal(got_e, (e + 127).astype(np.uint8))


# ---------------------------------------------------------------- MXFP4 GEMM
def random_mx4(rng, rows, K, emin=117, emax=137):
    """An MXFP4 operand drawn directly: uniform E2M1 codes (all 16) and E8M0
    codes uniform in [emin, emax], independent per block; returns the codes
    [rows, K] and the exponent bytes [rows, K / 32]."""
    codes = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
    scales = rng.integers(emin, emax + 1, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


def mx4_values(codes, scales):
    from oracle import mx_small as ms
    return ms.dequantize(ms.decode(codes, "e2m1"), scales.astype(np.int64) - 127)


@pytest.mark.parametrize("M,N,K", [(300, 264, 384), (517, 520, 1024), (64, 8, 128)])
def test_gemm_mxfp4_accum_and_store(M, N, K):
    """E2M1 operands through the same epilogues: fp32 accumulate onto a prior
    and bf16 store, against the oracle's float64 product of the dequantised
    operands.  K 384 has an odd number of 64-byte stages (the last pair's
    second exponent row lies past the operand), K 128 a single stage."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(M + N + K + 1)
    ca, sa = random_mx4(rng, M, K)
    cb, sb = random_mx4(rng, N, K)
    A, B = mx4_values(ca, sa), mx4_values(cb, sb)
    ref = A @ B.T
    qa, qb = u8(ms.pack_fp4(ca)), u8(ms.pack_fp4(cb))
    prior = ci.fp32_prior((M, N), 5)
    D32 = f32(prior)
    coda.gemm_mx4([(coda.EPI_ACCUM_F32, 0, 1.0)], qa, u8(to_words(sa)), qb, u8(to_words(sb)), D32)
    D16 = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx4([(coda.EPI_STORE_BF16, 0, 0.0)], qa, u8(to_words(sa)), qb, u8(to_words(sb)), D16)
    torch.cuda.synchronize()
    bound = mfma_fp8_bound(A, B)
    got32 = to_np(D32).astype(np.float64) - prior
    assert np.all(np.abs(got32 - ref) <= bound + 2.0 ** -23 * (np.abs(ref) + np.abs(prior))), \
        float(np.max(np.abs(got32 - ref) - bound))
    got16 = to_np(D16).astype(np.float64)
    assert np.all(np.abs(got16 - ref) <= 1.01 * bound + 2.0 ** -8 * np.abs(ref)), \
        float(np.max(np.abs(got16 - ref) - bound))
    assert np.linalg.norm(got32 - ref) <= 1e-3 * np.linalg.norm(ref)


def test_gemm_mxfp4_one_scale_per_block():
    """Exponents that differ between every block of a row and between rows:
    a scale taken from the wrong block, stage or row moves the result by a
    power of two."""
    rng = np.random.default_rng(19)
    M, N, K = 256, 256, 512
    ca, _ = random_mx4(rng, M, K)
    cb, _ = random_mx4(rng, N, K)
    sa = (120 + (np.arange(K // 32)[None, :] * 3 + np.arange(M)[:, None]) % 15).astype(np.uint8)
    sb = (121 + (np.arange(K // 32)[None, :] * 5 + 2 * np.arange(N)[:, None]) % 13).astype(np.uint8)
    from oracle import mx_small as ms
    A, B = mx4_values(ca, sa), mx4_values(cb, sb)
    D32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    coda.gemm_mx4([(coda.EPI_ACCUM_F32, 0, 0.0)], u8(ms.pack_fp4(ca)), u8(to_words(sa)), u8(ms.pack_fp4(cb)),
                  u8(to_words(sb)), D32)
    torch.cuda.synchronize()
    ref = A @ B.T
    assert np.all(np.abs(to_np(D32) - ref) <= mfma_fp8_bound(A, B))
    assert np.linalg.norm(to_np(D32) - ref) <= 1e-3 * np.linalg.norm(ref)


def test_gemm_mxfp4_from_bf16_residual():
    """bf16 inputs quantised by the library (bit-exact against the oracle, as
    tested above), then the residual program out = z + a W on the MXFP4
    product, against the oracle's product of its own quantisation."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(29)
    M, N, K = 300, 520, 640
    a = ci.to_bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    w = ci.to_bf16_values((rng.standard_normal((N, K)) * K ** -0.5).astype(np.float32))
    z = ci.to_bf16_values(rng.standard_normal((M, N)).astype(np.float32))
    QA, SA = coda.quantize_mxfp4(bf(a), 1)
    QB, SB = coda.quantize_mxfp4(bf(w), 1)
    out = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx4([(coda.EPI_ADD_TILE, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)], QA, SA, QB, SB, out, aux=[bf(z)])
    torch.cuda.synchronize()
    PA, eA = ms.quantize(a, "e2m1")
    PB, eB = ms.quantize(w, "e2m1")
    A, B = ms.dequantize(PA, eA), ms.dequantize(PB, eB)
    ref = z.astype(np.float64) + A @ B.T
    got = to_np(out).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1.01 * mfma_fp8_bound(A, B) + 2.0 ** -8 * np.abs(ref) + 1e-30)
    assert np.linalg.norm(got - nm.bf16(ref)) <= 3e-3 * np.linalg.norm(ref)


def test_gemm_mxfp4_full_size_sampled():
    """The MXFP4 layer the bench times: M 4096, K 28672, N 8192 with residual;
    the library quantises a and W; 128 sampled outputs are recomputed by the
    oracle from its own MXFP4 copies of the sampled rows of a and columns of
    W (whose packed codes and exponents must equal the library's bit for bit)."""
    from oracle import mx_small as msm
    M, K, N = 4096, 28672, 8192
    rng = np.random.default_rng(73)
    a = ci.to_bf16_values(rng.standard_normal((M, K), dtype=np.float32))
    W = ci.to_bf16_values(rng.standard_normal((K, N), dtype=np.float32) * np.float32(K ** -0.5))
    z = ci.to_bf16_values(rng.standard_normal((M, N), dtype=np.float32))
    ag, Wg, zg = bf(a), bf(W), bf(z)
    Qa, Sa = coda.quantize_mxfp4(ag, 1)
    Qw, Sw = coda.quantize_mxfp4(Wg, 0)
    out = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx4([(coda.EPI_ADD_TILE, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)], Qa, Sa, Qw, Sw, out, aux=[zg])
    torch.cuda.synchronize()
    ms = rng.integers(0, M, 128)
    ns = rng.integers(0, N, 128)
    um, un = np.unique(ms), np.unique(ns)
    Pa, ea = msm.quantize(a[um], "e2m1")
    Pw, ew = msm.quantize(W[:, un].T.copy(), "e2m1")
    assert np.array_equal(Qa[torch.from_numpy(um).to(DEV)].cpu().numpy(), msm.pack_fp4(msm.encode(Pa, "e2m1")))
    assert np.array_equal(from_words(Sa.cpu().numpy(), M, K // 32)[um], (ea + 127).astype(np.uint8))
    assert np.array_equal(Qw[torch.from_numpy(un).to(DEV)].cpu().numpy(), msm.pack_fp4(msm.encode(Pw, "e2m1")))
    assert np.array_equal(from_words(Sw.cpu().numpy(), N, K // 32)[un], (ew + 127).astype(np.uint8))
    Ad, Bd = msm.dequantize(Pa, ea), msm.dequantize(Pw, ew)
    im, jn = np.searchsorted(um, ms), np.searchsorted(un, ns)
    acc = np.einsum("ik,ik->i", Ad[im], Bd[jn])
    bound = 2.0 ** -10 * np.einsum("ik,ik->i", np.abs(Ad[im]), np.abs(Bd[jn]))
    ref = z[ms, ns].astype(np.float64) + acc
    got = out[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1.01 * bound + 2.0 ** -8 * np.abs(ref)), float(np.max(np.abs(got - ref) - bound))
    assert_bf16("sampled out", got, nm.bf16(ref))


def test_gemm_mxfp4_degenerate_shapes():
    """Empty M or N is a no-op that leaves D untouched; a single row and the
    smallest K (128 values: one 64-byte stage, one exponent word row) match
    the oracle."""
    from oracle import mx_small as msm
    rng = np.random.default_rng(31)
    sentinel = torch.full((64, 64), 3.0, dtype=BF, device=DEV)
    for M, N in ((0, 64), (64, 0)):
        qa = torch.empty((max(M, 1), 64), dtype=torch.uint8, device=DEV)[:M]
        qb = torch.empty((max(N, 1), 64), dtype=torch.uint8, device=DEV)[:N]
        sa = torch.empty((1, 4 * max(M, 1)), dtype=torch.uint8, device=DEV)[:, :4 * M]
        sb = torch.empty((1, 4 * max(N, 1)), dtype=torch.uint8, device=DEV)[:, :4 * N]
        coda.gemm_mx4([(coda.EPI_STORE_BF16, 0, 0.0)], qa, sa, qb, sb, sentinel[:M, :N])
    torch.cuda.synchronize()
    assert bool((sentinel == 3.0).all())
    ca, sa = random_mx4(rng, 1, 128)
    cb, sb = random_mx4(rng, 40, 128)
    D = torch.empty((1, 40), dtype=torch.float32, device=DEV)
    coda.gemm_mx4([(coda.EPI_ACCUM_F32, 0, 0.0)], u8(msm.pack_fp4(ca)), u8(to_words(sa)), u8(msm.pack_fp4(cb)),
                  u8(to_words(sb)), D)
    torch.cuda.synchronize()
    A, B = mx4_values(ca, sa), mx4_values(cb, sb)
    ref = A @ B.T
    assert np.all(np.abs(to_np(D) - ref) <= mfma_fp8_bound(A, B) + 1e-30)


# ---------------------------------------------------------------- MXFP6
FP6 = ("e2m3", "e3m2")


def fp6_ladder_bf16(rng, R, C, axis, fmt):
    """varied_bf16 plus, in every fourth block along `axis`, the FP6 ties of
    `fmt`: a block maximum of exactly 2^emax (so the block's exponent is the
    power of two it was scaled by) and elements on every midpoint between
    neighbouring values of the format, both signs, values past the largest
    (which saturate) and small negatives that round to zero."""
    from oracle import mx_small as ms
    _, _, _, emax, vmax = ms.fmt_params(fmt)
    E, M, _ = ms.FORMATS[fmt]
    vals = np.unique(np.abs(ms.decode(np.arange(2 ** (1 + E + M)), fmt)))
    mids = (vals[:-1] + vals[1:]) / 2
    over = np.array([vmax + 2.0 ** (emax - M - 1), (vmax + 2.0 ** (emax + 1)) / 2])
    ties = np.concatenate([mids, -mids, over, -over, [-vals[1] / 4, 0.0]]).astype(np.float32)
    X = varied_bf16(rng, R, C, axis)
    Xt = X if axis == 1 else X.T
    nb = Xt.shape[1] // 32
    k = 0
    for r in range(1, Xt.shape[0], 3):        # row 0 keeps its all-zero block
        for b in range(0, nb, 4):
            s = np.float32(2.0 ** int(rng.integers(-10, 10)))
            blk = ties[(32 * k + np.arange(32)) % ties.size] * s
            blk[rng.integers(0, 32)] = 2.0 ** emax * s
            Xt[r, 32 * b:32 * b + 32] = blk
            k += 1
    return ci.to_bf16_values(X if axis == 1 else Xt.T)


@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("axis,R,C", [(1, 300, 480), (1, 5, 32), (0, 480, 296), (0, 64, 7 * 8)])
def test_mxfp6_quantiser_bit_exact(fmt, axis, R, C):
    """Packed FP6 codes (with their zero padding) and E8M0 exponents equal the
    oracle's (oracle/mx_small.py) bit for bit, in both orientations, with
    ragged tiles, an all-zero block, a block of very large values and every
    rounding tie and saturation of the format."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(60 + axis + 2 * FP6.index(fmt))
    X = fp6_ladder_bf16(rng, R, C, axis, fmt)
    Q, S = coda.quantize_mxfp6(bf(X), axis, fmt)
    torch.cuda.synchronize()
    Xr = X if axis == 1 else np.ascontiguousarray(X.T)
    P, e = ms.quantize(Xr, fmt)
    want_q = ms.pack_fp6(ms.encode(P, fmt))
    got_q = to_np(Q).astype(np.uint8)
    rows, L = Xr.shape
    assert got_q.shape == (rows, L)
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, (bad[:5], got_q[tuple(bad[0])], want_q[tuple(bad[0])])
    got_e = from_words(to_np(S), rows, L // 32)
    np.testing.assert_array_equal(got_e, (e + 127).astype(np.uint8))


def random_mx6(rng, rows, K, fmt, emin=117, emax=137):
    """An MXFP6 operand drawn directly: uniform codes (all 64) and E8M0 codes
    uniform in [emin, emax], independent per block; returns the codes
    [rows, K] and the exponent bytes [rows, K / 32]."""
    codes = rng.integers(0, 64, size=(rows, K)).astype(np.uint8)
    scales = rng.integers(emin, emax + 1, size=(rows, K // 32)).astype(np.uint8)
    return codes, scales


def mx6_values(codes, scales, fmt):
    from oracle import mx_small as ms
    return ms.dequantize(ms.decode(codes, fmt), scales.astype(np.int64) - 127)


@pytest.mark.parametrize("fmt", FP6)
@pytest.mark.parametrize("M,N,K", [(300, 264, 384), (517, 520, 1024), (64, 8, 128)])
def test_gemm_mxfp6_accum_and_store(fmt, M, N, K):
    """FP6 operands through the fp32 accumulate and bf16 store epilogues,
    against the oracle's float64 product of the dequantised operands; K 384
    has an odd number of 64-value stages, K 128 a single stage pair."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(M + N + K + 3 + FP6.index(fmt))
    ca, sa = random_mx6(rng, M, K, fmt)
    cb, sb = random_mx6(rng, N, K, fmt)
    A, B = mx6_values(ca, sa, fmt), mx6_values(cb, sb, fmt)
    ref = A @ B.T
    qa, qb = u8(ms.pack_fp6(ca)), u8(ms.pack_fp6(cb))
    prior = ci.fp32_prior((M, N), 6)
    D32 = f32(prior)
    coda.gemm_mx6([(coda.EPI_ACCUM_F32, 0, 1.0)], fmt, qa, u8(to_words(sa)), qb, u8(to_words(sb)), D32)
    D16 = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx6([(coda.EPI_STORE_BF16, 0, 0.0)], fmt, qa, u8(to_words(sa)), qb, u8(to_words(sb)), D16)
    torch.cuda.synchronize()
    bound = mfma_fp8_bound(A, B)
    got32 = to_np(D32).astype(np.float64) - prior
    assert np.all(np.abs(got32 - ref) <= bound + 2.0 ** -23 * (np.abs(ref) + np.abs(prior))), \
        float(np.max(np.abs(got32 - ref) - bound))
    got16 = to_np(D16).astype(np.float64)
    assert np.all(np.abs(got16 - ref) <= 1.01 * bound + 2.0 ** -8 * np.abs(ref)), \
        float(np.max(np.abs(got16 - ref) - bound))
    assert np.linalg.norm(got32 - ref) <= 1e-3 * np.linalg.norm(ref)


@pytest.mark.parametrize("fmt", FP6)
def test_gemm_mxfp6_one_scale_per_block(fmt):
    """Exponents that differ between every block of a row and between rows
    (a scale from the wrong block, stage or row moves the result by a power
    of two), and padding bytes that are not zero (the matrix core must not
    read them)."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(23 + FP6.index(fmt))
    M, N, K = 256, 256, 512
    ca, _ = random_mx6(rng, M, K, fmt)
    cb, _ = random_mx6(rng, N, K, fmt)
    sa = (120 + (np.arange(K // 32)[None, :] * 3 + np.arange(M)[:, None]) % 15).astype(np.uint8)
    sb = (121 + (np.arange(K // 32)[None, :] * 5 + 2 * np.arange(N)[:, None]) % 13).astype(np.uint8)
    A, B = mx6_values(ca, sa, fmt), mx6_values(cb, sb, fmt)
    pa, pb = ms.pack_fp6(ca), ms.pack_fp6(cb)
    pad = (np.arange(K) % 32) >= 24
    pa[:, pad] = 0xA5
    pb[:, pad] = 0x5A
    D32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    coda.gemm_mx6([(coda.EPI_ACCUM_F32, 0, 0.0)], fmt, u8(pa), u8(to_words(sa)), u8(pb), u8(to_words(sb)), D32)
    torch.cuda.synchronize()
    ref = A @ B.T
    assert np.all(np.abs(to_np(D32) - ref) <= mfma_fp8_bound(A, B))
    assert np.linalg.norm(to_np(D32) - ref) <= 1e-3 * np.linalg.norm(ref)


@pytest.mark.parametrize("fmt", FP6)
def test_gemm_mxfp6_from_bf16_epilogues(fmt):
    """bf16 inputs quantised by the library (bit-exact against the oracle, as
    tested above), then the residual program out = z + a W and the SwiGLU
    program with given row factors on the MXFP6 product, against the
    oracle's product of its own quantisation."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(37 + FP6.index(fmt))
    M, N, K = 300, 576, 640       # SwiGLU packs gate/up in 64-column groups
    a = ci.to_bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    w = ci.to_bf16_values((rng.standard_normal((N, K)) * K ** -0.5).astype(np.float32))
    z = ci.to_bf16_values(rng.standard_normal((M, N)).astype(np.float32))
    QA, SA = coda.quantize_mxfp6(bf(a), 1, fmt)
    QB, SB = coda.quantize_mxfp6(bf(w), 1, fmt)
    out = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx6([(coda.EPI_ADD_TILE, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)], fmt, QA, SA, QB, SB, out,
                  aux=[bf(z)])
    r = rng.uniform(0.5, 2, M).astype(np.float32)
    D3 = torch.empty((M, N // 2), dtype=BF, device=DEV)
    coda.gemm_mx6([(coda.EPI_ROW_SCALE, 0, 0.0), (coda.EPI_SWIGLU, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)],
                  fmt, QA, SA, QB, SB, D3, aux=[f32(r)])
    torch.cuda.synchronize()
    PA, eA = ms.quantize(a, fmt)
    PB, eB = ms.quantize(w, fmt)
    A, B = ms.dequantize(PA, eA), ms.dequantize(PB, eB)
    acc = A @ B.T
    ref = z.astype(np.float64) + acc
    got = to_np(out).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1.01 * mfma_fp8_bound(A, B) + 2.0 ** -8 * np.abs(ref) + 1e-30)
    assert np.linalg.norm(got - nm.bf16(ref)) <= 3e-3 * np.linalg.norm(ref)
    hg, hu = unpack_gu(r[:, None] * acc)
    assert_bf16("swiglu", to_np(D3), nm.bf16(ops.swiglu(hg, hu)))


@pytest.mark.parametrize("fmt", FP6)
def test_gemm_mxfp6_degenerate_shapes(fmt):
    """Empty M or N is a no-op that leaves D untouched; a single row and the
    smallest K (128 values: one stage pair, one exponent word row) match the
    oracle."""
    from oracle import mx_small as msm
    rng = np.random.default_rng(41 + FP6.index(fmt))
    sentinel = torch.full((64, 64), 3.0, dtype=BF, device=DEV)
    for M, N in ((0, 64), (64, 0)):
        qa = torch.empty((max(M, 1), 128), dtype=torch.uint8, device=DEV)[:M]
        qb = torch.empty((max(N, 1), 128), dtype=torch.uint8, device=DEV)[:N]
        sa = torch.empty((1, 4 * max(M, 1)), dtype=torch.uint8, device=DEV)[:, :4 * M]
        sb = torch.empty((1, 4 * max(N, 1)), dtype=torch.uint8, device=DEV)[:, :4 * N]
        coda.gemm_mx6([(coda.EPI_STORE_BF16, 0, 0.0)], fmt, qa, sa, qb, sb, sentinel[:M, :N])
    torch.cuda.synchronize()
    assert bool((sentinel == 3.0).all())
    ca, sa = random_mx6(rng, 1, 128, fmt)
    cb, sb = random_mx6(rng, 40, 128, fmt)
    D = torch.empty((1, 40), dtype=torch.float32, device=DEV)
    coda.gemm_mx6([(coda.EPI_ACCUM_F32, 0, 0.0)], fmt, u8(msm.pack_fp6(ca)), u8(to_words(sa)),
                  u8(msm.pack_fp6(cb)), u8(to_words(sb)), D)
    torch.cuda.synchronize()
    A, B = mx6_values(ca, sa, fmt), mx6_values(cb, sb, fmt)
    ref = A @ B.T
    assert np.all(np.abs(to_np(D) - ref) <= mfma_fp8_bound(A, B) + 1e-30)


def test_gemm_mxfp6_full_size_sampled():
    """The MXFP4 full-size layer with E2M3 operands: M 4096, K 28672, N 8192
    with residual; the library quantises a and W; 128 sampled outputs are
    recomputed by the oracle from its own MXFP6 copies of the sampled rows
    of a and columns of W (whose packed codes and exponents must equal the
    library's bit for bit)."""
    from oracle import mx_small as msm
    fmt = "e2m3"
    M, K, N = 4096, 28672, 8192
    rng = np.random.default_rng(79)
    a = ci.to_bf16_values(rng.standard_normal((M, K), dtype=np.float32))
    W = ci.to_bf16_values(rng.standard_normal((K, N), dtype=np.float32) * np.float32(K ** -0.5))
    z = ci.to_bf16_values(rng.standard_normal((M, N), dtype=np.float32))
    ag, Wg, zg = bf(a), bf(W), bf(z)
    Qa, Sa = coda.quantize_mxfp6(ag, 1, fmt)
    Qw, Sw = coda.quantize_mxfp6(Wg, 0, fmt)
    out = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx6([(coda.EPI_ADD_TILE, 0, 0.0), (coda.EPI_STORE_BF16, 0, 0.0)], fmt, Qa, Sa, Qw, Sw, out, aux=[zg])
    torch.cuda.synchronize()
    ms = rng.integers(0, M, 128)
    ns = rng.integers(0, N, 128)
    um, un = np.unique(ms), np.unique(ns)
    Pa, ea = msm.quantize(a[um], fmt)
    Pw, ew = msm.quantize(W[:, un].T.copy(), fmt)
    assert np.array_equal(Qa[torch.from_numpy(um).to(DEV)].cpu().numpy(), msm.pack_fp6(msm.encode(Pa, fmt)))
    assert np.array_equal(from_words(Sa.cpu().numpy(), M, K // 32)[um], (ea + 127).astype(np.uint8))
    assert np.array_equal(Qw[torch.from_numpy(un).to(DEV)].cpu().numpy(), msm.pack_fp6(msm.encode(Pw, fmt)))
    assert np.array_equal(from_words(Sw.cpu().numpy(), N, K // 32)[un], (ew + 127).astype(np.uint8))
    Ad, Bd = msm.dequantize(Pa, ea), msm.dequantize(Pw, ew)
    im, jn = np.searchsorted(um, ms), np.searchsorted(un, ns)
    acc = np.einsum("ik,ik->i", Ad[im], Bd[jn])
    bound = 2.0 ** -10 * np.einsum("ik,ik->i", np.abs(Ad[im]), np.abs(Bd[jn]))
    ref = z[ms, ns].astype(np.float64) + acc
    got = out[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1.01 * bound + 2.0 ** -8 * np.abs(ref)), float(np.max(np.abs(got - ref) - bound))
    assert_bf16("sampled out", got, nm.bf16(ref))


@pytest.mark.parametrize("fmt", FP6)
def test_gemm_mxfp6_remaining_chains(fmt):
    """The other forward programs compiled for FP6 operands, on operands the
    library quantised (bit-exact against the oracle, as tested above):
    row/column scales, residual + sum-of-squares partials, sigmoid with its
    saved pre-activation, and RMS-from-partials + QK-norm + RoPE on a QKV
    layer (two heads of 128), against the oracle's float64 product of its
    own quantisation with the same epilogue formulas."""
    from oracle import mx_small as ms
    rng = np.random.default_rng(47 + FP6.index(fmt))
    M, K, Dh, seq = 300, 256, 256, 100
    N = 3 * Dh
    x = ci.to_bf16_values(rng.standard_normal((M, K)).astype(np.float32))
    W = ci.to_bf16_values((rng.standard_normal((N, K)) * K ** -0.5).astype(np.float32))   # stored [N, K]
    QA, SA = coda.quantize_mxfp6(bf(x), 1, fmt)
    QB, SB = coda.quantize_mxfp6(bf(W), 1, fmt)
    PA, eA = ms.quantize(x, fmt)
    PB, eB = ms.quantize(W, fmt)
    acc = ms.dequantize(PA, eA) @ ms.dequantize(PB, eB).T
    E = coda

    rv = rng.uniform(0.5, 2, M).astype(np.float32)
    cv = rng.uniform(0.5, 2, N).astype(np.float32)
    D1 = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx6([(E.EPI_ROW_SCALE, 0, 0.0), (E.EPI_COL_SCALE, 1, 0.0), (E.EPI_STORE_BF16, 0, 0.0)], fmt,
                  QA, SA, QB, SB, D1, aux=[f32(rv), f32(cv)])
    Z = ci.to_bf16_values(rng.standard_normal((M, N)).astype(np.float32))
    P = torch.empty((coda.partials_cols(N), M), dtype=torch.float32, device=DEV)
    D2 = torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx6([(E.EPI_ADD_TILE, 0, 0.0), (E.EPI_STORE_BF16, 0, 0.0), (E.EPI_ROW_SUMSQ_PARTIAL, 1, 0.0)], fmt,
                  QA, SA, QB, SB, D2, aux=[bf(Z), P])
    r = rng.uniform(0.5, 2, M).astype(np.float32)
    D3, h = torch.empty((M, N), dtype=BF, device=DEV), torch.empty((M, N), dtype=BF, device=DEV)
    coda.gemm_mx6([(E.EPI_ROW_SCALE, 0, 0.0), (E.EPI_SAVE_PRE, 1, 0.0), (E.EPI_SIGMOID, 0, 0.0),
                   (E.EPI_STORE_BF16, 0, 0.0)], fmt, QA, SA, QB, SB, D3, aux=[f32(r), h])
    gains = (1 + 0.1 * rng.standard_normal((2, 128))).astype(np.float32)
    table = torch.empty((seq, 128), dtype=torch.float32, device=DEV)
    coda.rope_table(seq, table)
    Px = np.stack([(x.astype(np.float64) ** 2)[:, :K // 2].sum(axis=1),
                   (x.astype(np.float64) ** 2)[:, K // 2:].sum(axis=1)]).astype(np.float32)
    D4, r4, save = (torch.empty((M, N), dtype=BF, device=DEV), torch.empty(M, dtype=torch.float32, device=DEV),
                    torch.empty((M, 2 * Dh), dtype=BF, device=DEV))
    coda.gemm_mx6([(E.EPI_ROW_RMS_FROM_PARTIALS, 0, 1e-6), (E.EPI_STORE_ROW_VEC, 1, 0.0), (E.EPI_SAVE_PRE, 2, 0.0),
                   (E.EPI_QKNORM_ROPE, (3, 4), 1e-6), (E.EPI_STORE_BF16, 0, 0.0)], fmt, QA, SA, QB, SB, D4,
                  aux=[f32(Px), r4, save, f32(gains), table])
    torch.cuda.synchronize()

    assert_bf16("row/col scaled", to_np(D1), nm.bf16((acc * rv[:, None]) * cv[None, :]))
    y = nm.bf16(Z + acc)
    assert_bf16("residual", to_np(D2), y)
    assert_grad("sumsq partials", to_np(P), ob.tile_partials(y.astype(np.float64) ** 2, 256))
    hh = r[:, None] * acc
    assert_bf16("sigmoid h", to_np(h), nm.bf16(hh))
    assert_bf16("sigmoid", to_np(D3), nm.bf16(ops.sigmoid(hh)))
    rr = ops.inv_rms(x, 1e-6)
    assert_grad("r", to_np(r4), rr)
    t = rr[:, None] * acc
    cos, sin = ops.rope_tables(seq, 128, 5e5)
    pos = np.arange(M) % seq
    got = to_np(D4)
    assert_bf16("q", got[:, :Dh], nm.bf16(ops.rope(ops.qk_norm(t[:, :Dh], gains[0], 1e-6), pos, cos, sin)))
    assert_bf16("k", got[:, Dh:2 * Dh], nm.bf16(ops.rope(ops.qk_norm(t[:, Dh:2 * Dh], gains[1], 1e-6), pos, cos, sin)))
    assert_bf16("v", got[:, 2 * Dh:], nm.bf16(t[:, 2 * Dh:]))
    assert_bf16("q_pre|k_pre", to_np(save), nm.bf16(t[:, :2 * Dh]))
