"""Pins of the MXFP4 / MXFP6 oracle (oracle/mx_small.py) against things
other than itself: the element values the MX specification tabulates, a
brute-force nearest search over every code, exact round trips of values that
are already MX, and a triple-loop matrix product."""
import numpy as np
import pytest

from oracle import mx_small as ms

FMTS = ("e2m1", "e2m3", "e3m2")


def all_codes(fmt):
    E, M, _ = ms.FORMATS[fmt]
    return np.arange(2 ** (1 + E + M))


def test_e2m1_values_table():
    # the eight magnitudes of FP4 E2M1 as the MX specification lists them
    np.testing.assert_array_equal(ms.decode(np.arange(8), "e2m1"), [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    np.testing.assert_array_equal(ms.decode(np.arange(8, 16), "e2m1"), -np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6]))


@pytest.mark.parametrize("fmt,vmax,vmin_sub,emax", [("e2m3", 7.5, 0.125, 2), ("e3m2", 28.0, 0.0625, 4),
                                                    ("e2m1", 6.0, 0.5, 2)])
def test_fp6_fp4_extremes(fmt, vmax, vmin_sub, emax):
    v = ms.decode(all_codes(fmt), fmt)
    assert v.max() == vmax and v.min() == -vmax
    assert np.min(v[v > 0]) == vmin_sub
    assert ms.fmt_params(fmt)[3] == emax


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_decode_round_trip(fmt):
    c = all_codes(fmt)
    E, M, _ = ms.FORMATS[fmt]
    neg_zero = 1 << (E + M)
    c = c[c != neg_zero]
    np.testing.assert_array_equal(ms.encode(ms.decode(c, fmt), fmt), c)


@pytest.mark.parametrize("fmt", FMTS)
def test_round_nearest_even_brute_force(fmt):
    """round_elem(x) is the nearest code value (after saturation), ties to
    the code with an even mantissa, on random values and on every midpoint
    between neighbouring values."""
    E, M, _ = ms.FORMATS[fmt]
    vals = ms.decode(all_codes(fmt), fmt)
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(5)
    xs = np.concatenate([mids, -mids, rng.standard_normal(400) * pos.max() * 0.6, [pos.max() * 1.3, -1e9, 0.0]])
    got = ms.round_elem(xs, fmt)
    codes = all_codes(fmt)
    for x, g in zip(xs, got):
        t = min(max(x, -pos.max()), pos.max())
        d = np.abs(vals - t)
        best = codes[d == d.min()]
        if len(best) > 1:
            best = [c for c in best if c % 2 == 0] or best
        want = ms.decode(best[0], fmt)
        assert g == want or (g == 0 and want == 0), (fmt, x, g, want)


@pytest.mark.parametrize("fmt", FMTS)
def test_block_max_lands_in_top_binade(fmt):
    emax = ms.fmt_params(fmt)[3]
    rng = np.random.default_rng(6)
    X = (rng.standard_normal((30, 96)) * np.exp2(rng.integers(-30, 30, size=(30, 1)))).astype(np.float32)
    e = ms.block_exponents(X, fmt)
    amax = np.abs(X.reshape(30, 3, 32)).max(axis=2) / np.exp2(e.astype(np.float64))
    assert np.all((amax >= 2.0 ** emax) & (amax < 2.0 ** (emax + 1)))


@pytest.mark.parametrize("fmt", FMTS)
def test_exact_round_trip(fmt):
    """Blocks that are already MX (element values with one of them in the top
    binade, times 2^e) come back unchanged, with that exponent."""
    emax = ms.fmt_params(fmt)[3]
    vals = ms.decode(all_codes(fmt), fmt)
    top = vals[np.abs(vals) >= 2.0 ** emax]
    rng = np.random.default_rng(7)
    X = np.empty((4, 64))
    E = rng.integers(-60, 60, size=(4, 2))
    for r in range(4):
        for b in range(2):
            blk = np.concatenate([[rng.choice(top)], rng.choice(vals, size=31)])
            rng.shuffle(blk)
            X[r, 32 * b:32 * b + 32] = blk * 2.0 ** E[r, b]
    P, e = ms.quantize(X.astype(np.float32), fmt)
    np.testing.assert_array_equal(e, E)
    np.testing.assert_array_equal(ms.dequantize(P, e), X)


def test_zero_block_and_saturation():
    X = np.zeros((1, 64), dtype=np.float32)
    X[0, 32] = 7.5          # block max 7.5: e = 2 - 2 = 0, 7.5 saturates to 6
    X[0, 33] = -0.3         # -0.3 -> -0.5 (nearest; 0.25 would tie to 0)
    X[0, 34] = 0.25         # a tie between 0 and 0.5: 0 (even)
    X[0, 35] = 5.0          # a tie between 4 and 6: 4 (even mantissa)
    P, e = ms.quantize(X, "e2m1")
    assert e[0, 0] == -127 and e[0, 1] == 0
    assert np.all(P[0, :32] == 0)
    assert list(P[0, 32:36]) == [6.0, -0.5, 0.0, 4.0]


def test_fp4_packing_order():
    codes = np.array([[1, 2, 15, 0]], dtype=np.uint8)
    b = ms.pack_fp4(codes)
    assert b.tolist() == [[0x21, 0x0F]]
    np.testing.assert_array_equal(ms.unpack_fp4(b), codes)


def test_fp6_packing_order():
    # worked by hand: code 1 at bits 0-5, code 2 at bits 6-11, code 3 at 12-17
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, :3] = [1, 2, 3]
    b = ms.pack_fp6(codes)
    assert b[0, :3].tolist() == [0x81, 0x30, 0x00]
    assert np.all(b[0, 3:] == 0)
    # the last code sits in the top six bits of byte 23; bytes 24-31 stay zero
    codes = np.zeros((2, 64), dtype=np.uint8)
    codes[0, 31] = 0x3F
    codes[1, 32:] = 0x3F
    b = ms.pack_fp6(codes)
    assert b[0, 23] == 0xFC and np.count_nonzero(b[0]) == 1
    assert np.all(b[1, :32] == 0) and np.all(b[1, 32:56] == 0xFF) and np.all(b[1, 56:] == 0)
    rng = np.random.default_rng(5)
    c = rng.integers(0, 64, size=(3, 96)).astype(np.uint8)
    np.testing.assert_array_equal(ms.unpack_fp6(ms.pack_fp6(c)), c)


def test_matmul_triple_loop():
    rng = np.random.default_rng(8)
    A = rng.standard_normal((3, 64)).astype(np.float32)
    B = rng.standard_normal((4, 64)).astype(np.float32)
    PA, eA = ms.quantize(A, "e2m1")
    PB, eB = ms.quantize(B, "e2m1")
    C = ms.matmul_nt(PA, eA, PB, eB)
    for m in range(3):
        for n in range(4):
            ref = 0.0
            for k in range(64):
                ref += float(PA[m, k]) * 2.0 ** eA[m, k // 32] * float(PB[n, k]) * 2.0 ** eB[n, k // 32]
            assert C[m, n] == pytest.approx(ref, rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("mode,fmt", [("mx4", "e2m1"), ("mx6_e2m3", "e2m3"), ("mx6_e3m2", "e3m2")])
def test_block_gemm_mx_small_mode_axes(mode, fmt):
    """oracle.block.mm(A, B, mode) quantises A along its rows and B down its
    columns in the mode's element format: operands that are already MX in
    that format along those axes come back as the exact product; quantising
    B along its rows instead changes it."""
    from oracle import block as ob
    rng = np.random.default_rng(11)
    vals = ms.decode(all_codes(fmt), fmt)
    emax = ms.fmt_params(fmt)[3]
    top = vals[np.abs(vals) >= 2.0 ** emax]     # a block maximum in the top binade keeps the exponent

    def mx4_rows(rows, nblocks):
        X = np.empty((rows, 32 * nblocks))
        for r in range(rows):
            for b in range(nblocks):
                blk = np.concatenate([[rng.choice(top)], rng.choice(vals, size=31)])
                rng.shuffle(blk)
                X[r, 32 * b:32 * b + 32] = blk * 2.0 ** rng.integers(-6, 2)
        return X.astype(np.float32)

    A = mx4_rows(5, 3)
    B = np.ascontiguousarray(mx4_rows(64, 3).T)       # [96, 64], MX down its columns
    got = ob.mm(A, B, mode)
    ref = (A.astype(np.float64) @ B.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(got, ref)
    P, e = ms.quantize(B, fmt)
    assert not np.array_equal(ms.dequantize(P, e), B.astype(np.float64))
