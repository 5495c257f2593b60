"""Pins of the MXFP8 oracle (oracle/mx.py) against things other than itself:
exact round trips of values that are already MXFP8, a brute-force nearest
search over every E4M3 code, the E8M0 codes against torch's float8_e8m0fnu
cast, and a triple-loop matrix product."""
import numpy as np
import pytest

from oracle import mx
from oracle.numerics import e4m3_decode

FINITE = np.array([c for c in range(256) if not np.isnan(e4m3_decode(c))], dtype=np.int64)
VALUES = e4m3_decode(FINITE).astype(np.float64)


def _mx_blocks(rng, rows, nblocks):
    """Values that are exactly MXFP8 with a known shared exponent: each block
    holds E4M3 values whose largest magnitude lies in [256, 448], times 2^e."""
    big = VALUES[(np.abs(VALUES) >= 256)]
    X = np.empty((rows, nblocks * 32))
    E = rng.integers(-100, 100, size=(rows, nblocks))
    for r in range(rows):
        for b in range(nblocks):
            top = rng.choice(big)
            small = rng.choice(VALUES[np.abs(VALUES) <= abs(top)], size=31)
            blk = np.concatenate([[top], small])
            rng.shuffle(blk)
            X[r, 32 * b:32 * b + 32] = blk * 2.0 ** E[r, b]
    return X.astype(np.float32), E


def test_exact_round_trip():
    rng = np.random.default_rng(1)
    X, E = _mx_blocks(rng, 6, 5)
    P, e = mx.quantize(X)
    np.testing.assert_array_equal(e, E)
    np.testing.assert_array_equal(mx.dequantize(P, e), X.astype(np.float64))


def test_exponent_puts_block_max_in_256_512():
    rng = np.random.default_rng(2)
    X = (rng.standard_normal((40, 64)) * np.exp2(rng.integers(-20, 20, size=(40, 1)))).astype(np.float32)
    e = mx.block_exponents(X)
    amax = np.abs(X.reshape(40, 2, 32)).max(axis=2)
    scaled = amax / np.exp2(e.astype(np.float64))
    assert np.all((scaled >= 256) & (scaled < 512))


def test_nearest_code_brute_force():
    """Every element is the nearest point of {2^e v : v an E4M3 value} to x,
    ties to the even code, after saturation at 448."""
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((4, 64)) * 3).astype(np.float32)
    P, e = mx.quantize(X)
    codes = mx.codes(P)
    for r in range(4):
        for k in range(64):
            s = 2.0 ** e[r, k // 32]
            t = min(max(float(X[r, k]) / s, -448.0), 448.0)
            d = np.abs(VALUES - t)
            best = FINITE[d == d.min()]
            if len(best) > 1:                      # a tie: the even mantissa wins
                best = [c for c in best if c % 2 == 0]
            got = int(codes[r, k])
            want = int(best[0])
            if VALUES[FINITE == want][0] == 0:     # +0 and -0 are both nearest to 0
                assert e4m3_decode(got) == 0
            else:
                assert got == want, (r, k, X[r, k], got, want)


def test_zero_block_and_saturation():
    X = np.zeros((2, 64), dtype=np.float32)
    X[1, 32] = 1.9 * 2.0 ** 5          # block max 1.9 * 2^5: scaled 486.4 saturates
    X[1, 33] = -1.0
    P, e = mx.quantize(X)
    assert e[0, 0] == -127 and e[0, 1] == -127 and e[1, 0] == -127
    assert np.all(P[0] == 0) and np.all(P[1, :32] == 0)
    assert e[1, 1] == 5 - 8
    assert P[1, 32] == 448.0
    assert P[1, 33] == -8.0             # -1 / 2^-3


def test_e8m0_codes_match_torch():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e8m0fnu"):
        pytest.skip("no float8_e8m0fnu in this torch")
    e = np.arange(-127, 128)
    codes = mx.e8m0_codes(e)
    vals = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e8m0fnu).float().numpy()
    np.testing.assert_array_equal(vals.astype(np.float64), np.exp2(e.astype(np.float64)))


def test_matmul_triple_loop():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((3, 64)).astype(np.float32)
    B = rng.standard_normal((5, 64)).astype(np.float32)
    PA, eA = mx.quantize(A)
    PB, eB = mx.quantize(B)
    C = mx.matmul_nt(PA, eA, PB, eB)
    for m in range(3):
        for n in range(5):
            ref = 0.0
            for k in range(64):
                ref += float(PA[m, k]) * 2.0 ** eA[m, k // 32] * float(PB[n, k]) * 2.0 ** eB[n, k // 32]
            assert C[m, n] == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_block_gemm_mx_mode_axes():
    """oracle.block.mm(A, B, "mx") quantises A along its rows and B down its
    columns (the contracted axis of both): operands that are already MXFP8
    along those axes come back as the exact product; quantising B along its
    rows instead would have changed it."""
    from oracle import block as ob
    rng = np.random.default_rng(9)

    def mx_rows(rows, nblocks):
        # E4M3 values with a block maximum in [256, 448], times 2^e, e small
        big = VALUES[np.abs(VALUES) >= 256]
        X = np.empty((rows, 32 * nblocks))
        for r in range(rows):
            for b in range(nblocks):
                top = rng.choice(big)
                blk = np.concatenate([[top], rng.choice(VALUES[np.abs(VALUES) <= abs(top)], size=31)])
                rng.shuffle(blk)
                X[r, 32 * b:32 * b + 32] = blk * 2.0 ** rng.integers(-12, -6)
        return X.astype(np.float32)

    A = mx_rows(5, 3)                            # [5, 96], MXFP8 along K
    Bt = mx_rows(64, 3)                          # B = Bt^T [96, 64], MXFP8 down its columns
    B = np.ascontiguousarray(Bt.T)
    got = ob.mm(A, B, "mx")
    ref = (A.astype(np.float64) @ B.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(got, ref)
    P, e = mx.quantize(B)                        # the wrong axis: blocks along B's rows
    assert not np.array_equal(mx.dequantize(P, e), B.astype(np.float64))
