"""Pins for the oracle's number formats (CPU only).

bf16: against torch's CPU bfloat16 cast (a library routine) on random values
over the whole exponent range and on edge patterns.  E4M3FN: exhaustive
decoding of the 256 codes from the OCP format definition, round trips,
ties-to-even midpoints, and torch's CPU float8_e4m3fn cast on |v| <= 448.
"""
import numpy as np
import pytest
import torch

from oracle import numerics as nm


def _torch_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def test_bf16_matches_torch_random():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    got, ref = nm.bf16(x), _torch_bf16(x)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_edge_patterns():
    e = np.float32
    cases = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 2 ** -8),
                      1e-40, -1e-41, 2 ** -133, 3.3895313892515355e38, np.finfo(np.float32).max,
                      np.inf, -np.inf, np.nan, 0.0, -0.0, 65504.0, 1.0 / 3.0], dtype=e)
    got, ref = nm.bf16(cases), _torch_bf16(cases)
    assert np.array_equal(got, ref, equal_nan=True)
    assert nm.bf16(e(1 + 2 ** -8)) == 1.0              # tie rounds to even (down)
    assert nm.bf16(e(1 + 3 * 2 ** -8)) == e(1 + 2 ** -6)  # tie rounds to even (up)
    assert np.isinf(nm.bf16(np.finfo(np.float32).max))  # overflow rounds to inf
    assert nm.bf16_bits(e(1.0)) == 0x3F80


def test_e4m3_decode_exhaustive():
    v = nm.e4m3_decode(np.arange(256))
    finite = v[np.isfinite(v)]
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert len(finite) == 254
    assert finite.max() == 448.0 and finite.min() == -448.0
    assert v[1] == 2.0 ** -9                      # smallest subnormal
    assert v[8] == 2.0 ** -6                      # smallest normal
    assert v[0x38] == 1.0                         # exponent field 7 = bias
    pos = v[0:0x7F]
    assert np.all(np.diff(pos) > 0)               # codes are ordered
    assert np.array_equal(v[0x80:0xFF], -v[0:0x7F])


def test_e4m3_round_trip_all_codes():
    v = nm.e4m3_decode(np.arange(256))
    fin = np.isfinite(v)
    assert np.array_equal(nm.e4m3(v[fin]), v[fin])
    codes = nm.e4m3_codes(v[fin])
    assert np.array_equal(nm.e4m3_decode(codes), v[fin])


def test_e4m3_midpoints_ties_to_even():
    v = nm.e4m3_decode(np.arange(0, 0x7F)).astype(np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    got = nm.e4m3(mids)
    codes = nm.e4m3_codes(got)
    assert np.all(codes % 2 == 0)                 # even mantissa wins every tie
    nudged_up = nm.e4m3(np.nextafter(mids, np.float32(np.inf)))
    assert np.array_equal(nudged_up, v[1:].astype(np.float32))


def test_e4m3_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(500_000).astype(np.float32) * 50,
                        rng.uniform(-448, 448, 500_000).astype(np.float32),
                        (rng.standard_normal(200_000) * 1e-2).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(nm.e4m3(x), ref)


def test_e4m3_clamps():
    assert nm.e4m3(np.float32(1e6)) == 448.0
    assert nm.e4m3(np.float32(-465.0)) == -448.0


def test_quantize_axes_and_scales():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((6, 40)).astype(np.float32) * np.array([1e-3, 1, 10, 100, 0, 5], np.float32)[:, None]
    Q, s = nm.quantize_e4m3(A, axis=1)
    assert s.shape == (6,)
    assert s[4] == 1.0 and np.all(Q[4] == 0)       # all-zero row
    for i in (0, 1, 2, 3, 5):
        amax = np.abs(A[i]).max()
        assert s[i] == np.float32(amax) / np.float32(448)
        assert np.abs(Q[i]).max() == 448.0        # the amax maps onto the top code
        rel = np.abs(Q[i] * s[i] - A[i]) / amax
        assert rel.max() <= 2.0 ** -4 * 448 / 256 + 1e-6  # half a grid step at the top binade
    Qc, sc = nm.quantize_e4m3(A.T, axis=0)          # per column of the transpose
    assert np.array_equal(Qc, Q.T) and np.array_equal(sc, s)
