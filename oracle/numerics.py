"""Number formats used by the oracle: bf16 and OCP E4M3FN rounding, and the
amax-scaled fp8 quantiser.

Test infrastructure only: the oracle is imported by tests, by the smoke check
and by the benchmark's CPU-baseline leg, never by the product path.

The bf16 rounding is written from the format's definition (keep the top 16
bits of the IEEE-754 binary32 pattern, round to nearest, ties to even).  The
E4M3FN rounding is written from the OCP 8-bit floating point definition
(1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, the
all-ones pattern is NaN, largest finite value 448).  Both are pinned against
torch's CPU casts and exhaustive code round trips in tests/test_oracle_numerics.py.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even).

    Returns float32 values that are exactly representable in bf16.  NaN stays
    NaN, infinities stay infinite, values above the largest bf16 round to inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = r.astype(np.uint32).view(np.float32).reshape(x.shape)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32("nan")
    return out


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16(x)."""
    return (bf16(x).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3FN byte code (float32; the NaN codes give NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    v = np.where(e == 0, sub, nor) * sign
    v = np.where((e == 0xF) & (m == 0x7), np.nan, v)
    return v.astype(np.float32)


def e4m3(x) -> np.ndarray:
    """Round float32 values (|x| <= 448 expected) to the nearest E4M3FN value,
    ties to even.  Values beyond +-448 are clamped first: the quantiser below
    always clamps, so this never produces the NaN pattern.
    """
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    ax = np.abs(x)
    # spacing of the grid around |x|: 2^(e-3) in the binade [2^e, 2^(e+1)),
    # and 2^-9 below the smallest normal 2^-6 (the subnormal range)
    _, ex = np.frexp(np.where(ax > 0, ax, 1.0))     # ax = f * 2^ex, f in [0.5, 1)
    binade = ex - 1
    quantum = np.exp2(np.maximum(binade, -6) - 3.0)
    q = np.rint(x / quantum) * quantum                # rint: ties to even
    return q.astype(np.float32)


def e4m3_codes(x) -> np.ndarray:
    """Byte codes (uint8) of e4m3(x)."""
    v = e4m3(x).astype(np.float64)
    table = e4m3_decode(np.arange(256)).astype(np.float64)
    # map every finite value to its code: positive codes 0..126, negative 128..254
    pos = {float(table[c]): c for c in range(0, 127)}
    neg = {float(table[c]): c for c in range(129, 255)}
    neg[-0.0] = 128
    flat = v.ravel()
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, val in enumerate(flat):
        if val > 0 or (val == 0 and not np.signbit(val)):
            out[i] = pos[val]
        else:
            out[i] = neg[val] if val != 0 else 128
    return out.reshape(v.shape)


def quantize_e4m3(X, axis: int):
    """Amax-scaled E4M3FN quantisation.

    The amax is taken over ``axis`` (the axis that the GEMM contracts), so one
    scale belongs to each index of the other axis.  With amax > 0:
    ``mult = fp32(448 / amax)``, ``Q = e4m3(clamp(fp32(X * mult), +-448))`` and
    ``s = fp32(amax / 448)``; an all-zero line uses ``s = 1`` (and Q = 0).
    Dequantised value: ``Q * s``.  Returns (Q as float32 values, s float32 with
    ``axis`` removed).
    """
    X = np.asarray(X, dtype=np.float32)
    amax = np.max(np.abs(X), axis=axis, keepdims=True).astype(np.float32)
    amax = np.where(amax > 0, amax, np.float32(E4M3_MAX)).astype(np.float32)
    mult = (np.float32(E4M3_MAX) / amax).astype(np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    prod = (X * mult).astype(np.float32)
    Q = e4m3(np.clip(prod, -E4M3_MAX, E4M3_MAX))
    return Q, np.squeeze(s, axis=axis)
