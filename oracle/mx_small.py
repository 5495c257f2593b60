"""Block-scaled FP4 and FP6 operands (MXFP4, MXFP6) for the oracle.

Test infrastructure only: imported by tests, never by the product path.

Written from the OCP Microscaling Formats (MX) Specification v1.0 (the
element data types FP6 E2M3, FP6 E3M2 and FP4 E2M1, and the conversion of a
block to MX): 32 consecutive elements along the contracted axis share one
E8M0 scale 2^e, and for a block V
    e = floor(log2(max |V_i|)) - emax       (emax: exponent of the element
                                             format's largest power of two)
    e = clamp(e, -127, 127);  all-zero block: e = -127
    P_i = elem(V_i / 2^e)                   round to nearest, ties to even,
                                             saturated at the format's max
The element formats have no infinities or NaNs.  A value with E exponent
bits, M mantissa bits and bias B is
    exponent field 0:  (-1)^s * 2^(1 - B) * (m / 2^M)          (subnormal)
    exponent field f:  (-1)^s * 2^(f - B) * (1 + m / 2^M)
so E2M1 (B = 1) holds 0, 0.5, 1, 1.5, 2, 3, 4, 6; E2M3 (B = 1) tops out
at 7.5 and E3M2 (B = 3) at 28.  Codes are sign | exponent | mantissa, from
the high bit down.  FP4 codes are packed two to a byte, element 2i in the low
nibble of byte i (a reading: the specification leaves packing to the
implementation).  FP6 codes of a 32-element block are packed into 24 bytes,
element v at bits [6 v, 6 v + 6) of the block read as one little-endian
192-bit number, followed by 8 zero bytes, so a row of L elements takes L
bytes (a reading too: the padding keeps every block on a 32-byte boundary).

The CODA paper names only the trend towards FP8 and FP4 operands (§1); the
formats and the conversion are the MX specification's.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E8M0_BIAS = 127

# name: (exponent bits, mantissa bits, bias)
FORMATS = {"e2m1": (2, 1, 1), "e2m3": (2, 3, 1), "e3m2": (3, 2, 3)}


def fmt_params(fmt: str):
    E, M, B = FORMATS[fmt]
    emax = (2 ** E - 1) - B
    vmax = (2.0 - 2.0 ** -M) * 2.0 ** emax
    return E, M, B, emax, vmax


def decode(codes, fmt: str) -> np.ndarray:
    """Values of element codes, from the bit layout."""
    E, M, B, _, _ = fmt_params(fmt)
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> (E + M)) & 1
    f = (c >> M) & (2 ** E - 1)
    m = c & (2 ** M - 1)
    mag = np.where(f == 0, 2.0 ** (1 - B) * (m / 2.0 ** M), 2.0 ** (f - B) * (1.0 + m / 2.0 ** M))
    return np.where(s == 1, -mag, mag)


def round_elem(x, fmt: str) -> np.ndarray:
    """Nearest element value, ties to even, saturated at the format's max.

    Within the binade [2^k, 2^(k+1)) the values are the multiples of
    q = 2^(k - M); below the smallest normal 2^(1 - B) they are the multiples
    of 2^(1 - B - M).  An even multiple of q has an even mantissa, so
    rounding x / q half to even is ties-to-even.
    """
    _, M, B, _, vmax = fmt_params(fmt)
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    k = np.frexp(np.where(a > 0, a, 1.0))[1] - 1      # floor(log2 a), exactly
    k = np.maximum(k, 1 - B)                          # the subnormal range shares the lowest binade's step
    q = 2.0 ** (k - M)
    v = np.minimum(np.rint(a / q) * q, vmax)
    return np.where(x < 0, -v, v)


def encode(v, fmt: str) -> np.ndarray:
    """Codes of values that are exactly representable (the output of
    round_elem); -0 and +0 both give code 0."""
    E, M, B, _, _ = fmt_params(fmt)
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    k = np.frexp(np.where(a > 0, a, 1.0))[1] - 1
    normal = a >= 2.0 ** (1 - B)
    f = np.where(normal, k + B, 0)
    m = np.where(normal, a / 2.0 ** (k - M) - 2 ** M, a / 2.0 ** (1 - B - M))
    s = (v < 0) & (a > 0)
    return ((s.astype(np.int64) << (E + M)) | (f.astype(np.int64) << M) | m.astype(np.int64)).astype(np.uint8)


def block_exponents(X, fmt: str, block: int = BLOCK) -> np.ndarray:
    """Shared exponents e [R, C / block] of the row-major blocks of X [R, C]."""
    _, _, _, emax, _ = fmt_params(fmt)
    X = np.asarray(X, dtype=np.float32)
    R, C = X.shape
    assert C % block == 0, "the contracted axis must be a multiple of the block"
    amax = np.max(np.abs(X.reshape(R, C // block, block)), axis=2).astype(np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))     # amax = f 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, (ex - 1) - emax, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize(X, fmt: str, block: int = BLOCK):
    """MX quantisation of X [R, C] along C: (P, e), P [R, C] float64 element
    values, e [R, C / block] int64 shared exponents."""
    X = np.asarray(X, dtype=np.float32)
    e = block_exponents(X, fmt, block)
    scale = np.repeat(np.exp2(-e.astype(np.float64)), block, axis=1)   # exact powers of two
    return round_elem(X.astype(np.float64) * scale, fmt), e


def pack_fp4(codes) -> np.ndarray:
    """[R, C] FP4 codes -> [R, C / 2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack_fp4(b) -> np.ndarray:
    """Inverse of pack_fp4."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def pack_fp6(codes) -> np.ndarray:
    """[R, C] FP6 codes (C a multiple of 32) -> [R, C] bytes: each block of 32
    codes becomes 24 bytes holding code v at bits [6 v, 6 v + 6) of a
    little-endian 192-bit number, then 8 zero bytes."""
    c = np.asarray(codes, dtype=np.uint64) & 0x3F
    R, C = c.shape
    assert C % 32 == 0, "FP6 rows are whole 32-element blocks"
    blk = c.reshape(R, C // 32, 32)
    out = np.zeros((R, C // 32, 32), dtype=np.uint8)
    for v in range(32):                      # value v starts at bit 6 v
        byte, shift = divmod(6 * v, 8)
        bits = blk[:, :, v] << np.uint64(shift)          # at most 13 bits
        out[:, :, byte] |= (bits & 0xFF).astype(np.uint8)
        if shift > 2:
            out[:, :, byte + 1] |= ((bits >> np.uint64(8)) & 0xFF).astype(np.uint8)
    return out.reshape(R, C)


def unpack_fp6(b) -> np.ndarray:
    """Inverse of pack_fp6 (the pad bytes are ignored)."""
    b = np.asarray(b, dtype=np.uint8)
    R, C = b.shape
    blk = b.reshape(R, C // 32, 32).astype(np.uint64)
    out = np.empty((R, C // 32, 32), dtype=np.uint8)
    for v in range(32):
        byte, shift = divmod(6 * v, 8)
        w = blk[:, :, byte] | ((blk[:, :, byte + 1] << np.uint64(8)) if byte + 1 < 24 else np.uint64(0))
        out[:, :, v] = ((w >> np.uint64(shift)) & np.uint64(0x3F)).astype(np.uint8)
    return out.reshape(R, C)


def dequantize(P, e, block: int = BLOCK) -> np.ndarray:
    """The operand the quantised form stands for, in float64 (exact)."""
    return np.asarray(P, dtype=np.float64) * np.repeat(np.exp2(np.asarray(e, dtype=np.float64)), block, axis=1)


def matmul_nt(PA, eA, PB, eB, block: int = BLOCK) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] B[n, k] of two MX operands stored with the
    contracted axis contiguous (A [M, K], B [N, K]); float64."""
    return dequantize(PA, eA, block) @ dequantize(PB, eB, block).T
