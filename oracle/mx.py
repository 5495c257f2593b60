"""Block-scaled E4M3 operands (MXFP8) for the oracle.

Test infrastructure only: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Written from the OCP Microscaling Formats (MX) Specification v1.0 (section
on the MXFP8 format and on converting a block to MX): a block of 32
consecutive elements along the contracted axis shares one E8M0 scale, a pure
power of two 2^e with e in [-127, 127] (code e + 127; code 255 is NaN and is
never produced here).  For a block V:
    e = floor(log2(max |V_i|)) - 8          (8 = exponent of E4M3's largest
                                             power of two, 448 = 1.75 * 2^8)
    e = clamp(e, -127, 127);  all-zero block: e = -127
    P_i = E4M3(V_i / 2^e)                   (round to nearest even)
and the block's values are read back as 2^e * P_i.  max|V| / 2^e lies in
[256, 512), so values above 448 can occur; they saturate to +-448 (the same
reading as for the per-row amax quantiser: clamp before the cast).

The CODA paper names only the trend towards FP8 and FP4 operands (§1); the
block size, the scale format and the conversion are the MX specification's.
"""
from __future__ import annotations

import numpy as np

from .numerics import E4M3_MAX, e4m3, e4m3_codes

BLOCK = 32
EMAX_E4M3 = 8
E8M0_BIAS = 127


def block_exponents(X, block: int = BLOCK) -> np.ndarray:
    """Shared exponents e [R, C / block] of the row-major blocks of X [R, C]."""
    X = np.asarray(X, dtype=np.float32)
    R, C = X.shape
    assert C % block == 0, "the contracted axis must be a multiple of the block"
    amax = np.max(np.abs(X.reshape(R, C // block, block)), axis=2).astype(np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))     # amax = f 2^ex, f in [0.5, 1)
    e = (ex - 1) - EMAX_E4M3                             # floor(log2 amax) - 8
    e = np.where(amax > 0, e, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize(X, block: int = BLOCK):
    """MXFP8 quantisation of X [R, C] along C.

    Returns (P, e): P [R, C] float32 E4M3 values, e [R, C / block] int64
    shared exponents; the dequantised operand is P * 2^e (per block).
    """
    X = np.asarray(X, dtype=np.float32)
    R, C = X.shape
    e = block_exponents(X, block)
    scale = np.repeat(np.exp2(-e.astype(np.float64)), block, axis=1)   # exact powers of two
    P = e4m3(np.clip(X.astype(np.float64) * scale, -E4M3_MAX, E4M3_MAX))
    return P, e


def codes(P) -> np.ndarray:
    """E4M3 byte codes of quantised values."""
    return e4m3_codes(P)


def e8m0_codes(e) -> np.ndarray:
    """E8M0 byte codes (e + 127) of shared exponents."""
    return (np.asarray(e, dtype=np.int64) + E8M0_BIAS).astype(np.uint8)


def dequantize(P, e, block: int = BLOCK) -> np.ndarray:
    """The operand the quantised form stands for, in float64 (exact)."""
    return np.asarray(P, dtype=np.float64) * np.repeat(np.exp2(np.asarray(e, dtype=np.float64)), block, axis=1)


def matmul_nt(PA, eA, PB, eB, block: int = BLOCK) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] B[n, k] of two MXFP8 operands, both stored with
    the contracted axis K contiguous (A [M, K], B [N, K]); float64."""
    return dequantize(PA, eA, block) @ dequantize(PB, eB, block).T
