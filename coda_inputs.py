"""Seeded synthetic inputs for the GEMM+epilogue workloads.

This module only draws random numbers and rounds them to the storage type the
workload names (bf16 through torch's CPU cast, fp32 kept as is).  It holds none
of the method's arithmetic, so that the CPU oracle and the GPU path can both
consume exactly the same bits without sharing any computation.

Every tensor of a workload is drawn from its own child stream of
``numpy.random.SeedSequence(seed)`` (PCG64), in a fixed order, so one tensor can
be regenerated without drawing the others.  ``N(0, v)`` means variance ``v``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """A LLaMA-style non-attention block: tokens M, hidden D, MLP width F."""
    M: int
    D: int
    F: int
    head_dim: int = 128
    seq_len: int = 2048
    theta: float = 5.0e5
    eps: float = 1.0e-6

    @property
    def heads(self) -> int:
        return self.D // self.head_dim


@dataclasses.dataclass(frozen=True)
class CEShape:
    """Linear + cross-entropy: tokens M, hidden D, vocabulary V."""
    M: int
    D: int
    V: int
    ignore_frac: float = 0.05


@dataclasses.dataclass(frozen=True)
class SwiGLUShape:
    """RMSNorm -> Linear -> SwiGLU: tokens M, in K, out F (per half)."""
    M: int
    K: int
    F: int
    eps: float = 1.0e-6


# The five workloads.  Sizes follow the problem statement of each.
CFG1 = SwiGLUShape(M=256, K=512, F=1024)
CFG2 = BlockShape(M=8192, D=2048, F=8192)
CFG3 = BlockShape(M=8192, D=4096, F=11008)
CFG4 = CEShape(M=8192, D=2048, V=128256)
CFG5 = BlockShape(M=4096, D=8192, F=28672)
SEEDS = {"cfg1": 0, "cfg2": 0, "cfg3": 1, "cfg4": 0, "cfg5": 2}

# Draw order of the block tensors (each gets its own child stream).
BLOCK_ORDER = ("x", "o", "g1", "g2", "gq", "gk", "Wqkv", "Wo", "Wg", "Wu", "Wd",
               "dY", "dq", "dk", "dv")
SWIGLU_ORDER = ("x", "g", "Wg", "Wu")
CE_ORDER = ("h", "W", "labels", "ignore_rows")


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 with torch's CPU cast; return float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _streams(seed: int, names) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(names))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(names, children)}


def _normal(rng, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _gain(rng, n: int) -> np.ndarray:
    return (np.float32(1.0) + np.float32(0.1) * rng.standard_normal(n, dtype=np.float32)).astype(np.float32)


def block_inputs(shape: BlockShape, seed: int, names=None) -> Dict[str, np.ndarray]:
    """Block tensors: bf16 values as float32 arrays, gains as fp32.

    x, o ~ N(0,1); gains 1 + 0.1 N(0,1); weights ~ N(0, 1/K_in) stored
    [K_in, N_out]; dY, dq, dk, dv ~ N(0, 1e-2).  ``names`` limits the draw.
    """
    M, D, F = shape.M, shape.D, shape.F
    st = _streams(seed, BLOCK_ORDER)
    spec = {
        "x": ((M, D), 1.0, True), "o": ((M, D), 1.0, True),
        "Wqkv": ((D, 3 * D), D ** -0.5, True), "Wo": ((D, D), D ** -0.5, True),
        "Wg": ((D, F), D ** -0.5, True), "Wu": ((D, F), D ** -0.5, True),
        "Wd": ((F, D), F ** -0.5, True),
        "dY": ((M, D), 0.1, True), "dq": ((M, D), 0.1, True),
        "dk": ((M, D), 0.1, True), "dv": ((M, D), 0.1, True),
    }
    out = {}
    for n in BLOCK_ORDER:
        if names is not None and n not in names:
            continue
        if n in ("g1", "g2"):
            out[n] = _gain(st[n], D)
        elif n in ("gq", "gk"):
            out[n] = _gain(st[n], shape.head_dim)
        else:
            shp, std, is_bf16 = spec[n]
            a = _normal(st[n], shp, std)
            out[n] = to_bf16_values(a) if is_bf16 else a
    return out


def swiglu_inputs(shape: SwiGLUShape, seed: int) -> Dict[str, np.ndarray]:
    """x ~ N(0,1) bf16, g = 1 + 0.1 N(0,1) fp32, W_gate, W_up ~ N(0, 1/K) bf16."""
    st = _streams(seed, SWIGLU_ORDER)
    return {
        "x": to_bf16_values(_normal(st["x"], (shape.M, shape.K), 1.0)),
        "g": _gain(st["g"], shape.K),
        "Wg": to_bf16_values(_normal(st["Wg"], (shape.K, shape.F), shape.K ** -0.5)),
        "Wu": to_bf16_values(_normal(st["Wu"], (shape.K, shape.F), shape.K ** -0.5)),
    }


def ce_inputs(shape: CEShape, seed: int, n_ignore: Optional[int] = None) -> Dict[str, np.ndarray]:
    """h ~ N(0,1) bf16, W ~ N(0, 1/D) bf16 [D, V], labels uniform in [0, V)
    with round(ignore_frac * M) distinct rows set to the ignore index."""
    st = _streams(seed, CE_ORDER)
    M, D, V = shape.M, shape.D, shape.V
    labels = st["labels"].integers(0, V, size=M, dtype=np.int64).astype(np.int32)
    if n_ignore is None:
        n_ignore = int(round(shape.ignore_frac * M))
    rows = st["ignore_rows"].choice(M, size=n_ignore, replace=False)
    labels[rows] = IGNORE_INDEX
    return {
        "h": to_bf16_values(_normal(st["h"], (M, D), 1.0)),
        "W": to_bf16_values(_normal(st["W"], (D, V), D ** -0.5)),
        "labels": labels,
    }


def fp32_prior(shape, seed: int, std: float = 1e-3) -> np.ndarray:
    """A seeded fp32 tensor used as the prior value of an accumulated gradient."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7777])))
    return _normal(rng, shape, std)


def rolled_rows(seed: int, K: int, shifts) -> "RolledRows":
    """Rows of a very long matrix without storing it on the host: one seeded
    bf16 row of K values ~N(0,1), and row i is that row rotated left by
    ``shifts[i]`` places (numpy.roll by -shift)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4242])))
    return RolledRows(to_bf16_values(_normal(rng, (K,), 1.0)), tuple(int(s) for s in shifts))


@dataclasses.dataclass(frozen=True)
class RolledRows:
    base: np.ndarray
    shifts: tuple

    def row(self, i: int) -> np.ndarray:
        return np.roll(self.base, -self.shifts[i])
