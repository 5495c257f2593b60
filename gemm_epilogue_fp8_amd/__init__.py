"""MI355X (gfx950) GEMM + epilogue library: Python binding of libcoda.so.

Every function here only marshals arguments (torch tensors -> matrix
descriptors, the current HIP stream, a cached workspace buffer) and calls
the C ABI declared in include/coda.h; all computation runs in the library's
HIP kernels.  There is no CPU fallback: a missing library raises.

Layouts: weights are [K_in, N_out] row-major; the gate/up weight is packed
with pack_gate_up (64-column blocks of 32 gate then 32 up columns).
"""
from __future__ import annotations

import ctypes as C
from typing import Iterable, Optional, Sequence

import torch

from . import _lib
from ._lib import (CODA_BF16, CODA_E2M1X2, CODA_E2M3, CODA_E3M2, CODA_E4M3, CODA_E8M0, CODA_F32, CODA_I32, PREC_BF16, PREC_FP8, PREC_MXFP8,
                   PREC_MXFP4, PREC_MXFP6_E2M3, PREC_MXFP6_E3M2,
                   EPI_STORE_BF16, EPI_ACCUM_F32, EPI_ROW_SCALE, EPI_COL_SCALE, EPI_ADD_TILE,
                   EPI_ROW_SUMSQ_PARTIAL, EPI_SWIGLU, EPI_ROW_RMS_FROM_PARTIALS, EPI_STORE_ROW_VEC,
                   EPI_SAVE_PRE, EPI_QKNORM_ROPE, EPI_DSWIGLU, EPI_ROW_DOT_PARTIAL, EPI_NORM_CORRECTION,
                   EPI_WGRAD_GAIN, EPI_CE_LSE_PARTIAL, EPI_CE_GRAD, EPI_SIGMOID, EPI_DSIGMOID, EPI_SCALE_DEV,
                   EPI_DEQUANT_E4M3, EPI_GELU, EPI_DGELU, SCHED_PINGPONG, SCHED_CORESIDENT)

__all__ = ["CodaError", "Weight", "lib", "mat", "fold_gain", "pack_gate_up", "rope_table", "row_sumsq",
           "quantize_e4m3", "quantize_weight", "gemm_epi", "partials_cols", "quantize_mxfp8", "gemm_mx",
           "linear_swiglu_fwd", "linear_swiglu_bwd", "linear_rmsnorm_residual_fwd",
           "linear_rmsnorm_residual_bwd", "linear_qknorm_rope_fwd", "linear_qknorm_rope_bwd",
           "linear_cross_entropy_fwd", "linear_cross_entropy_bwd", "linear_sigmoid_fwd", "linear_sigmoid_bwd",
           "linear_gelu_fwd", "linear_gelu_bwd", "set_schedule", "get_schedule", "schedule",
           "SCHED_PINGPONG", "SCHED_CORESIDENT", "PREC_BF16", "PREC_FP8", "PREC_MXFP8", "PREC_MXFP4",
           "PREC_MXFP6_E2M3", "PREC_MXFP6_E3M2"]


class CodaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_lib.STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    return _lib.load()


_DT = {torch.bfloat16: CODA_BF16, torch.float32: CODA_F32, torch.float8_e4m3fn: CODA_E4M3,
       torch.int32: CODA_I32, torch.uint8: CODA_E8M0, torch.float8_e8m0fnu: CODA_E8M0}


def mat(t: Optional[torch.Tensor]) -> _lib.CodaMat:
    """Descriptor of a 1-D (as 1 x n) or 2-D row-major tensor; None -> absent."""
    m = _lib.CodaMat()
    if t is None:
        return m
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() == 1:
        rows, cols, ld = 1, t.shape[0], t.shape[0]
        if t.numel() > 1 and t.stride(0) != 1:
            raise ValueError("vector must be contiguous")
    elif t.dim() == 2:
        rows, cols = t.shape
        if cols > 1 and t.stride(1) != 1:
            raise ValueError("matrix rows must be contiguous")
        ld = t.stride(0) if rows > 1 else cols
    else:
        raise ValueError("only 1-D and 2-D tensors")
    # an empty view keeps the address of the storage it views (torch reports
    # 0 for it), so an empty required argument is not taken as absent
    ptr = t.data_ptr() or (t.untyped_storage().data_ptr() if t.numel() == 0 else 0)
    m.ptr = ptr or None
    m.dtype, m.rows, m.cols, m.ld = _DT[t.dtype], rows, cols, ld
    return m


def _p(t):
    return C.byref(mat(t)) if t is not None else None


class Weight:
    """A weight W [K_in, N_out] (bf16) and its optional E4M3 copies."""

    def __init__(self, w: torch.Tensor, q_fwd=None, s_fwd=None, q_bwd=None, s_bwd=None):
        self.w, self.q_fwd, self.s_fwd, self.q_bwd, self.s_bwd = w, q_fwd, s_fwd, q_bwd, s_bwd

    # dtype of the uint8 copies: CODA_E2M1X2 (prepare_mxfp4), CODA_E2M3 or
    # CODA_E3M2 (prepare_mxfp6); None for the E4M3 copies
    elem_dtype = None

    @property
    def fp4(self) -> bool:
        return self.elem_dtype == CODA_E2M1X2

    def c(self) -> _lib.CodaWeight:
        cw = _lib.CodaWeight()
        cw.w = mat(self.w)
        cw.q_fwd, cw.s_fwd = mat(self.q_fwd), mat(self.s_fwd)
        if self.elem_dtype is not None:
            cw.q_fwd.dtype = self.elem_dtype
        cw.q_bwd, cw.s_bwd = mat(self.q_bwd), mat(self.s_bwd)
        if self.elem_dtype is not None and self.q_bwd is not None:
            cw.q_bwd.dtype = self.elem_dtype
        return cw

    def prepare_fp8(self):
        """Allocate and fill the per-output-channel (transposed) and
        per-input-channel E4M3 copies (coda_quantize_weight)."""
        K, N = self.w.shape
        dev = self.w.device
        self.q_fwd = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=dev)
        self.s_fwd = torch.empty(N, dtype=torch.float32, device=dev)
        self.q_bwd = torch.empty((K, N), dtype=torch.float8_e4m3fn, device=dev)
        self.s_bwd = torch.empty(K, dtype=torch.float32, device=dev)
        quantize_weight(self)
        return self

    def prepare_mxfp8(self):
        """Allocate and fill the two block-scaled E4M3 copies
        (coda_quantize_weight): q_fwd [N, K] with exponents along K_in and
        q_bwd [K, N] with exponents along N_out, both in word layout."""
        K, N = self.w.shape
        dev = self.w.device
        self.q_fwd = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=dev)
        self.s_fwd = torch.empty(((K + 127) // 128, 4 * N), dtype=torch.uint8, device=dev)
        self.q_bwd = torch.empty((K, N), dtype=torch.float8_e4m3fn, device=dev)
        self.s_bwd = torch.empty(((N + 127) // 128, 4 * K), dtype=torch.uint8, device=dev)
        quantize_weight(self)
        return self

    def prepare_mxfp4(self, backward: bool = True):
        """Allocate and fill the block-scaled E2M1 copies (coda_quantize_weight):
        q_fwd [N, K/2] bytes (two codes a byte) with exponents along K_in and,
        unless backward is False (an inference-only weight), q_bwd [K, N/2]
        bytes with exponents along N_out, both in word layout."""
        K, N = self.w.shape
        dev = self.w.device
        self.elem_dtype = CODA_E2M1X2
        self.q_fwd = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        self.s_fwd = torch.empty(((K + 127) // 128, 4 * N), dtype=torch.uint8, device=dev)
        if backward and N % 128 == 0:
            self.q_bwd = torch.empty((K, N // 2), dtype=torch.uint8, device=dev)
            self.s_bwd = torch.empty(((N + 127) // 128, 4 * K), dtype=torch.uint8, device=dev)
        else:
            self.q_bwd = self.s_bwd = None
        quantize_weight(self)
        return self

    def prepare_mxfp6(self, fmt: str = "e2m3", backward: bool = True):
        """Allocate and fill the block-scaled FP6 copies in format fmt
        ("e2m3" or "e3m2", coda_quantize_weight): q_fwd [N, K] bytes (32-value
        blocks of 24 packed bytes and 8 of padding) with exponents along K_in
        and, unless backward is False, q_bwd [K, N] with exponents along
        N_out, both in word layout."""
        K, N = self.w.shape
        dev = self.w.device
        self.elem_dtype = _FP6[fmt]
        self.q_fwd = torch.empty((N, K), dtype=torch.uint8, device=dev)
        self.s_fwd = torch.empty(((K + 127) // 128, 4 * N), dtype=torch.uint8, device=dev)
        if backward and N % 128 == 0:
            self.q_bwd = torch.empty((K, N), dtype=torch.uint8, device=dev)
            self.s_bwd = torch.empty(((N + 127) // 128, 4 * K), dtype=torch.uint8, device=dev)
        else:
            self.q_bwd = self.s_bwd = None
        quantize_weight(self)
        return self


def _wref(w):
    if w is None:
        return None
    if isinstance(w, torch.Tensor):
        w = Weight(w)
    return C.byref(w.c())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


_WS = {}
_WS_RETIRED = []


def _workspace(nbytes: int, device) -> torch.Tensor:
    """A per-device workspace buffer, grown on demand and reused by calls
    that run in order on one stream.  A buffer that is outgrown stays
    allocated: a HIP graph captured while it was current keeps using its
    address on every replay."""
    key = str(device)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        size = max(nbytes, 1 << 20)
        if buf is not None:
            _WS_RETIRED.append(buf)
            size = max(size, 2 * buf.numel())   # doubling: the retired buffers add up to less than the live one
        buf = torch.empty(size, dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


def _check(st: int):
    if st != 0:
        raise CodaError(st, lib().coda_last_error().decode())


def set_schedule(sched: int):
    """Process-wide launch schedule of the bf16 SwiGLU GEMM (coda_set_schedule)."""
    _check(lib().coda_set_schedule(sched))


def get_schedule() -> int:
    return lib().coda_get_schedule()


class schedule:
    """Context manager: `with schedule(SCHED_CORESIDENT): ...` restores the
    previous schedule on exit."""

    def __init__(self, sched: int):
        self.sched, self.prev = sched, None

    def __enter__(self):
        self.prev = get_schedule()
        set_schedule(self.sched)
        return self

    def __exit__(self, *exc):
        set_schedule(self.prev)
        return False


def _ws_call(size_fn, size_args, device):
    n = C.c_size_t(0)
    _check(size_fn(*size_args, C.byref(n)))
    if n.value == 0:
        return None, 0
    buf = _workspace(n.value, device)
    return C.c_void_p(buf.data_ptr()), n.value


# ---------------------------------------------------------------- prep
def fold_gain(W, g, W_out):
    _check(lib().coda_fold_gain(_p(W), _p(g), _p(W_out), _stream()))
    return W_out


def pack_gate_up(Wg, Wu, g, out):
    _check(lib().coda_pack_gate_up(_p(Wg), _p(Wu), _p(g), _p(out), _stream()))
    return out


def rope_table(seq_len: int, out, head_dim: int = 128, theta: float = 5e5):
    _check(lib().coda_rope_table(seq_len, head_dim, theta, _p(out), _stream()))
    return out


def row_sumsq(x, out):
    _check(lib().coda_row_sumsq(_p(x), _p(out), _stream()))
    return out


def quantize_e4m3(X, axis: int, Q, scale):
    ws, n = _ws_call(lib().coda_quantize_e4m3_workspace, (_p(X), axis), X.device)
    _check(lib().coda_quantize_e4m3(_p(X), axis, _p(Q), _p(scale), ws, n, _stream()))
    return Q, scale


def quantize_weight(wt: Weight):
    cw = wt.c()
    ws, n = _ws_call(lib().coda_quantize_weight_workspace, (C.byref(cw),), wt.w.device)
    _check(lib().coda_quantize_weight(C.byref(cw), ws, n, _stream()))
    return wt


def partials_cols(N: int) -> int:
    return int(lib().coda_partials_cols(N))


# ---------------------------------------------------------------- generic
def gemm_epi(program: Sequence[tuple], A, transA: int, B, transB: int, D, aux: Iterable = ()):
    """program: sequence of (opcode, slot, fparam) or (opcode, (slot, slot2,
    slot3), fparam) tuples (see coda.h); D may be None for chains that store
    nothing.  E4M3 operands (torch.float8_e4m3fn) when the program starts
    with EPI_DEQUANT_E4M3."""
    prog = _program(program)
    aux = list(aux)
    arr = (_lib.CodaMat * max(len(aux), 1))(*[mat(a) for a in aux])
    M = A.shape[1] if transA else A.shape[0]
    N = B.shape[0] if transB else B.shape[1]
    K = A.shape[0] if transA else A.shape[1]
    ws, n = _ws_call(lib().coda_gemm_epi_workspace, (C.byref(prog), M, N, K), A.device)
    _check(lib().coda_gemm_epi(C.byref(prog), _p(A), transA, _p(B), transB, _p(D),
                               arr if aux else None, len(aux), ws, n, _stream()))
    return D


def _program(program):
    prog = _lib.EpiProgram()
    prog.n_ops = len(program)
    for i, (op, slots, fparam) in enumerate(program):
        slots = tuple(slots) if isinstance(slots, (tuple, list)) else (slots,)
        slots = slots + (0,) * (3 - len(slots))
        o = prog.ops[i]
        o.op, o.slot, o.slot2, o.slot3, o.fparam = op, slots[0], slots[1], slots[2], fparam
    return prog


# ---------------------------------------------------------------- MXFP8
def quantize_mxfp8(X, axis: int, Q=None, S=None):
    """MXFP8 copy of X [R, C] (bf16): axis 1 -> Q [R, C] with the exponents
    of R rows; axis 0 -> Q [C, R] (transposed) with those of C rows.  S holds
    E8M0 codes (uint8) in word layout, [ceil(L/128), 4 rows] (see coda.h)."""
    R, Cc = X.shape
    rows, L = (R, Cc) if axis == 1 else (Cc, R)
    if Q is None:
        Q = torch.empty((rows, L), dtype=torch.float8_e4m3fn, device=X.device)
    if S is None:
        S = torch.empty(((L + 127) // 128, 4 * rows), dtype=torch.uint8, device=X.device)
    _check(lib().coda_quantize_mxfp8(_p(X), axis, _p(Q), _p(S), _stream()))
    return Q, S


def quantize_mxfp4(X, axis: int, Q=None, S=None):
    """MXFP4 copy of X [R, C] (bf16): axis 1 -> Q [R, C / 2] bytes with the
    exponents of R rows; axis 0 -> Q [C, R / 2] (transposed) with those of
    C rows.  Q holds two E2M1 codes a byte (element 2i in the low nibble), S
    E8M0 codes in word layout, [ceil(L/128), 4 rows] (see coda.h)."""
    R, Cc = X.shape
    rows, L = (R, Cc) if axis == 1 else (Cc, R)
    if Q is None:
        Q = torch.empty((rows, L // 2), dtype=torch.uint8, device=X.device)
    if S is None:
        S = torch.empty(((L + 127) // 128, 4 * rows), dtype=torch.uint8, device=X.device)
    q = mat(Q)
    q.dtype = CODA_E2M1X2
    _check(lib().coda_quantize_mxfp4(_p(X), axis, C.byref(q), _p(S), _stream()))
    return Q, S


_FP6 = {"e2m3": CODA_E2M3, "e3m2": CODA_E3M2}


def quantize_mxfp6(X, axis: int, fmt: str, Q=None, S=None):
    """MXFP6 copy of X [R, C] (bf16) in format fmt ("e2m3" or "e3m2"): axis
    1 -> Q [R, C] bytes with the exponents of R rows; axis 0 -> Q [C, R]
    (transposed) with those of C rows.  Each 32-value block of Q is 24 bytes
    of packed six-bit codes and 8 zero bytes; S holds E8M0 codes in word
    layout, [ceil(L/128), 4 rows] (see coda.h)."""
    R, Cc = X.shape
    rows, L = (R, Cc) if axis == 1 else (Cc, R)
    if Q is None:
        Q = torch.empty((rows, L), dtype=torch.uint8, device=X.device)
    if S is None:
        S = torch.empty(((L + 127) // 128, 4 * rows), dtype=torch.uint8, device=X.device)
    q = mat(Q)
    q.dtype = _FP6[fmt]
    _check(lib().coda_quantize_mxfp6(_p(X), axis, C.byref(q), _p(S), _stream()))
    return Q, S


def gemm_mx(program: Sequence[tuple], A, SA, B, SB, D, aux: Iterable = ()):
    """D = epilogue(A~ B~^T) with MXFP8 operands A [M, K], B [N, K] and their
    E8M0 block exponents SA [K/128, 4M], SB [K/128, 4N] in word layout;
    program as in gemm_epi."""
    prog = _program(program)
    aux = list(aux)
    arr = (_lib.CodaMat * max(len(aux), 1))(*[mat(a) for a in aux])
    ws, n = _ws_call(lib().coda_gemm_epi_workspace, (C.byref(prog), A.shape[0], B.shape[0], A.shape[1]), A.device)
    _check(lib().coda_gemm_mx(C.byref(prog), _p(A), _p(SA), _p(B), _p(SB), _p(D),
                              arr if aux else None, len(aux), ws, n, _stream()))
    return D


def gemm_mx4(program: Sequence[tuple], A, SA, B, SB, D, aux: Iterable = ()):
    """D = epilogue(A~ B~^T) with MXFP4 operands A [M, K/2], B [N, K/2]
    (uint8, two E2M1 codes a byte, from quantize_mxfp4) and their E8M0
    exponents SA [K/128, 4M], SB [K/128, 4N] in word layout."""
    prog = _program(program)
    aux = list(aux)
    arr = (_lib.CodaMat * max(len(aux), 1))(*[mat(a) for a in aux])
    a, b = mat(A), mat(B)
    a.dtype = b.dtype = CODA_E2M1X2
    ws, n = _ws_call(lib().coda_gemm_epi_workspace, (C.byref(prog), A.shape[0], B.shape[0], 2 * A.shape[1]),
                     A.device)
    _check(lib().coda_gemm_mx(C.byref(prog), C.byref(a), _p(SA), C.byref(b), _p(SB), _p(D),
                              arr if aux else None, len(aux), ws, n, _stream()))
    return D


def gemm_mx6(program: Sequence[tuple], fmt: str, A, SA, B, SB, D, aux: Iterable = ()):
    """D = epilogue(A~ B~^T) with MXFP6 operands of format fmt ("e2m3" or
    "e3m2"), A [M, K], B [N, K] (uint8, from quantize_mxfp6) and their E8M0
    exponents SA [K/128, 4M], SB [K/128, 4N] in word layout."""
    prog = _program(program)
    aux = list(aux)
    arr = (_lib.CodaMat * max(len(aux), 1))(*[mat(a) for a in aux])
    a, b = mat(A), mat(B)
    a.dtype = b.dtype = _FP6[fmt]
    ws, n = _ws_call(lib().coda_gemm_epi_workspace, (C.byref(prog), A.shape[0], B.shape[0], A.shape[1]), A.device)
    _check(lib().coda_gemm_mx(C.byref(prog), C.byref(a), _p(SA), C.byref(b), _p(SB), _p(D),
                              arr if aux else None, len(aux), ws, n, _stream()))
    return D


# ---------------------------------------------------------------- forward
def linear_swiglu_fwd(x, Wgu, eps, out, sumsq_partials=None, save_hgu=None, r_out=None,
                      precision: int = PREC_BF16):
    L = lib()
    wc = Wgu if isinstance(Wgu, Weight) else Weight(Wgu)
    M, K = x.shape
    ws, n = _ws_call(L.coda_linear_swiglu_fwd_workspace, (M, K, int(sumsq_partials is not None), precision),
                     x.device)
    _check(L.coda_linear_swiglu_fwd(_p(x), _p(sumsq_partials), C.byref(wc.c()), eps, _p(out), _p(save_hgu),
                                    _p(r_out), precision, ws, n, _stream()))
    return out


def linear_rmsnorm_residual_fwd(a, W, residual, out, sumsq_partials_out=None, precision: int = PREC_BF16):
    L = lib()
    M, K = a.shape
    wc = W if isinstance(W, Weight) else Weight(W)
    ws, n = _ws_call(L.coda_linear_rmsnorm_residual_fwd_workspace, (M, K, wc.w.shape[1], precision), a.device)
    _check(L.coda_linear_rmsnorm_residual_fwd(_p(a), C.byref(wc.c()), _p(residual), _p(out),
                                              _p(sumsq_partials_out), precision, ws, n, _stream()))
    return out


def linear_qknorm_rope_fwd(x, Wqkv, gq, gk, rope, seq_len, eps, q, k, v, sumsq_partials=None,
                           save_qk_pre=None, r_out=None, precision: int = PREC_BF16):
    L = lib()
    M, D = x.shape
    wc = Wqkv if isinstance(Wqkv, Weight) else Weight(Wqkv)
    ws, n = _ws_call(L.coda_linear_qknorm_rope_fwd_workspace,
                     (M, D, int(sumsq_partials is not None), precision), x.device)
    _check(L.coda_linear_qknorm_rope_fwd(_p(x), _p(sumsq_partials), C.byref(wc.c()), _p(gq), _p(gk), _p(rope),
                                         seq_len, eps, _p(q), _p(k), _p(v), _p(save_qk_pre), _p(r_out),
                                         precision, ws, n, _stream()))
    return q, k, v


# ---------------------------------------------------------------- backward
def linear_swiglu_bwd(dY, Wd, saved_hgu, r, u, Wgu, Wgu_unfolded, g, dres, du, dWgu, dg, beta=0.0,
                      dh_gu_out=None, precision: int = PREC_BF16):
    L = lib()
    M, D = dY.shape
    wd = Wd if isinstance(Wd, Weight) else Weight(Wd)
    wgu = Wgu if isinstance(Wgu, Weight) else Weight(Wgu)
    F = wd.w.shape[0]
    ws, n = _ws_call(L.coda_linear_swiglu_bwd_workspace, (M, D, F, precision), dY.device)
    _check(L.coda_linear_swiglu_bwd(_p(dY), C.byref(wd.c()), _p(saved_hgu), _p(r), _p(u), C.byref(wgu.c()),
                                    _p(Wgu_unfolded), _p(g), _p(dres), _p(du), _p(dWgu), _p(dg), beta,
                                    _p(dh_gu_out), precision, ws, n, _stream()))
    return du, dWgu, dg


def linear_rmsnorm_residual_bwd(d_out, a, W, dW, da=None, beta=0.0, precision: int = PREC_BF16):
    L = lib()
    M, N = d_out.shape
    wc = W if isinstance(W, Weight) else Weight(W)
    ws, n = _ws_call(L.coda_linear_rmsnorm_residual_bwd_workspace, (M, a.shape[1], N, precision), d_out.device)
    _check(L.coda_linear_rmsnorm_residual_bwd(_p(d_out), _p(a), C.byref(wc.c()), _p(da), _p(dW), beta,
                                              precision, ws, n, _stream()))
    return da, dW


def linear_qknorm_rope_bwd(dq, dk, dv, x, r, qk_pre, v, Wqkv, Wqkv_unfolded, g, gq, gk, rope, seq_len, eps,
                           dres, dx, dW, dg, dgq, dgk, beta=0.0, dh_qkv_out=None, precision: int = PREC_BF16):
    L = lib()
    M, D = x.shape
    wc = Wqkv if isinstance(Wqkv, Weight) else Weight(Wqkv)
    ws, n = _ws_call(L.coda_linear_qknorm_rope_bwd_workspace, (M, D, precision), x.device)
    _check(L.coda_linear_qknorm_rope_bwd(_p(dq), _p(dk), _p(dv), _p(x), _p(r), _p(qk_pre), _p(v), C.byref(wc.c()),
                                         _p(Wqkv_unfolded), _p(g), _p(gq), _p(gk), _p(rope), seq_len, eps, _p(dres),
                                         _p(dx), _p(dW), _p(dg), _p(dgq), _p(dgk), beta, _p(dh_qkv_out), precision,
                                         ws, n, _stream()))
    return dx, dW, dg, dgq, dgk


# ---------------------------------------------------------------- cross-entropy
def linear_cross_entropy_fwd(h, W, labels, loss, lse, n_valid, per_row=None, n_bad=None, ignore_index=-100,
                             precision: int = PREC_BF16):
    L = lib()
    wc = W if isinstance(W, Weight) else Weight(W)
    ws, n = _ws_call(L.coda_linear_cross_entropy_fwd_workspace, (h.shape[0], h.shape[1], wc.w.shape[1], precision),
                     h.device)
    _check(L.coda_linear_cross_entropy_fwd(_p(h), C.byref(wc.c()), _p(labels), ignore_index, _p(loss), _p(lse),
                                           _p(per_row), _p(n_valid), _p(n_bad), precision, ws, n, _stream()))
    return loss


def linear_cross_entropy_fwd_noalloc(h, W, labels, loss, lse, n_valid, per_row=None, n_bad=None,
                                     ignore_index=-100):
    """bf16 linear + cross-entropy forward through the entry point that takes
    no workspace (its partials live in the library's per-GPU scratch array)."""
    wc = W if isinstance(W, Weight) else Weight(W)
    _check(lib().coda_linear_cross_entropy_fwd_noalloc(_p(h), C.byref(wc.c()), _p(labels), ignore_index, _p(loss),
                                                       _p(lse), _p(per_row), _p(n_valid), _p(n_bad), _stream()))
    return loss


def linear_cross_entropy_bwd(h, W, labels, lse, n_valid, dloss, dh, dW, beta=0.0, chunk_rows=0, ignore_index=-100,
                             precision: int = PREC_BF16):
    L = lib()
    wc = W if isinstance(W, Weight) else Weight(W)
    M, D = h.shape
    ws, n = _ws_call(L.coda_linear_cross_entropy_bwd_workspace, (M, D, wc.w.shape[1], chunk_rows, precision),
                     h.device)
    _check(L.coda_linear_cross_entropy_bwd(_p(h), C.byref(wc.c()), _p(labels), ignore_index, _p(lse), _p(n_valid),
                                           dloss, _p(dh), _p(dW), beta, chunk_rows, precision, ws, n, _stream()))
    return dh, dW


def linear_rmsnorm_cross_entropy_fwd(y, W, eps, labels, loss, lse, n_valid, sumsq_partials=None, per_row=None,
                                     n_bad=None, r_out=None, ignore_index=-100, precision: int = PREC_BF16):
    """Final RMSNorm (gain folded into W) -> LM head -> mean cross-entropy."""
    L = lib()
    wc = W if isinstance(W, Weight) else Weight(W)
    M, D = y.shape
    ws, n = _ws_call(L.coda_linear_rmsnorm_cross_entropy_fwd_workspace,
                     (M, D, wc.w.shape[1], int(sumsq_partials is not None), precision), y.device)
    _check(L.coda_linear_rmsnorm_cross_entropy_fwd(_p(y), _p(sumsq_partials), C.byref(wc.c()), eps, _p(labels),
                                                   ignore_index, _p(loss), _p(lse), _p(per_row), _p(n_valid),
                                                   _p(n_bad), _p(r_out), precision, ws, n, _stream()))
    return loss


def linear_rmsnorm_cross_entropy_bwd(y, r, W, W_unfolded, g, labels, lse, n_valid, dloss, dy, dW, dg, dres=None,
                                     beta=0.0, chunk_rows=0, ignore_index=-100, precision: int = PREC_BF16):
    L = lib()
    wc = W if isinstance(W, Weight) else Weight(W)
    M, D = y.shape
    ws, n = _ws_call(L.coda_linear_rmsnorm_cross_entropy_bwd_workspace, (M, D, wc.w.shape[1], chunk_rows, precision),
                     y.device)
    _check(L.coda_linear_rmsnorm_cross_entropy_bwd(_p(y), _p(r), C.byref(wc.c()), _p(W_unfolded), _p(g), _p(labels),
                                                   ignore_index, _p(lse), _p(n_valid), dloss, _p(dres), _p(dy),
                                                   _p(dW), _p(dg), beta, chunk_rows, precision, ws, n, _stream()))
    return dy, dW, dg


# ---------------------------------------------------------------- RMSNorm -> Linear -> sigmoid | GELU
def _map_fwd(act, x, W, eps, out, sumsq_partials, save_h, r_out, precision):
    L = lib()
    wc = W if isinstance(W, Weight) else Weight(W)
    M, K = x.shape
    ws, n = _ws_call(getattr(L, f"coda_linear_{act}_fwd_workspace"),
                     (M, K, int(sumsq_partials is not None), precision), x.device)
    _check(getattr(L, f"coda_linear_{act}_fwd")(_p(x), _p(sumsq_partials), C.byref(wc.c()), eps, _p(out),
                                               _p(save_h), _p(r_out), precision, ws, n, _stream()))
    return out


def _map_bwd(act, dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta, dh_out, precision):
    L = lib()
    wn = Wn if isinstance(Wn, Weight) else Weight(Wn)
    wc = W if isinstance(W, Weight) else Weight(W)
    M, D = dY.shape
    ws, n = _ws_call(getattr(L, f"coda_linear_{act}_bwd_workspace"), (M, D, wn.w.shape[0], precision), dY.device)
    _check(getattr(L, f"coda_linear_{act}_bwd")(_p(dY), C.byref(wn.c()), _p(saved_h), _p(r), _p(u),
                                               C.byref(wc.c()), _p(W_unfolded), _p(g), _p(dres), _p(du), _p(dW),
                                               _p(dg), beta, _p(dh_out), precision, ws, n, _stream()))
    return du, dW, dg


def linear_sigmoid_fwd(x, W, eps, out, sumsq_partials=None, save_h=None, r_out=None, precision: int = PREC_BF16):
    return _map_fwd("sigmoid", x, W, eps, out, sumsq_partials, save_h, r_out, precision)


def linear_sigmoid_bwd(dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta=0.0, dh_out=None,
                       precision: int = PREC_BF16):
    return _map_bwd("sigmoid", dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta, dh_out, precision)


def linear_gelu_fwd(x, W, eps, out, sumsq_partials=None, save_h=None, r_out=None, precision: int = PREC_BF16):
    return _map_fwd("gelu", x, W, eps, out, sumsq_partials, save_h, r_out, precision)


def linear_gelu_bwd(dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta=0.0, dh_out=None,
                    precision: int = PREC_BF16):
    return _map_bwd("gelu", dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta, dh_out, precision)


def probe_mfma_loop(dtype: int, blocks: int, iters: int, out=None):
    """MFMA-only loop (include/coda_probe.h): `blocks` workgroups of 8
    waves, `iters` rounds of 4 independent MFMA chains a wave.  Returns
    (flops, out) with out fp32 [blocks, 3] = (checksum, engine-clock
    cycles, 100 MHz ticks) per workgroup; the caller times the launch."""
    L = lib()
    if out is None:
        out = torch.zeros(blocks * 3, dtype=torch.float32, device="cuda")
    fl = C.c_double(0.0)
    _check(L.coda_probe_mfma_loop(dtype, blocks, iters, C.byref(mat(out.view(1, -1))), C.byref(fl), _stream()))
    return fl.value, out.view(blocks, 3)
