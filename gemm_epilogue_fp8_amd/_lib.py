"""ctypes declarations of the C ABI in include/coda.h.

Argument marshalling only: tensors become (pointer, dtype, rows, cols, ld)
descriptors and the current HIP stream handle; all work runs in libcoda.so.
Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcoda.so")

CODA_BF16, CODA_F32, CODA_E4M3, CODA_I32, CODA_E8M0, CODA_E2M1X2 = 1, 2, 3, 4, 5, 6
CODA_E2M3, CODA_E3M2 = 7, 8
PREC_BF16, PREC_FP8, PREC_MXFP8, PREC_MXFP4 = 0, 1, 2, 3
PREC_MXFP6_E2M3, PREC_MXFP6_E3M2 = 4, 5
STATUS = {0: "CODA_OK", 1: "CODA_ERR_NULL", 2: "CODA_ERR_DTYPE", 3: "CODA_ERR_SHAPE",
          4: "CODA_ERR_LAYOUT", 5: "CODA_ERR_ALIGN", 6: "CODA_ERR_WORKSPACE",
          7: "CODA_ERR_UNSUPPORTED", 8: "CODA_ERR_LAUNCH", 9: "CODA_ERR_VALUE"}

EPI_STORE_BF16, EPI_ACCUM_F32, EPI_ROW_SCALE, EPI_COL_SCALE = 1, 2, 3, 4
EPI_ADD_TILE, EPI_ROW_SUMSQ_PARTIAL, EPI_SWIGLU, EPI_ROW_RMS_FROM_PARTIALS = 5, 6, 7, 8
EPI_STORE_ROW_VEC, EPI_SAVE_PRE, EPI_QKNORM_ROPE, EPI_DSWIGLU = 9, 10, 11, 12
EPI_ROW_DOT_PARTIAL, EPI_NORM_CORRECTION, EPI_WGRAD_GAIN, EPI_CE_LSE_PARTIAL = 13, 14, 15, 16
EPI_CE_GRAD, EPI_SIGMOID, EPI_DSIGMOID, EPI_SCALE_DEV, EPI_DEQUANT_E4M3 = 17, 18, 19, 20, 21
EPI_GELU, EPI_DGELU = 22, 23
SCHED_PINGPONG, SCHED_CORESIDENT = 0, 1
MAX_EPI_OPS = 8


class CodaMat(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("dtype", C.c_int32), ("reserved", C.c_int32),
                ("rows", C.c_int64), ("cols", C.c_int64), ("ld", C.c_int64)]


class CodaWeight(C.Structure):
    _fields_ = [("w", CodaMat), ("q_fwd", CodaMat), ("s_fwd", CodaMat),
                ("q_bwd", CodaMat), ("s_bwd", CodaMat)]


class EpiOp(C.Structure):
    _fields_ = [("op", C.c_uint16), ("slot", C.c_uint16), ("slot2", C.c_uint16),
                ("slot3", C.c_uint16), ("fparam", C.c_float)]


class EpiProgram(C.Structure):
    _fields_ = [("n_ops", C.c_uint32), ("ops", EpiOp * MAX_EPI_OPS)]


M_ = C.POINTER(CodaMat)
W_ = C.POINTER(CodaWeight)
vp, i32, i64, f32, f64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_size_t
szp = C.POINTER(C.c_size_t)

# name -> argument types (all return int status unless listed in _RET)
SIGNATURES = {
    "coda_abi_version": [],
    "coda_status_string": [C.c_int],
    "coda_last_error": [],
    "coda_set_schedule": [i32],
    "coda_get_schedule": [],
    "coda_partials_cols": [i64],
    "coda_fold_gain": [M_, M_, M_, vp],
    "coda_pack_gate_up": [M_, M_, M_, M_, vp],
    "coda_rope_table": [i32, i32, f64, M_, vp],
    "coda_row_sumsq": [M_, M_, vp],
    "coda_quantize_e4m3_workspace": [M_, i32, szp],
    "coda_quantize_e4m3": [M_, i32, M_, M_, vp, sz, vp],
    "coda_quantize_weight_workspace": [W_, szp],
    "coda_quantize_weight": [W_, vp, sz, vp],
    "coda_gemm_epi_workspace": [C.POINTER(EpiProgram), i64, i64, i64, szp],
    "coda_gemm_epi": [C.POINTER(EpiProgram), M_, i32, M_, i32, M_, M_, C.c_uint32, vp, sz, vp],
    "coda_quantize_mxfp8": [M_, i32, M_, M_, vp],
    "coda_quantize_mxfp4": [M_, i32, M_, M_, vp],
    "coda_quantize_mxfp6": [M_, i32, M_, M_, vp],
    "coda_gemm_mx": [C.POINTER(EpiProgram), M_, M_, M_, M_, M_, M_, C.c_uint32, vp, sz, vp],
    "coda_linear_swiglu_fwd_workspace": [i64, i64, i32, i32, szp],
    "coda_linear_swiglu_fwd": [M_, M_, W_, f32, M_, M_, M_, i32, vp, sz, vp],
    "coda_linear_rmsnorm_residual_fwd_workspace": [i64, i64, i64, i32, szp],
    "coda_linear_rmsnorm_residual_fwd": [M_, W_, M_, M_, M_, i32, vp, sz, vp],
    "coda_linear_qknorm_rope_fwd_workspace": [i64, i64, i32, i32, szp],
    "coda_linear_qknorm_rope_fwd": [M_, M_, W_, M_, M_, M_, i32, f32, M_, M_, M_, M_, M_, i32, vp, sz, vp],
    "coda_linear_swiglu_bwd_workspace": [i64, i64, i64, i32, szp],
    "coda_linear_swiglu_bwd": [M_, W_, M_, M_, M_, W_, M_, M_, M_, M_, M_, M_, f32, M_, i32, vp, sz, vp],
    "coda_linear_rmsnorm_residual_bwd_workspace": [i64, i64, i64, i32, szp],
    "coda_linear_rmsnorm_residual_bwd": [M_, M_, W_, M_, M_, f32, i32, vp, sz, vp],
    "coda_linear_qknorm_rope_bwd_workspace": [i64, i64, i32, szp],
    "coda_linear_qknorm_rope_bwd": [M_, M_, M_, M_, M_, M_, M_, W_, M_, M_, M_, M_, M_, i32, f32, M_,
                                    M_, M_, M_, M_, M_, f32, M_, i32, vp, sz, vp],
    "coda_linear_cross_entropy_fwd_workspace": [i64, i64, i64, i32, szp],
    "coda_linear_cross_entropy_fwd": [M_, W_, M_, i32, M_, M_, M_, M_, M_, i32, vp, sz, vp],
    "coda_linear_cross_entropy_fwd_noalloc": [M_, W_, M_, i32, M_, M_, M_, M_, M_, vp],
    "coda_linear_cross_entropy_bwd_workspace": [i64, i64, i64, i64, i32, szp],
    "coda_linear_cross_entropy_bwd": [M_, W_, M_, i32, M_, M_, f32, M_, M_, f32, i64, i32, vp, sz, vp],
    "coda_linear_sigmoid_fwd_workspace": [i64, i64, i32, i32, szp],
    "coda_linear_sigmoid_fwd": [M_, M_, W_, f32, M_, M_, M_, i32, vp, sz, vp],
    "coda_linear_sigmoid_bwd_workspace": [i64, i64, i64, i32, szp],
    "coda_linear_sigmoid_bwd": [M_, W_, M_, M_, M_, W_, M_, M_, M_, M_, M_, M_, f32, M_, i32, vp, sz, vp],
    "coda_linear_gelu_fwd_workspace": [i64, i64, i32, i32, szp],
    "coda_linear_gelu_fwd": [M_, M_, W_, f32, M_, M_, M_, i32, vp, sz, vp],
    "coda_linear_gelu_bwd_workspace": [i64, i64, i64, i32, szp],
    "coda_linear_gelu_bwd": [M_, W_, M_, M_, M_, W_, M_, M_, M_, M_, M_, M_, f32, M_, i32, vp, sz, vp],
    "coda_linear_rmsnorm_cross_entropy_fwd_workspace": [i64, i64, i64, i32, i32, szp],
    "coda_linear_rmsnorm_cross_entropy_fwd": [M_, M_, W_, f32, M_, i32, M_, M_, M_, M_, M_, M_, i32, vp, sz, vp],
    "coda_linear_rmsnorm_cross_entropy_bwd_workspace": [i64, i64, i64, i64, i32, szp],
    "coda_linear_rmsnorm_cross_entropy_bwd": [M_, M_, W_, M_, M_, M_, i32, M_, M_, f32, M_, M_, M_, M_, f32, i64,
                                              i32, vp, sz, vp],
    # unfused baseline (include/coda_unfused.h)
    "coda_unfused_rmsnorm_fwd": [M_, M_, f32, M_, M_, vp],
    "coda_unfused_rmsnorm_bwd_workspace": [i64, i64, szp],
    "coda_unfused_rmsnorm_bwd": [M_, M_, M_, M_, M_, M_, M_, f32, vp, sz, vp],
    "coda_unfused_add": [M_, M_, M_, vp],
    "coda_unfused_swiglu_fwd": [M_, M_, vp],
    "coda_unfused_swiglu_bwd": [M_, M_, M_, vp],
    "coda_unfused_qknorm_rope_fwd": [M_, M_, M_, M_, i32, f32, M_, M_, vp],
    "coda_unfused_qknorm_rope_bwd_workspace": [i64, i64, szp],
    "coda_unfused_qknorm_rope_bwd": [M_, M_, M_, M_, M_, M_, M_, i32, f32, M_, M_, M_, f32, vp, sz, vp],
    # measurement helper (include/coda_probe.h)
    "coda_probe_mfma_loop": [i32, i32, i32, M_, C.POINTER(C.c_double), vp],
}
_RET = {"coda_status_string": C.c_char_p, "coda_last_error": C.c_char_p, "coda_partials_cols": C.c_int64}

_lib = None


def load(path: str = LIB_PATH):
    """Load libcoda.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libcoda.so not built at {path}: run gemm_epilogue_fp8_amd.build.build() first")
    lib = C.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RET.get(name, C.c_int)
    _lib = lib
    return lib
