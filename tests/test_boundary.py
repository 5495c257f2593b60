"""The C-ABI library loads on a GPU-less host, exports every function that
the headers under include/ declare, and rejects bad arguments before any HIP call.

No compute call is made here: every call fails host-side validation (fake,
never-dereferenced device pointers are used for the shape checks)."""
import ctypes as C
import os
import re

import pytest

import gemm_epilogue_fp8_amd as g
from gemm_epilogue_fp8_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = "".join(open(os.path.join(ROOT, "include", h)).read() for h in ("coda.h", "coda_unfused.h", "coda_probe.h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coda_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = g.lib()
    names = header_functions()
    assert len(names) >= 25
    for n in names:
        assert hasattr(L, n), f"{n} declared in coda.h but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    assert L.coda_abi_version() == 2


def test_status_strings():
    L = g.lib()
    for st in range(10):
        assert L.coda_status_string(st)
    assert L.coda_status_string(0) == b"ok"


FAKE = 1 << 40     # 16-byte aligned, never dereferenced (validation fails first)


def fake(dtype, rows, cols, ld=None, ptr=FAKE):
    m = _lib.CodaMat()
    m.ptr, m.dtype, m.rows, m.cols, m.ld = ptr, dtype, rows, cols, cols if ld is None else ld
    return m


def call_sumsq(x, out):
    L = g.lib()
    return L.coda_row_sumsq(C.byref(x) if x else None, C.byref(out) if out else None, None)


def test_validation_codes():
    L = g.lib()
    BF, F32 = _lib.CODA_BF16, _lib.CODA_F32
    x = fake(BF, 4, 8)
    assert call_sumsq(None, fake(F32, 1, 4)) == 1                      # NULL
    assert call_sumsq(fake(F32, 4, 8), fake(F32, 1, 4)) == 2           # dtype
    assert call_sumsq(x, fake(F32, 1, 5)) == 3                         # shape
    assert call_sumsq(fake(BF, 4, 8, ld=6), fake(F32, 1, 4)) == 4      # ld < cols
    assert call_sumsq(fake(BF, 4, 12, ld=12), fake(F32, 1, 4)) == 4    # cols not a multiple of 8
    assert call_sumsq(fake(BF, 4, 8, ptr=FAKE + 2), fake(F32, 1, 4)) == 5   # alignment
    assert b"aligned" in L.coda_last_error()


def test_gemm_epi_rejects_unknown_programs():
    L = g.lib()
    BF = _lib.CODA_BF16
    A, B, D = fake(BF, 64, 64), fake(BF, 64, 64), fake(BF, 64, 64)
    prog = _lib.EpiProgram()
    prog.n_ops = 2
    prog.ops[0].op = _lib.EPI_SWIGLU
    prog.ops[1].op = _lib.EPI_ROW_SCALE
    st = L.coda_gemm_epi(C.byref(prog), C.byref(A), 0, C.byref(B), 0, C.byref(D), None, 0, None, 0, None)
    assert st == 7 and b"not in the compiled set" in L.coda_last_error()
    prog.n_ops = 0
    assert L.coda_gemm_epi(C.byref(prog), C.byref(A), 0, C.byref(B), 0, C.byref(D), None, 0, None, 0, None) == 7
    prog.n_ops = 1
    prog.ops[0].op = _lib.EPI_STORE_BF16
    Bbad = fake(BF, 32, 64)
    assert L.coda_gemm_epi(C.byref(prog), C.byref(A), 0, C.byref(Bbad), 0, C.byref(D), None, 0, None, 0, None) == 3


def _prog(ops):
    prog = _lib.EpiProgram()
    prog.n_ops = len(ops)
    for i, (op, slots, fp) in enumerate(ops):
        slots = tuple(slots) + (0,) * (3 - len(slots))
        prog.ops[i].op, prog.ops[i].slot, prog.ops[i].slot2, prog.ops[i].slot3 = op, *slots
        prog.ops[i].fparam = fp
    return prog


def test_epilogue_descriptor_chains_and_operand_checks():
    """Every compiled chain is recognised (the workspace query accepts it) and
    its operands are checked before any launch: each case below is one
    chain with one wrong operand and the status it must return."""
    L = g.lib()
    BF, F32, I32, E4 = _lib.CODA_BF16, _lib.CODA_F32, _lib.CODA_I32, _lib.CODA_E4M3
    E = _lib
    M, N, K = 64, 768, 128
    tn = (N + 255) // 256
    n = C.c_size_t(123)
    chains = {
        "swiglu": [(E.EPI_ROW_RMS_FROM_PARTIALS, (0,), 1e-6), (E.EPI_STORE_ROW_VEC, (1,), 0), (E.EPI_SAVE_PRE, (2,), 0),
                   (E.EPI_SWIGLU, (), 0), (E.EPI_STORE_BF16, (), 0)],
        "sigmoid": [(E.EPI_ROW_SCALE, (0,), 0), (E.EPI_SIGMOID, (), 0), (E.EPI_STORE_BF16, (), 0)],
        "gelu": [(E.EPI_ROW_SCALE, (0,), 0), (E.EPI_SAVE_PRE, (1,), 0), (E.EPI_GELU, (), 0), (E.EPI_STORE_BF16, (), 0)],
        "qkrope": [(E.EPI_ROW_SCALE, (0,), 0), (E.EPI_SAVE_PRE, (1,), 0), (E.EPI_QKNORM_ROPE, (2, 3), 1e-6),
                   (E.EPI_STORE_BF16, (), 0)],
        "dswiglu": [(E.EPI_DSWIGLU, (0,), 0), (E.EPI_ROW_SCALE, (1,), 0), (E.EPI_STORE_BF16, (), 0),
                    (E.EPI_ROW_DOT_PARTIAL, (2,), 0)],
        "dsigmoid": [(E.EPI_DSIGMOID, (0,), 0), (E.EPI_ROW_SCALE, (1,), 0), (E.EPI_STORE_BF16, (), 0),
                     (E.EPI_ROW_DOT_PARTIAL, (2,), 0)],
        "dgelu": [(E.EPI_DGELU, (0,), 0), (E.EPI_ROW_SCALE, (1,), 0), (E.EPI_STORE_BF16, (), 0),
                  (E.EPI_ROW_DOT_PARTIAL, (2,), 0)],
        "normcorr": [(E.EPI_NORM_CORRECTION, (0, 1, 2), 0), (E.EPI_SCALE_DEV, (3,), 0), (E.EPI_ADD_TILE, (4,), 0),
                     (E.EPI_STORE_BF16, (), 0)],
        "wgrad": [(E.EPI_SCALE_DEV, (0,), 0), (E.EPI_WGRAD_GAIN, (1, 2, 3), 1.0)],
        "ce": [(E.EPI_CE_LSE_PARTIAL, (0, 1, 2), 0)],
        "ce_norm": [(E.EPI_ROW_RMS_FROM_PARTIALS, (0,), 1e-6), (E.EPI_CE_LSE_PARTIAL, (1, 2, 3), 0)],
        "ce_grad": [(E.EPI_CE_GRAD, (0, 1), 0), (E.EPI_STORE_BF16, (), 0)],
        "ce_grad_norm": [(E.EPI_ROW_SCALE, (0,), 0), (E.EPI_CE_GRAD, (1, 2), 0), (E.EPI_STORE_BF16, (), 0),
                         (E.EPI_ROW_DOT_PARTIAL, (3,), 0)],
        "store_dev": [(E.EPI_SCALE_DEV, (0,), 0), (E.EPI_STORE_BF16, (), 0)],
        "f32_dev": [(E.EPI_SCALE_DEV, (0,), 0), (E.EPI_ACCUM_F32, (), 1.0)],
        "fp8_resid": [(E.EPI_DEQUANT_E4M3, (0, 1), 0), (E.EPI_ADD_TILE, (2,), 0), (E.EPI_STORE_BF16, (), 0)],
    }
    for name, ops in chains.items():
        pr = _prog(ops)
        assert L.coda_gemm_epi_workspace(C.byref(pr), M, N, K, C.byref(n)) == 0, (name, L.coda_last_error())
        need = n.value
        assert need == (M * 4 if name in ("swiglu", "normcorr", "ce_norm") else 0), (name, need)
    pr = _prog([(E.EPI_SWIGLU, (), 0), (E.EPI_ROW_SCALE, (0,), 0)])
    assert L.coda_gemm_epi_workspace(C.byref(pr), M, N, K, C.byref(n)) == 7
    A, B, Bt = fake(BF, M, K), fake(BF, K, N), fake(BF, N, K)

    def run(ops, aux, D=fake(BF, M, N), A=A, B=B, tB=0, ws=None, nws=0):
        arr = (_lib.CodaMat * len(aux))(*aux)
        return L.coda_gemm_epi(C.byref(_prog(ops)), C.byref(A), 0, C.byref(B), tB, C.byref(D) if D else None,
                               arr, len(aux), ws, nws, None)

    v = lambda dt, k: fake(dt, 1, k)
    part = lambda rows: fake(F32, rows, M)
    # SwiGLU: partials with 33 rows; then the workspace missing for 12 rows
    sw = chains["swiglu"]
    assert run(sw, [part(33), v(F32, M), fake(BF, M, N)], D=fake(BF, M, N // 2)) == 3
    assert run(sw, [part(12), v(F32, M), fake(BF, M, N)], D=fake(BF, M, N // 2)) == 6
    assert run(sw, [part(4), v(F32, M), fake(BF, M, N + 8)], D=fake(BF, M, N // 2)) == 3      # save shape
    assert run(sw, [part(4), v(F32, M), fake(BF, M, N)], D=fake(BF, M, N)) == 3               # D is [M, N/2]
    # QK-norm + RoPE: gains [2, 128], table [seq, 128]; N must be 3 x 128 k
    qk = chains["qkrope"]
    good_qk = [v(F32, M), fake(BF, M, 2 * N // 3), fake(F32, 2, 128), fake(F32, 16, 128)]
    assert run(qk, [v(F32, M), fake(BF, M, 2 * N // 3), fake(F32, 1, 128), fake(F32, 16, 128)]) == 3
    assert run(qk, good_qk[:3] + [fake(F32, 16, 64)]) == 3
    assert run(qk, good_qk, D=fake(BF, M, 512), B=fake(BF, K, 512)) == 3                      # 512 % 384
    bad_eps = list(qk)
    bad_eps[0] = (E.EPI_ROW_RMS_FROM_PARTIALS, (0,), 1e-5)
    assert run(bad_eps, [part(1)] + good_qk[1:]) == 9                                        # two eps
    # dSwiGLU: saved [M, 2N], D [M, 2N], partials [tiles_n, M]
    ds = chains["dswiglu"]
    assert run(ds, [fake(BF, M, N), v(F32, M), part(tn)], D=fake(BF, M, 2 * N), B=Bt, tB=1) == 3
    assert run(ds, [fake(BF, M, 2 * N), v(F32, M), part(tn + 1)], D=fake(BF, M, 2 * N), B=Bt, tB=1) == 3
    # norm correction: u, r, T; r of the wrong length; a 2-element device scale
    nc = chains["normcorr"]
    assert run(nc, [fake(BF, M, N), v(F32, M + 1), part(2), v(F32, 1), fake(BF, M, N)], B=Bt, tB=1) == 3
    assert run(nc, [fake(BF, M, N), v(F32, M), part(2), v(F32, 2), fake(BF, M, N)], B=Bt, tB=1) == 3
    # weight gradient through the gain: D must be fp32
    wg = chains["wgrad"]
    At = fake(BF, K, M)
    arr = (_lib.CodaMat * 4)(v(F32, 1), fake(BF, M, N), v(F32, M), part(tn))
    assert L.coda_gemm_epi(C.byref(_prog(wg)), C.byref(At), 1, C.byref(B), 0, C.byref(fake(BF, M, N)), arr, 4,
                           None, 0, None) == 2
    # cross-entropy: labels int32, partials [2 tiles_n, M], D unused
    ce = chains["ce"]
    assert run(ce, [v(F32, M), part(2 * tn), v(F32, M)], D=None) == 2                        # labels dtype
    assert run(ce, [v(I32, M), part(tn), v(F32, M)], D=None) == 3                            # one partial set
    # a chain that exists but is not compiled for the layout: sigmoid on NT operands
    assert run(chains["sigmoid"], [v(F32, M)], B=Bt, tB=1) == 7
    assert run(chains["dgelu"], [fake(BF, M, N), v(F32, M), part(tn)], tB=0) == 7       # DGELU on NN operands
    # GELU: the saved pre-activation must be [M, N]; DGELU: the saved h [M, N]
    assert run(chains["gelu"], [v(F32, M), fake(BF, M, N + 8)]) == 3
    assert run(chains["dgelu"], [fake(BF, M, 2 * N), v(F32, M), part(tn)], B=Bt, tB=1) == 3
    # E4M3: A [M, K], B [N, K] only, scales [M] and [N]
    f8 = chains["fp8_resid"]
    A8, B8 = fake(E4, M, K), fake(E4, N, K)
    assert run(f8, [v(F32, M), v(F32, N), fake(BF, M, N)], A=A8, B=fake(E4, K, N), tB=0) == 4   # B layout
    assert run(f8, [v(F32, M), v(F32, N + 4), fake(BF, M, N)], A=A8, B=B8, tB=1) == 3
    assert run(f8, [v(F32, M), v(F32, N), fake(BF, M, N)], A=fake(BF, M, K), B=B8, tB=1) == 2    # A not E4M3


def test_functional_validation():
    L = g.lib()
    BF, F32, I32 = _lib.CODA_BF16, _lib.CODA_F32, _lib.CODA_I32
    x = fake(BF, 16, 64)
    w = _lib.CodaWeight()
    w.w = fake(BF, 64, 96)                 # 2F = 96 is not a multiple of 64
    out = fake(BF, 16, 48)
    st = L.coda_linear_swiglu_fwd(C.byref(x), None, C.byref(w), 1e-6, C.byref(out), None, None, 0, None, 0, None)
    assert st == 3
    w.w = fake(BF, 64, 128)
    out = fake(BF, 16, 64)
    # workspace required (no partials given) but none passed
    st = L.coda_linear_swiglu_fwd(C.byref(x), None, C.byref(w), 1e-6, C.byref(out), None, None, 0, None, 0, None)
    assert st == 6
    # bad precision
    st = L.coda_linear_swiglu_fwd(C.byref(x), None, C.byref(w), 1e-6, C.byref(out), None, None, 9, None, 0, None)
    assert st == 9
    # fp8 without quantised copies
    st = L.coda_linear_swiglu_fwd(C.byref(x), None, C.byref(w), 1e-6, C.byref(out), None, None, 1, None, 0, None)
    assert st == 1
    # cross-entropy: ignore index inside [0, V)
    h = fake(BF, 16, 64)
    wv = _lib.CodaWeight()
    wv.w = fake(BF, 64, 256)
    lab, loss, lse, nv = fake(I32, 1, 16), fake(F32, 1, 1), fake(F32, 1, 16), fake(I32, 1, 1)
    st = L.coda_linear_cross_entropy_fwd(C.byref(h), C.byref(wv), C.byref(lab), 3, C.byref(loss), C.byref(lse),
                                         None, C.byref(nv), None, 0, None, 0, None)
    assert st == 9
    # QKV needs D % 128 == 0
    xq = fake(BF, 16, 64)
    wq = _lib.CodaWeight()
    wq.w = fake(BF, 64, 192)
    st = L.coda_linear_qknorm_rope_fwd(C.byref(xq), None, C.byref(wq), None, None, None, 16, 1e-6, None, None,
                                       None, None, None, 0, None, 0, None)
    assert st == 3


def test_workspace_queries():
    L = g.lib()
    n = C.c_size_t(0)
    assert L.coda_linear_swiglu_bwd_workspace(8192, 4096, 11008, 0, C.byref(n)) == 0
    # T partials + collapsed T + gain partials + dh~ copy
    assert n.value >= 8192 * 2 * 11008 * 2
    m = C.c_size_t(0)
    assert L.coda_linear_swiglu_bwd_workspace(8192, 4096, 11008, 1, C.byref(m)) == 0
    assert m.value > n.value               # fp8 adds the quantised operands
    assert L.coda_linear_cross_entropy_bwd_workspace(8192, 2048, 128256, 1024, 0, C.byref(n)) == 0
    assert n.value >= 1024 * 128256 * 2
    assert g.partials_cols(128256) == 501 and g.partials_cols(1) == 1


def test_mx_validation_codes():
    """MXFP8 entry points: block-multiple sizes, E8M0 exponent matrices in
    word layout ([ceil(L/128), 4 rows]), dtype and 4-byte layout, checked
    before any HIP call."""
    L = g.lib()
    BF, E4, E8 = _lib.CODA_BF16, _lib.CODA_E4M3, _lib.CODA_E8M0
    q = lambda X, axis, Q, S: L.coda_quantize_mxfp8(C.byref(X), axis, C.byref(Q), C.byref(S), None)
    assert q(fake(BF, 40, 48), 1, fake(E4, 40, 48), fake(E8, 1, 160)) == 3      # 48 not a multiple of 32
    assert q(fake(BF, 40, 64), 0, fake(E4, 64, 40), fake(E8, 1, 256)) == 3      # 40 rows: not a multiple of 32
    assert q(fake(BF, 40, 64), 1, fake(E4, 40, 64), fake(E8, 1, 156)) == 3      # wrong byte count
    assert q(fake(BF, 40, 256), 1, fake(E4, 40, 256), fake(E8, 1, 160)) == 3    # 256 values = 2 word rows
    assert q(fake(BF, 40, 256), 1, fake(E4, 40, 256), fake(E4, 2, 160, ld=160)) == 2  # exponent dtype
    assert q(fake(BF, 40, 256), 1, fake(E4, 40, 256), fake(E8, 2, 160, ld=162)) == 4  # ld not a multiple of 4
    assert q(fake(BF, 40, 256), 1, fake(E4, 40, 256), fake(E8, 2, 160, ptr=FAKE + 2)) == 5
    assert q(fake(BF, 40, 256), 2, fake(E4, 40, 256), fake(E8, 2, 160)) == 9   # axis

    prog = _lib.EpiProgram()
    prog.n_ops = 1
    prog.ops[0].op = _lib.EPI_STORE_BF16
    gm = lambda A, SA, B, SB, D: L.coda_gemm_mx(C.byref(prog), C.byref(A), C.byref(SA), C.byref(B), C.byref(SB),
                                                C.byref(D), None, 0, None, 0, None)
    M, N = 64, 32
    assert gm(fake(E4, M, 192), fake(E8, 2, 4 * M), fake(E4, N, 192), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 3                                             # K = 192: not a multiple of 128
    assert gm(fake(E4, M, 256), fake(E8, 2, 4 * M), fake(E4, N, 128), fake(E8, 1, 4 * N),
              fake(BF, M, N)) == 3                                             # inner sizes differ
    assert gm(fake(E4, M, 256), fake(E8, 1, 4 * M), fake(E4, N, 256), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 3                                             # SA has 1 word row, K needs 2
    assert gm(fake(E4, M, 256), fake(E8, 2, M), fake(E4, N, 256), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 3                                             # SA is not 4 M bytes wide
    assert gm(fake(BF, M, 256), fake(E8, 2, 4 * M), fake(E4, N, 256), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 2                                             # A not E4M3
    assert gm(fake(E4, M, 256), fake(E8, 2, 4 * M), fake(E4, N, 256), fake(E8, 2, 4 * N),
              fake(BF, M, N + 8)) == 3                                         # D shape


def test_mxfp8_functional_validation():
    """MXFP8 precision: weight dimensions must be multiples of 128, the
    block-scaled copies must carry E8M0 exponents in word layout, and the
    tokens of a backward must be a multiple of 128."""
    L = g.lib()
    BF, F32, E4, E8 = _lib.CODA_BF16, _lib.CODA_F32, _lib.CODA_E4M3, _lib.CODA_E8M0
    MX = _lib.PREC_MXFP8

    def weight(K, N, sdt=E8):
        w = _lib.CodaWeight()
        w.w = fake(BF, K, N)
        w.q_fwd, w.q_bwd = fake(E4, N, K), fake(E4, K, N)
        if sdt == E8:
            w.s_fwd, w.s_bwd = fake(E8, (K + 127) // 128, 4 * N), fake(E8, (N + 127) // 128, 4 * K)
        else:
            w.s_fwd, w.s_bwd = fake(F32, 1, N), fake(F32, 1, K)
        return w

    def fwd(M, K, N, w):
        a, z, out = fake(BF, M, K), fake(BF, M, N), fake(BF, M, N)
        return L.coda_linear_rmsnorm_residual_fwd(C.byref(a), C.byref(w), C.byref(z), C.byref(out), None, MX,
                                                  None, 0, None)

    assert fwd(64, 192, 256, weight(192, 256)) == 3          # K_in = 192: not a multiple of 128
    assert fwd(64, 256, 192, weight(256, 192)) == 3          # N_out = 192
    assert fwd(64, 256, 256, weight(256, 256, F32)) == 2     # per-channel scales given for MXFP8
    w = weight(256, 256)
    w.s_bwd = fake(E8, 3, 4 * 256)                           # one word row too many
    assert fwd(64, 256, 256, w) == 3
    assert fwd(64, 256, 256, weight(256, 256)) == 6          # valid; the activation copy needs a workspace
    # backward with 200 tokens
    d_out, a, dW = fake(BF, 200, 256), fake(BF, 200, 256), fake(F32, 256, 256)
    st = L.coda_linear_rmsnorm_residual_bwd(C.byref(d_out), C.byref(a), C.byref(weight(256, 256)), None,
                                            C.byref(dW), 0.0, MX, None, 0, None)
    assert st == 3


def test_probe_validation_codes():
    """The MFMA-loop probe rejects bad arguments before any launch."""
    L = g.lib()
    fl = C.c_double(0.0)
    out = fake(_lib.CODA_F32, 1, 12)
    call = lambda dt, b, it, o=out, f=C.byref(fl): L.coda_probe_mfma_loop(dt, b, it, C.byref(o) if o else None, f, None)
    assert call(_lib.CODA_F32, 4, 10) == 2                       # dtype
    assert call(_lib.CODA_BF16, 0, 10) == 3                      # blocks
    assert call(_lib.CODA_BF16, 4, 0) == 3                       # iters
    assert call(_lib.CODA_BF16, 4, 1 << 21) == 3
    assert call(_lib.CODA_BF16, 4, 10, f=None) == 1              # flops pointer
    assert call(_lib.CODA_BF16, 4, 10, o=None) == 1              # out
    assert call(_lib.CODA_BF16, 5, 10) == 3                      # out holds 3 values a block


def test_row_stride_limit():
    """A matrix whose row stride reaches 16 MiB is rejected (tile rows are
    addressed by 32-bit offsets); one byte row below the limit passes the
    stride check."""
    BF, F32 = _lib.CODA_BF16, _lib.CODA_F32
    big = (1 << 23)                                    # bf16 elements: 16 MiB a row
    assert call_sumsq(fake(BF, 4, 8, ld=big), fake(F32, 1, 4)) == 4          # layout
    ok = call_sumsq(fake(BF, 4, 8, ld=big - 8), fake(F32, 1, 3))           # passes the stride check,
    assert ok == 3                                                          # then fails on the output shape


def test_mxfp4_quantiser_validation_codes():
    """coda_quantize_mxfp4 checks axis, block multiple, the packed Q shape and
    dtype, and the exponent layout before any launch."""
    L = g.lib()
    BF, E4, E2, E8 = _lib.CODA_BF16, _lib.CODA_E4M3, _lib.CODA_E2M1X2, _lib.CODA_E8M0
    X = fake(BF, 64, 96)
    q_ok, s_ok = fake(E2, 64, 48), fake(E8, 1, 256)
    call = lambda x, ax, q, s: L.coda_quantize_mxfp4(C.byref(x), ax, C.byref(q), C.byref(s), None)
    assert call(X, 2, q_ok, s_ok) == 9                                   # axis
    assert call(fake(BF, 64, 80), 1, fake(E2, 64, 40), s_ok) == 3        # 80 not a multiple of 32
    assert call(X, 1, fake(E4, 64, 48), s_ok) == 2                       # Q dtype
    assert call(X, 1, fake(E2, 64, 96), s_ok) == 3                       # Q holds C / 2 bytes a row
    assert call(X, 1, q_ok, fake(E8, 2, 256)) == 3                       # word rows: ceil(96 / 128) = 1
    # transposed shapes pass the Q and S shape checks and stop at S's alignment
    assert call(X, 0, fake(E2, 96, 32), fake(E8, 1, 384, ptr=FAKE + 2)) == 5


def test_mxfp6_quantiser_validation_codes():
    """coda_quantize_mxfp6 takes its format from Q's dtype (E2M3 or E3M2) and
    checks axis, block multiple, Q's shape (a byte a value) and the exponent
    layout before any launch."""
    L = g.lib()
    BF, E4, E8 = _lib.CODA_BF16, _lib.CODA_E4M3, _lib.CODA_E8M0
    X = fake(BF, 64, 96)
    s_ok = fake(E8, 1, 256)
    call = lambda x, ax, q, s: L.coda_quantize_mxfp6(C.byref(x), ax, C.byref(q), C.byref(s), None)
    for F6 in (_lib.CODA_E2M3, _lib.CODA_E3M2):
        q_ok = fake(F6, 64, 96)
        assert call(X, 2, q_ok, s_ok) == 9                               # axis
        assert call(fake(BF, 64, 80), 1, fake(F6, 64, 80), s_ok) == 3    # 80 not a multiple of 32
        assert call(X, 1, fake(F6, 64, 48), s_ok) == 3                   # Q holds C bytes a row
        assert call(X, 1, q_ok, fake(E8, 2, 256)) == 3                   # word rows: ceil(96 / 128) = 1
        assert call(X, 0, fake(F6, 96, 64), fake(E8, 1, 384, ptr=FAKE + 2)) == 5   # transposed: S alignment
    assert call(X, 1, fake(E4, 64, 96), s_ok) == 2                       # Q neither FP6 dtype
    assert call(X, 1, fake(_lib.CODA_E2M1X2, 64, 48), s_ok) == 2


def test_mxfp6_gemm_validation_codes():
    """coda_gemm_mx with FP6 operands: B must carry A's FP6 dtype, K a
    multiple of 128 and the exponents sized for K values."""
    L = g.lib()
    BF, E8, E23, E32 = _lib.CODA_BF16, _lib.CODA_E8M0, _lib.CODA_E2M3, _lib.CODA_E3M2
    prog = _lib.EpiProgram()
    prog.n_ops = 1
    prog.ops[0].op = _lib.EPI_STORE_BF16
    gm = lambda A, SA, B, SB, D: L.coda_gemm_mx(C.byref(prog), C.byref(A), C.byref(SA), C.byref(B), C.byref(SB),
                                                C.byref(D), None, 0, None, 0, None)
    M, N = 64, 32
    assert gm(fake(E23, M, 256), fake(E8, 2, 4 * M), fake(E32, N, 256), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 2                                             # formats differ
    assert gm(fake(E32, M, 96), fake(E8, 1, 4 * M), fake(E32, N, 96), fake(E8, 1, 4 * N),
              fake(BF, M, N)) == 3                                             # K = 96
    assert gm(fake(E23, M, 256), fake(E8, 1, 4 * M), fake(E23, N, 256), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 3                                             # 256 values need 2 word rows
    assert gm(fake(E23, M, 256), fake(E8, 2, 4 * M), fake(E23, N, 256), fake(E8, 2, 4 * N),
              fake(BF, M, N + 8)) == 3                                         # D shape


def test_mxfp4_gemm_validation_codes():
    """coda_gemm_mx with E2M1X2 operands: both operands must be E2M1X2, K
    (twice the byte count) a multiple of 128, and the exponents sized for K
    values, all checked before any launch."""
    L = g.lib()
    BF, E4, E2, E8 = _lib.CODA_BF16, _lib.CODA_E4M3, _lib.CODA_E2M1X2, _lib.CODA_E8M0
    prog = _lib.EpiProgram()
    prog.n_ops = 1
    prog.ops[0].op = _lib.EPI_STORE_BF16
    gm = lambda A, SA, B, SB, D: L.coda_gemm_mx(C.byref(prog), C.byref(A), C.byref(SA), C.byref(B), C.byref(SB),
                                                C.byref(D), None, 0, None, 0, None)
    M, N = 64, 32
    assert gm(fake(E2, M, 128), fake(E8, 2, 4 * M), fake(E4, N, 128), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 2                                             # B is not E2M1X2
    assert gm(fake(E2, M, 96), fake(E8, 2, 4 * M), fake(E2, N, 96), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 3                                             # K = 192 values
    assert gm(fake(E2, M, 128), fake(E8, 1, 4 * M), fake(E2, N, 128), fake(E8, 2, 4 * N),
              fake(BF, M, N)) == 3                                             # 256 values need 2 word rows
    assert gm(fake(E2, M, 128), fake(E8, 2, 4 * M), fake(E2, N, 128), fake(E8, 2, 4 * N),
              fake(BF, M, N + 8)) == 3                                         # D shape


def test_mxfp6_weight_validation_codes():
    """The MXFP6 precisions check the weight copies before any launch: q_fwd
    [N, K] of the precision's FP6 dtype with exponents of N rows along K_in
    (K_in a multiple of 128), the optional q_bwd [K, N] likewise along N_out."""
    L = g.lib()
    BF, E8 = _lib.CODA_BF16, _lib.CODA_E8M0
    E23, E32 = _lib.CODA_E2M3, _lib.CODA_E3M2
    M, K, N = 64, 256, 128

    def weight(qdt, qf=(N, K), qb=(K, N), K_=K):
        w = _lib.CodaWeight()
        w.w = fake(BF, K_, N)
        w.q_fwd, w.s_fwd = fake(qdt, *qf), fake(E8, (K_ + 127) // 128, 4 * N)
        w.q_bwd, w.s_bwd = fake(qdt, *qb), fake(E8, (N + 127) // 128, 4 * K_)
        return w

    def call(w, prec, K_=K):
        a, res, out = fake(BF, M, K_), fake(BF, M, N), fake(BF, M, N)
        return L.coda_linear_rmsnorm_residual_fwd(C.byref(a), C.byref(w), C.byref(res), C.byref(out), None, prec,
                                                  None, 0, None)

    for prec, dt, other in ((_lib.PREC_MXFP6_E2M3, E23, E32), (_lib.PREC_MXFP6_E3M2, E32, E23)):
        assert call(weight(dt), prec) == 6                                # valid weight; stops at the workspace
        assert call(weight(other), prec) == 2                             # the other FP6 format
        assert call(weight(_lib.CODA_E2M1X2, qf=(N, K // 2)), prec) == 2   # E2M1 copies
        assert call(weight(dt, qf=(N, K // 2)), prec) == 3                # FP6 is a byte a value
        assert call(weight(dt, qb=(K, N // 2)), prec) == 3                # input-gradient copy shape
        assert call(weight(dt, K_=192), prec, K_=192) == 3                # K_in not a multiple of 128


def test_schedule_setting():
    """The launch schedule is process-wide: set, read back, unknown values refused."""
    L = g.lib()
    assert L.coda_get_schedule() == _lib.SCHED_PINGPONG
    assert L.coda_set_schedule(_lib.SCHED_CORESIDENT) == 0
    assert L.coda_get_schedule() == _lib.SCHED_CORESIDENT
    assert L.coda_set_schedule(2) == 9 and L.coda_set_schedule(-1) == 9
    assert L.coda_get_schedule() == _lib.SCHED_CORESIDENT
    with g.schedule(_lib.SCHED_PINGPONG):
        assert L.coda_get_schedule() == _lib.SCHED_PINGPONG
    assert L.coda_get_schedule() == _lib.SCHED_CORESIDENT
    assert L.coda_set_schedule(_lib.SCHED_PINGPONG) == 0


def test_empty_normalised_rows_and_null_empty_matrices():
    """A normalised row of width 0 has no RMS: the RMSNorm entry points refuse
    it before any HIP call.  An empty required matrix may carry a NULL
    pointer, and a non-empty one may not."""
    L = g.lib()
    BF, F32 = _lib.CODA_BF16, _lib.CODA_F32
    M, N = 16, 128
    w = _lib.CodaWeight()
    w.w = fake(BF, 0, N)
    x0 = fake(BF, M, 0)
    st = L.coda_linear_swiglu_fwd(C.byref(x0), None, C.byref(w), 1e-6, C.byref(fake(BF, M, N // 2)), None, None,
                                  0, None, 0, None)
    assert st == 3 and b"K = 0" in L.coda_last_error()
    for fn in (L.coda_linear_sigmoid_fwd, L.coda_linear_gelu_fwd):
        assert fn(C.byref(x0), None, C.byref(w), 1e-6, C.byref(fake(BF, M, N)), None, None, 0, None, 0, None) == 3
    # a required input with rows but no pointer
    w.w = fake(BF, 64, N)
    st = L.coda_linear_sigmoid_fwd(C.byref(fake(BF, M, 64, ptr=None)), None, C.byref(w), 1e-6,
                                   C.byref(fake(BF, M, N)), None, None, 0, None, 0, None)
    assert st == 1
    # M = 0 with NULL pointers passes validation (its sizes are still checked)
    assert L.coda_linear_sigmoid_fwd(C.byref(fake(BF, 0, 64, ptr=None)), None, C.byref(w), 1e-6,
                                     C.byref(fake(BF, 0, N + 8, ptr=None)), None, None, 0, None, 0, None) == 3
