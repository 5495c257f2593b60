// C ABI of the GEMM+epilogue library: host-side validation, workspace
// carving and the launch sequences of the functional entry points.  See
// include/coda.h for the contract of every entry point.
#include <atomic>
#include <mutex>

#include "capi_util.hpp"
#include "aux_kernels.hpp"
#include "launch.hpp"

using namespace coda;

namespace coda {
std::string& last_error_slot() {
  static thread_local std::string e;
  return e;
}
}  // namespace coda

namespace {

// ---------------------------------------------------------------- fp8 operand staging
struct Q8 { uint8_t* q; float* s; int64_t ld; };

// Quantise X [R, C] (bf16) along `axis` into workspace-carved buffers.
// axis 1: Q [R, C], scale per row.  axis 0: Q^T [C, R], scale per column.
Q8 take_q8(Carver& cv, int64_t R, int64_t C, int axis) {
  Q8 q;
  const int64_t rows = axis == 1 ? R : C, cols = axis == 1 ? C : R;
  q.ld = (cols + 15) / 16 * 16;
  q.q = cv.take<uint8_t>((size_t)rows * q.ld);
  q.s = cv.take<float>(rows);
  return q;
}
float* take_amax_ws(Carver& cv, int64_t R, int64_t C, int axis) {
  if (axis == 1) return cv.take<float>(R);
  const int64_t parts = (R + 255) / 256;
  cv.take<float>(C);                       // amax
  return cv.take<float>((size_t)parts * C);  // partials
}

coda_status run_quant(const void* X, int64_t ldx, int64_t R, int64_t C, int axis, uint8_t* Q, int64_t ldq,
                      float* scale, float* amax, float* parts, hipStream_t s) {
  const int64_t ns = axis == 1 ? R : C;   // one scale per row (axis 1) or per column (axis 0)
  if (R == 0 || C == 0) {
    // an empty contracted axis has amax 0, whose scale is 1 (no codes to scale)
    if (ns == 0) return CODA_OK;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, s, scale, (int)ns, 1.0f);
    return check_launch("quantize_e4m3: empty axis");
  }
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (axis == 1) {
    hipLaunchKernelGGL(quant_rows_kernel, dim3((R + 3) / 4), dim3(256), 0, s, x, ldx, (int)R, (int)C, Q, ldq, scale);
  } else {
    const int rpb = 256;
    const int nparts = (int)((R + rpb - 1) / rpb);
    hipLaunchKernelGGL(amax_cols_partial_kernel, dim3((C / 2 + 255) / 256, nparts), dim3(256), 0, s, x, ldx,
                       (int)R, (int)C, rpb, parts);
    hipLaunchKernelGGL(amax_cols_finish_kernel, dim3((C + 255) / 256), dim3(256), 0, s, parts, nparts, (int)C, amax);
    hipLaunchKernelGGL(quant_cols_t_kernel, dim3((C + 63) / 64, (R + 63) / 64), dim3(256), 0, s, x, ldx, (int)R,
                       (int)C, amax, Q, ldq, scale);
  }
  return check_launch("quantize_e4m3");
}

// Activation operand of a GEMM in fp8: quantised into the workspace, either
// with one amax scale per row of the operand (q.s) or, for MXFP8, with one
// E8M0 exponent per 32 values of the contracted axis (e, word layout: ceil(L /
// 128) word rows of 4 rows bytes, stride e_ld).
struct ActQ {
  Q8 q;
  float* amax;
  float* parts;
  bool mx;
  // block-scaled element format as the scaled MFMA codes it: 0 = E4M3,
  // 2 = E2M3 and 3 = E3M2 (FP6, a byte a value with the block padding),
  // 4 = E2M1 (two codes a byte; q.ld counts bytes)
  int elem;
  uint8_t* e;
  int64_t e_ld;
};
ActQ take_act(Carver& cv, int64_t R, int64_t C, int axis, bool mx = false, int elem = 0) {
  ActQ a{};
  a.mx = mx;
  a.elem = elem;
  if (mx) {
    const int64_t rows = axis == 1 ? R : C, L = axis == 1 ? C : R;
    a.q.ld = ((elem == 4 ? L / 2 : L) + 15) / 16 * 16;
    a.q.q = cv.take<uint8_t>((size_t)rows * a.q.ld);
    a.q.s = nullptr;
    a.e_ld = 4 * rows;
    a.e = cv.take<uint8_t>((size_t)((L + 127) / 128) * a.e_ld);
    return a;
  }
  a.q = take_q8(cv, R, C, axis);
  if (axis == 1) { a.amax = cv.take<float>(R); a.parts = nullptr; }
  else { a.amax = cv.take<float>(C); a.parts = cv.take<float>((size_t)((R + 255) / 256) * C); }
  return a;
}
coda_status run_quant_mx(const void* X, int64_t ldx, int64_t R, int64_t C, int axis, uint8_t* Q, int64_t ldq,
                         uint8_t* E, int64_t lde, hipStream_t s) {
  if (R == 0 || C == 0) return CODA_OK;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (axis == 1)
    hipLaunchKernelGGL(quant_mx_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, x, ldx, (int)R, (int)C,
                       Q, ldq, E, lde);
  else
    hipLaunchKernelGGL(quant_mx_cols_t_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)), dim3(256),
                       0, s, x, ldx, (int)R, (int)C, Q, ldq, E, lde);
  return check_launch("quantize_mxfp8");
}
coda_status run_quant_mx4(const void* X, int64_t ldx, int64_t R, int64_t C, int axis, uint8_t* Q, int64_t ldq,
                          uint8_t* E, int64_t lde, hipStream_t s) {
  if (R == 0 || C == 0) return CODA_OK;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (axis == 1)
    hipLaunchKernelGGL(quant_mx4_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, x, ldx, (int)R, (int)C,
                       Q, ldq, E, lde);
  else
    hipLaunchKernelGGL(quant_mx4_cols_t_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)),
                       dim3(256), 0, s, x, ldx, (int)R, (int)C, Q, ldq, E, lde);
  return check_launch("quantize_mxfp4");
}
coda_status run_quant_mx6(const void* X, int64_t ldx, int64_t R, int64_t C, int axis, uint8_t* Q, int64_t ldq,
                          uint8_t* E, int64_t lde, int f6, hipStream_t s) {
  if (f6 != 2 && f6 != 3) return fail(CODA_ERR_VALUE, "quantize_mxfp6: element format %d", f6);
  if (R == 0 || C == 0) return CODA_OK;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (axis == 1)
    hipLaunchKernelGGL(quant_mx6_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, x, ldx, (int)R, (int)C,
                       Q, ldq, E, lde, f6);
  else
    hipLaunchKernelGGL(quant_mx6_cols_t_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)),
                       dim3(256), 0, s, x, ldx, (int)R, (int)C, Q, ldq, E, lde, f6);
  return check_launch("quantize_mxfp6");
}
coda_status quant_act(const ActQ& a, const void* X, int64_t ldx, int64_t R, int64_t C, int axis, hipStream_t s) {
  if (a.elem == 4) return run_quant_mx4(X, ldx, R, C, axis, a.q.q, a.q.ld, a.e, a.e_ld, s);
  if (a.elem) return run_quant_mx6(X, ldx, R, C, axis, a.q.q, a.q.ld, a.e, a.e_ld, a.elem, s);
  if (a.mx) return run_quant_mx(X, ldx, R, C, axis, a.q.q, a.q.ld, a.e, a.e_ld, s);
  return run_quant(X, ldx, R, C, axis, a.q.q, a.q.ld, a.q.s, a.amax, a.parts, s);
}
// A forward GEMM: MXFP4 and MXFP6 operands go to their own instantiations
// (for MXFP4 K counts bytes); elem as in ActQ
hipError_t launch_fwd(Prog p, int layout, bool fp8, int elem, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  if (elem == 4) return launch_gemm_mx4(p, g, e, s);
  if (elem) return launch_gemm_mx6(p, elem, g, e, s);
  return launch_gemm(p, layout, fp8, g, e, s);
}
// A GEMM at a functional precision: MXFP4 operands go to their own
// instantiations, whose mainloop counts the contracted axis (K and a split's
// kchunk) in bytes, two E2M1 values a byte
hipError_t launch_prec(Prog p, int layout, int prec, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  if (prec == CODA_PREC_MXFP4) {
    g.K /= 2;
    g.kchunk /= 2;
    return launch_gemm_mx4(p, g, e, s);
  }
  if (prec == CODA_PREC_MXFP6_E2M3) return launch_gemm_mx6(p, 2, g, e, s);
  if (prec == CODA_PREC_MXFP6_E3M2) return launch_gemm_mx6(p, 3, g, e, s);
  return launch_gemm(p, layout, prec != CODA_PREC_BF16, g, e, s);
}
// MXFP8 / MXFP4: the exponents of both operands go with the GEMM; the epilogue applies
// no dequantisation scales
void mx_args(GemmArgs* g, EpiArgs* e, const void* ea, int64_t lda_e, const coda_mat* eb) {
  g->sA = ea;
  g->lds_a = lda_e;
  g->sB = eb->ptr;
  g->lds_b = eb->rows > 1 ? eb->ld : eb->cols;
  e->rowscale = nullptr;
  e->colscale = nullptr;
}

// E8M0 block exponents of an operand with `nrows` rows and a contracted
// axis of L values, in word layout: ceil(L / 128) word rows of 4 nrows
// bytes; byte (g, 4 r + j) is the exponent of block 4 g + j of row r.
// Word rows are whole 4-byte words (ld % 4 == 0, pointer 4-byte aligned):
// the GEMM moves the exponents of 128 K values of a row as one word.
coda_status check_scales(const coda_mat* S, const char* name, int64_t nrows, int64_t L) {
  if (!present(S)) return fail(CODA_ERR_NULL, "%s: required pointer is NULL", name);
  if (S->dtype != CODA_E8M0) return fail(CODA_ERR_DTYPE, "%s: dtype %d, expected E8M0", name, S->dtype);
  const int64_t rows = (L + 127) / 128, cols = 4 * nrows;
  if (S->rows != rows || S->cols != cols)
    return fail(CODA_ERR_SHAPE, "%s: %lld x %lld, expected %lld x %lld (word layout)", name, (long long)S->rows,
                (long long)S->cols, (long long)rows, (long long)cols);
  if (reinterpret_cast<uintptr_t>(S->ptr) % 4 != 0) return fail(CODA_ERR_ALIGN, "%s: pointer not 4-byte aligned", name);
  if (S->rows > 1 && (S->ld < S->cols || S->ld % 4 != 0))
    return fail(CODA_ERR_LAYOUT, "%s: ld must be >= cols and a multiple of 4", name);
  return CODA_OK;
}

coda_status check_weight(const coda_weight* wt, const char* name, int64_t K, int64_t N, int precision) {
  if (!wt) return fail(CODA_ERR_NULL, "%s: NULL weight", name);
  TRY(check_mat(&wt->w, name, CODA_BF16, K, N));
  if (precision == CODA_PREC_FP8) {
    TRY(check_mat(&wt->q_fwd, "q_fwd", CODA_E4M3, N, K));
    TRY(check_vec(&wt->s_fwd, "s_fwd", CODA_F32, N));
    TRY(check_mat(&wt->q_bwd, "q_bwd", CODA_E4M3, K, N));
    TRY(check_vec(&wt->s_bwd, "s_bwd", CODA_F32, K));
  } else if (precision == CODA_PREC_MXFP8) {
    if (K % 128 != 0 || N % 128 != 0)
      return fail(CODA_ERR_SHAPE, "%s: MXFP8 needs both weight dimensions to be multiples of 128", name);
    TRY(check_mat(&wt->q_fwd, "q_fwd", CODA_E4M3, N, K));
    TRY(check_scales(&wt->s_fwd, "s_fwd", N, K));
    TRY(check_mat(&wt->q_bwd, "q_bwd", CODA_E4M3, K, N));
    TRY(check_scales(&wt->s_bwd, "s_bwd", K, N));
  } else if (precision == CODA_PREC_MXFP4) {
    // forward copy q_fwd [N, K / 2 bytes] with blocks along K_in; the
    // input-gradient copy q_bwd [K, N / 2 bytes] with blocks along N_out is
    // optional (a forward-only weight has none; dgrad refuses such a weight)
    if (K % 128 != 0) return fail(CODA_ERR_SHAPE, "%s: MXFP4 needs K_in to be a multiple of 128", name);
    TRY(check_mat(&wt->q_fwd, "q_fwd", CODA_E2M1X2, N, K / 2));
    TRY(check_scales(&wt->s_fwd, "s_fwd", N, K));
    if (present(&wt->q_bwd)) {
      if (N % 128 != 0) return fail(CODA_ERR_SHAPE, "%s: an MXFP4 backward copy needs N_out to be a multiple of 128", name);
      TRY(check_mat(&wt->q_bwd, "q_bwd", CODA_E2M1X2, K, N / 2));
      TRY(check_scales(&wt->s_bwd, "s_bwd", K, N));
    }
  } else if (precision == CODA_PREC_MXFP6_E2M3 || precision == CODA_PREC_MXFP6_E3M2) {
    // forward copy q_fwd [N, K] of the precision's FP6 dtype with blocks
    // along K_in; the input-gradient copy q_bwd [K, N] (blocks along N_out)
    // is optional as for MXFP4
    const int dt = precision == CODA_PREC_MXFP6_E2M3 ? CODA_E2M3 : CODA_E3M2;
    if (K % 128 != 0) return fail(CODA_ERR_SHAPE, "%s: MXFP6 needs K_in to be a multiple of 128", name);
    TRY(check_mat(&wt->q_fwd, "q_fwd", dt, N, K));
    TRY(check_scales(&wt->s_fwd, "s_fwd", N, K));
    if (present(&wt->q_bwd)) {
      if (N % 128 != 0) return fail(CODA_ERR_SHAPE, "%s: an MXFP6 backward copy needs N_out to be a multiple of 128", name);
      TRY(check_mat(&wt->q_bwd, "q_bwd", dt, K, N));
      TRY(check_scales(&wt->s_bwd, "s_bwd", K, N));
    }
  } else if (precision != CODA_PREC_BF16) {
    return fail(CODA_ERR_VALUE, "precision %d", precision);
  }
  return CODA_OK;
}
coda_status check_precision(int p) {
  if (p != CODA_PREC_BF16 && p != CODA_PREC_FP8 && p != CODA_PREC_MXFP8 && p != CODA_PREC_MXFP4 &&
      p != CODA_PREC_MXFP6_E2M3 && p != CODA_PREC_MXFP6_E3M2)
    return fail(CODA_ERR_VALUE, "precision %d", p);
  return CODA_OK;
}
coda_status check_precision_fwd(int p) { return check_precision(p); }
bool is_mx(int p) {
  return p == CODA_PREC_MXFP8 || p == CODA_PREC_MXFP4 || p == CODA_PREC_MXFP6_E2M3 || p == CODA_PREC_MXFP6_E3M2;
}
// the ActQ element code of a precision (0 for E4M3 and bf16)
int prec_elem(int p) {
  return p == CODA_PREC_MXFP4 ? 4 : p == CODA_PREC_MXFP6_E2M3 ? 2 : p == CODA_PREC_MXFP6_E3M2 ? 3 : 0;
}


// Forward-direction GEMM of an activation a [M, K] with a weight [K, N].
// bf16: NN with the stored weight.  fp8: quantise a per row, NT with q_fwd.
struct FwdOperands {
  GemmArgs g;
  int layout;
  bool fp8;
};

}  // namespace

// ======================================================================== misc
extern "C" int coda_abi_version(void) { return CODA_ABI_VERSION; }

extern "C" const char* coda_status_string(int st) {
  switch (st) {
    case CODA_OK: return "ok";
    case CODA_ERR_NULL: return "null pointer";
    case CODA_ERR_DTYPE: return "wrong dtype";
    case CODA_ERR_SHAPE: return "bad shape";
    case CODA_ERR_LAYOUT: return "bad layout";
    case CODA_ERR_ALIGN: return "misaligned pointer";
    case CODA_ERR_WORKSPACE: return "workspace too small";
    case CODA_ERR_UNSUPPORTED: return "unsupported";
    case CODA_ERR_LAUNCH: return "kernel launch failed";
    case CODA_ERR_VALUE: return "invalid value";
    default: return "unknown status";
  }
}

extern "C" const char* coda_last_error(void) { return coda::last_error_slot().c_str(); }

namespace coda {
static std::atomic<int> g_schedule{CODA_SCHED_PINGPONG};
bool coresident_schedule() { return g_schedule.load(std::memory_order_relaxed) == CODA_SCHED_CORESIDENT; }
}  // namespace coda

extern "C" coda_status coda_set_schedule(int32_t schedule) {
  if (schedule != CODA_SCHED_PINGPONG && schedule != CODA_SCHED_CORESIDENT)
    return fail(CODA_ERR_VALUE, "unknown schedule %d", (int)schedule);
  coda::g_schedule.store(schedule, std::memory_order_relaxed);
  return CODA_OK;
}

extern "C" int32_t coda_get_schedule(void) { return coda::g_schedule.load(std::memory_order_relaxed); }

extern "C" int64_t coda_partials_cols(int64_t N) { return (N + kBN - 1) / kBN; }

// ======================================================================== prep
extern "C" coda_status coda_fold_gain(const coda_mat* W, const coda_mat* g, const coda_mat* W_out, void* stream) {
  TRY(check_mat(W, "W", CODA_BF16, -1, -1));
  TRY(check_vec(g, "g", CODA_F32, W->rows));
  TRY(check_mat(W_out, "W_out", CODA_BF16, W->rows, W->cols));
  if (W->rows == 0 || W->cols == 0) return CODA_OK;
  hipLaunchKernelGGL(fold_gain_kernel, dim3((unsigned)((W->cols / 4 + 255) / 256), (unsigned)W->rows), dim3(256), 0,
                     S(stream), static_cast<const uint16_t*>(W->ptr), W->ld, static_cast<const float*>(g->ptr),
                     static_cast<uint16_t*>(W_out->ptr), W_out->ld, (int)W->rows, (int)W->cols);
  return check_launch("fold_gain");
}

extern "C" coda_status coda_pack_gate_up(const coda_mat* Wg, const coda_mat* Wu, const coda_mat* g_or_null,
                                         const coda_mat* Wgu_out, void* stream) {
  TRY(check_mat(Wg, "Wg", CODA_BF16, -1, -1));
  TRY(check_mat(Wu, "Wu", CODA_BF16, Wg->rows, Wg->cols));
  TRY(check_vec(g_or_null, "g", CODA_F32, Wg->rows, true));
  TRY(check_mat(Wgu_out, "Wgu_out", CODA_BF16, Wg->rows, 2 * Wg->cols));
  if (Wg->cols % 32 != 0) return fail(CODA_ERR_SHAPE, "pack_gate_up: F must be a multiple of 32");
  if (Wg->rows == 0 || Wg->cols == 0) return CODA_OK;
  hipLaunchKernelGGL(pack_gate_up_kernel, dim3((unsigned)((2 * Wg->cols / 4 + 255) / 256), (unsigned)Wg->rows),
                     dim3(256), 0, S(stream), static_cast<const uint16_t*>(Wg->ptr), Wg->ld,
                     static_cast<const uint16_t*>(Wu->ptr), Wu->ld, fptr(g_or_null),
                     static_cast<uint16_t*>(Wgu_out->ptr), Wgu_out->ld, (int)Wg->rows, (int)Wg->cols);
  return check_launch("pack_gate_up");
}

extern "C" coda_status coda_rope_table(int32_t seq_len, int32_t head_dim, double theta, const coda_mat* out,
                                       void* stream) {
  if (head_dim != 128) return fail(CODA_ERR_UNSUPPORTED, "rope_table: head_dim must be 128");
  if (seq_len <= 0 || !(theta > 1.0)) return fail(CODA_ERR_VALUE, "rope_table: bad seq_len or theta");
  TRY(check_mat(out, "rope", CODA_F32, seq_len, head_dim));
  if (out->ld != head_dim) return fail(CODA_ERR_LAYOUT, "rope_table: ld must equal head_dim");
  const int n = seq_len * head_dim / 2;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, S(stream), seq_len, head_dim, theta,
                     static_cast<float*>(out->ptr));
  return check_launch("rope_table");
}

// Partial rows a consumer GEMM's prologue reduces itself (they stay in
// registers through its mainloop).
constexpr int kProloguePartials = RowPartials<GemmCfg<kBM, kBN, 2, 4, true, false>>::MAX_PARTIALS;

// A wider set of row partials is first summed to one row, in a fixed order,
// by a small kernel (the light merge step of the paper, §3.1) into `tmp` [M].
static coda_status narrow_partials(const float** P, int* nP, int64_t M, float* tmp, hipStream_t s) {
  if (*nP <= kProloguePartials || M == 0) return CODA_OK;
  hipLaunchKernelGGL(rows_finish_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, *P, *nP, (int)M, 0,
                     (const float*)nullptr, 0, 0.0f, tmp);
  TRY(check_launch("merge row partials"));
  *P = tmp;
  *nP = 1;
  return CODA_OK;
}

static coda_status row_sumsq_launch(const void* x, int64_t ld, int64_t M, int64_t K, float* out, hipStream_t s) {
  if (M == 0) return CODA_OK;
  hipLaunchKernelGGL(row_sumsq_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), ld, (int)M, (int)K, out);
  return check_launch("row_sumsq");
}

extern "C" coda_status coda_row_sumsq(const coda_mat* x, const coda_mat* out, void* stream) {
  TRY(check_mat(x, "x", CODA_BF16, -1, -1));
  TRY(check_vec(out, "out", CODA_F32, x->rows));
  return row_sumsq_launch(x->ptr, x->ld, x->rows, x->cols, static_cast<float*>(out->ptr), S(stream));
}

extern "C" coda_status coda_quantize_e4m3_workspace(const coda_mat* X, int32_t axis, size_t* bytes) {
  if (!X || !bytes) return fail(CODA_ERR_NULL, "quantize_e4m3_workspace: NULL argument");
  if (axis != 0 && axis != 1) return fail(CODA_ERR_VALUE, "axis must be 0 or 1");
  Carver cv(nullptr);
  take_amax_ws(cv, X->rows, X->cols, axis);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_quantize_e4m3(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* scale,
                                          void* ws, size_t ws_bytes, void* stream) {
  TRY(check_mat(X, "X", CODA_BF16, -1, -1));
  if (axis != 0 && axis != 1) return fail(CODA_ERR_VALUE, "axis must be 0 or 1");
  const int64_t R = X->rows, C = X->cols;
  if (axis == 1) {
    TRY(check_mat(Q, "Q", CODA_E4M3, R, C));
    TRY(check_vec(scale, "scale", CODA_F32, R));
  } else {
    TRY(check_mat(Q, "Q", CODA_E4M3, C, R));
    TRY(check_vec(scale, "scale", CODA_F32, C));
  }
  Carver cv(ws);
  float* amax = nullptr;
  float* parts = nullptr;
  if (axis == 1) amax = cv.take<float>(R);
  else { amax = cv.take<float>(C); parts = cv.take<float>((size_t)((R + 255) / 256) * C); }
  TRY(ws_check(cv, ws_bytes, ws));
  return run_quant(X->ptr, X->ld, R, C, axis, static_cast<uint8_t*>(Q->ptr), Q->ld, static_cast<float*>(scale->ptr),
                   amax, parts, S(stream));
}

extern "C" coda_status coda_quantize_weight_workspace(const coda_weight* wt, size_t* bytes) {
  if (!wt || !bytes) return fail(CODA_ERR_NULL, "quantize_weight_workspace: NULL argument");
  Carver cv(nullptr);
  const int64_t K = wt->w.rows, N = wt->w.cols;
  cv.take<float>(std::max(K, N));
  cv.take<float>((size_t)((K + 255) / 256) * N);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_quantize_weight(const coda_weight* wt, void* ws, size_t ws_bytes, void* stream) {
  if (!wt) return fail(CODA_ERR_NULL, "quantize_weight: NULL weight");
  const int64_t K = wt->w.rows, N = wt->w.cols;
  if (wt->q_fwd.dtype == CODA_E2M3 || wt->q_fwd.dtype == CODA_E3M2) {
    // MXFP6 copies of the q_fwd dtype's format: q_fwd [N, K] with blocks
    // along K_in, the optional q_bwd [K, N] with blocks along N_out
    const bool e23 = wt->q_fwd.dtype == CODA_E2M3;
    TRY(check_weight(wt, "W", K, N, e23 ? CODA_PREC_MXFP6_E2M3 : CODA_PREC_MXFP6_E3M2));
    TRY(run_quant_mx6(wt->w.ptr, wt->w.ld, K, N, 0, static_cast<uint8_t*>(wt->q_fwd.ptr), wt->q_fwd.ld,
                      static_cast<uint8_t*>(wt->s_fwd.ptr), wt->s_fwd.ld, e23 ? 2 : 3, S(stream)));
    if (!present(&wt->q_bwd)) return CODA_OK;
    return run_quant_mx6(wt->w.ptr, wt->w.ld, K, N, 1, static_cast<uint8_t*>(wt->q_bwd.ptr), wt->q_bwd.ld,
                         static_cast<uint8_t*>(wt->s_bwd.ptr), wt->s_bwd.ld, e23 ? 2 : 3, S(stream));
  }
  if (wt->q_fwd.dtype == CODA_E2M1X2) {
    // MXFP4 forward copy: q_fwd [N, K / 2 bytes] with blocks along K_in
    TRY(check_weight(wt, "W", K, N, CODA_PREC_MXFP4));
    TRY(run_quant_mx4(wt->w.ptr, wt->w.ld, K, N, 0, static_cast<uint8_t*>(wt->q_fwd.ptr), wt->q_fwd.ld,
                      static_cast<uint8_t*>(wt->s_fwd.ptr), wt->s_fwd.ld, S(stream)));
    if (!present(&wt->q_bwd)) return CODA_OK;
    // input-gradient copy: q_bwd [K, N / 2 bytes] with blocks along N_out
    return run_quant_mx4(wt->w.ptr, wt->w.ld, K, N, 1, static_cast<uint8_t*>(wt->q_bwd.ptr), wt->q_bwd.ld,
                         static_cast<uint8_t*>(wt->s_bwd.ptr), wt->s_bwd.ld, S(stream));
  }
  if (wt->s_fwd.dtype == CODA_E8M0) {
    // MXFP8 copies: q_fwd [N, K] with blocks along K_in, q_bwd [K, N] with
    // blocks along N_out, exponents in word layout
    TRY(check_weight(wt, "W", K, N, CODA_PREC_MXFP8));
    TRY(run_quant_mx(wt->w.ptr, wt->w.ld, K, N, 0, static_cast<uint8_t*>(wt->q_fwd.ptr), wt->q_fwd.ld,
                     static_cast<uint8_t*>(wt->s_fwd.ptr), wt->s_fwd.ld, S(stream)));
    return run_quant_mx(wt->w.ptr, wt->w.ld, K, N, 1, static_cast<uint8_t*>(wt->q_bwd.ptr), wt->q_bwd.ld,
                        static_cast<uint8_t*>(wt->s_bwd.ptr), wt->s_bwd.ld, S(stream));
  }
  TRY(check_weight(wt, "W", K, N, CODA_PREC_FP8));
  Carver cv(ws);
  float* amax = cv.take<float>(std::max(K, N));
  float* parts = cv.take<float>((size_t)((K + 255) / 256) * N);
  TRY(ws_check(cv, ws_bytes, ws));
  // forward copy: contracted axis K_in -> one scale per output channel, Q^T [N, K]
  TRY(run_quant(wt->w.ptr, wt->w.ld, K, N, 0, static_cast<uint8_t*>(wt->q_fwd.ptr), wt->q_fwd.ld,
                static_cast<float*>(wt->s_fwd.ptr), amax, parts, S(stream)));
  // input-gradient copy: contracted axis N_out -> one scale per input channel, Q [K, N]
  return run_quant(wt->w.ptr, wt->w.ld, K, N, 1, static_cast<uint8_t*>(wt->q_bwd.ptr), wt->q_bwd.ld,
                   static_cast<float*>(wt->s_bwd.ptr), amax, parts, S(stream));
}

// ======================================================================== generic
namespace {
// The compiled epilogue chains of the generic entry point.  A program is
// first matched against these opcode patterns (an element may have an
// alternative opcode and may be optional); the matched ops then bind their
// aux operands, each checked, into the epilogue arguments of that chain.
enum : uint16_t {
  OP_STORE = CODA_EPI_STORE_BF16, OP_ACCUM = CODA_EPI_ACCUM_F32, OP_ROW = CODA_EPI_ROW_SCALE,
  OP_COL = CODA_EPI_COL_SCALE, OP_ADD = CODA_EPI_ADD_TILE, OP_SUMSQ = CODA_EPI_ROW_SUMSQ_PARTIAL,
  OP_SWIGLU = CODA_EPI_SWIGLU, OP_RMS = CODA_EPI_ROW_RMS_FROM_PARTIALS, OP_ROWOUT = CODA_EPI_STORE_ROW_VEC,
  OP_SAVE = CODA_EPI_SAVE_PRE, OP_QKROPE = CODA_EPI_QKNORM_ROPE, OP_DSWIGLU = CODA_EPI_DSWIGLU,
  OP_DOT = CODA_EPI_ROW_DOT_PARTIAL, OP_NORMCORR = CODA_EPI_NORM_CORRECTION, OP_WGRAD = CODA_EPI_WGRAD_GAIN,
  OP_CELSE = CODA_EPI_CE_LSE_PARTIAL, OP_CEGRAD = CODA_EPI_CE_GRAD, OP_SIGMOID = CODA_EPI_SIGMOID,
  OP_DSIGMOID = CODA_EPI_DSIGMOID, OP_SDEV = CODA_EPI_SCALE_DEV, OP_DEQUANT = CODA_EPI_DEQUANT_E4M3,
  OP_GELU = CODA_EPI_GELU, OP_DGELU = CODA_EPI_DGELU,
};

struct PatEl { uint16_t op, alt; bool opt; };
struct ChainDef {
  Prog prog;
  int n;
  PatEl el[6];
};
constexpr PatEl R(uint16_t o, uint16_t a = 0) { return PatEl{o, a, false}; }
constexpr PatEl O(uint16_t o) { return PatEl{o, 0, true}; }

// Chains whose prologue or map differ get their own entries, in the order
// they are tried; a chain matches when every op is consumed in order.
const ChainDef kChains[] = {
    {Prog::Store, 1, {R(OP_STORE)}},
    {Prog::StoreF32, 1, {R(OP_ACCUM)}},
    {Prog::RowColStore, 3, {R(OP_ROW), R(OP_COL), R(OP_STORE)}},
    {Prog::ResidSumsq, 3, {R(OP_ADD), R(OP_STORE), R(OP_SUMSQ)}},
    {Prog::Resid, 2, {R(OP_ADD), R(OP_STORE)}},
    {Prog::SwiGLU, 5, {R(OP_ROW, OP_RMS), O(OP_ROWOUT), O(OP_SAVE), R(OP_SWIGLU), R(OP_STORE)}},
    {Prog::Sigmoid, 5, {R(OP_ROW, OP_RMS), O(OP_ROWOUT), O(OP_SAVE), R(OP_SIGMOID), R(OP_STORE)}},
    {Prog::Gelu, 5, {R(OP_ROW, OP_RMS), O(OP_ROWOUT), O(OP_SAVE), R(OP_GELU), R(OP_STORE)}},
    {Prog::QKRope, 5, {R(OP_ROW, OP_RMS), O(OP_ROWOUT), O(OP_SAVE), R(OP_QKROPE), R(OP_STORE)}},
    {Prog::DSwiGLU, 4, {R(OP_DSWIGLU), R(OP_ROW), R(OP_STORE), R(OP_DOT)}},
    {Prog::DSigmoid, 4, {R(OP_DSIGMOID), R(OP_ROW), R(OP_STORE), R(OP_DOT)}},
    {Prog::DGelu, 4, {R(OP_DGELU), R(OP_ROW), R(OP_STORE), R(OP_DOT)}},
    {Prog::NormCorr, 4, {R(OP_NORMCORR), O(OP_SDEV), O(OP_ADD), R(OP_STORE)}},
    {Prog::WgradGain, 2, {O(OP_SDEV), R(OP_WGRAD)}},
    {Prog::CrossEntropyNorm, 3, {R(OP_RMS), O(OP_ROWOUT), R(OP_CELSE)}},
    {Prog::CrossEntropy, 1, {R(OP_CELSE)}},
    {Prog::CrossEntropyG, 2, {R(OP_CEGRAD), R(OP_STORE)}},
    {Prog::CrossEntropyGNorm, 4, {R(OP_ROW), R(OP_CEGRAD), R(OP_STORE), R(OP_DOT)}},
    {Prog::StoreAlphaDev, 2, {R(OP_SDEV), R(OP_STORE)}},
    {Prog::F32AlphaDev, 2, {R(OP_SDEV), R(OP_ACCUM)}},
};

// Matches ops[0..n) against a chain; at[i] is the op of pattern element i or null.
bool match_chain(const ChainDef& c, const coda_epi_op* ops, uint32_t n, const coda_epi_op** at) {
  uint32_t k = 0;
  for (int i = 0; i < c.n; ++i) {
    const PatEl& p = c.el[i];
    if (k < n && (ops[k].op == p.op || (p.alt && ops[k].op == p.alt))) {
      at[i] = &ops[k++];
    } else if (p.opt) {
      at[i] = nullptr;
    } else {
      return false;
    }
  }
  return k == n;
}

// Splits off a leading DEQUANT_E4M3 and finds the compiled chain.
coda_status find_chain(const coda_epi_program* prog, const char* who, const ChainDef** chain,
                       const coda_epi_op** at, const coda_epi_op** dequant) {
  if (!prog) return fail(CODA_ERR_NULL, "%s: NULL program", who);
  if (prog->n_ops == 0 || prog->n_ops > CODA_MAX_EPI_OPS)
    return fail(CODA_ERR_UNSUPPORTED, "%s: empty or too long program", who);
  const coda_epi_op* ops = prog->ops;
  uint32_t n = prog->n_ops;
  *dequant = nullptr;
  if (ops[0].op == OP_DEQUANT) {
    *dequant = &ops[0];
    ++ops;
    --n;
  }
  for (const ChainDef& c : kChains)
    if (match_chain(c, ops, n, at)) {
      *chain = &c;
      return CODA_OK;
    }
  char buf[96];
  int o = 0;
  for (uint32_t i = 0; i < prog->n_ops && o < 80; ++i) o += snprintf(buf + o, sizeof(buf) - o, " %u", prog->ops[i].op);
  return fail(CODA_ERR_UNSUPPORTED, "%s: epilogue program (opcodes%s) not in the compiled set", who, o ? buf : "");
}

bool has_partial_merge(const ChainDef& c, const coda_epi_op* const* at) {
  for (int i = 0; i < c.n; ++i)
    if (at[i] && (at[i]->op == OP_RMS || at[i]->op == OP_NORMCORR)) return true;
  return false;
}

// What a decoded program launches: the chain, its arguments, D's shape and type.
struct Decoded {
  Prog p;
  EpiArgs e;
  int64_t out_cols;
  int out_dtype;            // CODA_BF16, CODA_F32, or 0: D unused
  bool e4m3;
  const float* merge_src;   // partial rows to merge to one before the GEMM (n > 8)
  int merge_n;
  const float** merge_dst;  // where the merged row goes (e.row_partials)
};

constexpr int kMaxPartialRows = 32;

// Decodes and checks a program for the product C [M, N] with contracted
// size K into `d`.  `mx`: the operands carry block exponents (coda_gemm_mx).
coda_status decode_program(const coda_epi_program* prog, int64_t M, int64_t N, int64_t K, const coda_mat* aux,
                           uint32_t n_aux, const char* who, bool mx, Decoded* d) {
  const ChainDef* c;
  const coda_epi_op* at[6];
  const coda_epi_op* dq;
  TRY(find_chain(prog, who, &c, at, &dq));
  if (dq && mx) return fail(CODA_ERR_UNSUPPORTED, "%s: DEQUANT_E4M3 does not apply to block-scaled operands", who);
  EpiArgs& e = d->e;
  e = epi0();
  d->p = c->prog;
  d->out_cols = N;
  d->out_dtype = CODA_BF16;
  d->e4m3 = dq != nullptr;
  d->merge_src = nullptr;
  d->merge_n = 0;
  d->merge_dst = nullptr;
  const int64_t tn = coda_partials_cols(N);
  // operand of `slot` (slot index into aux), checked
  auto A_ = [&](uint16_t slot) -> const coda_mat* { return (aux && slot < n_aux) ? &aux[slot] : nullptr; };
  auto vec = [&](uint16_t slot, const char* name, int dt, int64_t n, const coda_mat** out) -> coda_status {
    TRY(check_vec(A_(slot), name, dt, n));
    *out = A_(slot);
    return CODA_OK;
  };
  auto tile = [&](uint16_t slot, const char* name, int dt, int64_t rows, int64_t cols,
                  const coda_mat** out) -> coda_status {
    TRY(check_mat(A_(slot), name, dt, rows, cols));
    *out = A_(slot);
    return CODA_OK;
  };
  // fp32 partials [rows, M] (rows < 0: 1..kMaxPartialRows), ld == M
  auto partials = [&](uint16_t slot, const char* name, int64_t rows, const coda_mat** out) -> coda_status {
    const coda_mat* P = A_(slot);
    TRY(check_mat(P, name, CODA_F32, rows, M));
    if (rows < 0 && (P->rows < 1 || P->rows > kMaxPartialRows))
      return fail(CODA_ERR_SHAPE, "%s: %s must have 1..%d rows", who, name, kMaxPartialRows);
    if (P->rows > 1 && P->ld != M) return fail(CODA_ERR_LAYOUT, "%s: %s ld must be M", who, name);
    *out = P;
    return CODA_OK;
  };
  const coda_mat* m;
  const coda_mat* m2;
  const coda_mat* m3;
  // the row factor of a pre-norm chain: given (ROW_SCALE) or finished from partials
  auto row_factor = [&](const coda_epi_op* op) -> coda_status {
    if (op->op == OP_ROW) {
      TRY(vec(op->slot, "row scale", CODA_F32, M, &m));
      e.rowvec = fptr(m);
    } else {
      TRY(partials(op->slot, "row partials", -1, &m));
      if (!(op->fparam >= 0.0f)) return fail(CODA_ERR_VALUE, "%s: eps must be >= 0", who);
      e.row_partials = fptr(m);
      e.n_row_partials = (int)m->rows;
      e.norm_dim = (int)K;
      e.eps = op->fparam;
      if (m->rows > kProloguePartials) {
        d->merge_src = fptr(m);
        d->merge_n = (int)m->rows;
        d->merge_dst = &e.row_partials;
      }
    }
    return CODA_OK;
  };
  auto row_out = [&](const coda_epi_op* op, float** dst) -> coda_status {
    if (!op) return CODA_OK;
    TRY(vec(op->slot, "row vector output", CODA_F32, M, &m));
    *dst = static_cast<float*>(m->ptr);
    return CODA_OK;
  };
  auto save = [&](const coda_epi_op* op, int64_t cols) -> coda_status {
    if (!op) return CODA_OK;
    TRY(tile(op->slot, "save", CODA_BF16, M, cols, &m));
    e.save = m->ptr;
    e.ld_save = m->ld;
    return CODA_OK;
  };
  auto dev_scale = [&](const coda_epi_op* op) -> coda_status {
    if (!op) return CODA_OK;
    TRY(vec(op->slot, "device scale", CODA_F32, 1, &m));
    e.alpha_dev = fptr(m);
    return CODA_OK;
  };
  switch (c->prog) {
    case Prog::Store: break;
    case Prog::StoreF32:
      e.beta = at[0]->fparam;
      d->out_dtype = CODA_F32;
      break;
    case Prog::RowColStore:
      TRY(vec(at[0]->slot, "row scale", CODA_F32, M, &m));
      TRY(vec(at[1]->slot, "col scale", CODA_F32, N, &m2));
      e.rowvec = fptr(m);
      e.colvec = fptr(m2);
      break;
    case Prog::ResidSumsq:
      TRY(partials(at[2]->slot, "sumsq partials", tn, &m2));
      e.partial_out = static_cast<float*>(m2->ptr);
      [[fallthrough]];
    case Prog::Resid:
      TRY(tile(at[0]->slot, "tile", CODA_BF16, M, N, &m));
      e.aux0 = m->ptr;
      e.ld_aux0 = m->ld;
      break;
    case Prog::SwiGLU:
    case Prog::Sigmoid:
    case Prog::Gelu:
    case Prog::QKRope: {
      TRY(row_factor(at[0]));
      TRY(row_out(at[1], &e.rowvec_out));
      if (c->prog == Prog::SwiGLU) {
        if (N % 64 != 0) return fail(CODA_ERR_SHAPE, "%s: SWIGLU needs N %% 64 == 0 (packed gate/up)", who);
        d->out_cols = N / 2;
        TRY(save(at[2], N));
      } else if (c->prog == Prog::Sigmoid || c->prog == Prog::Gelu) {
        TRY(save(at[2], N));
      } else {
        if (N % 384 != 0) return fail(CODA_ERR_SHAPE, "%s: QKNORM_ROPE needs N = 3 x a multiple of 128", who);
        const coda_epi_op* q = at[3];
        TRY(tile(q->slot, "qk gains", CODA_F32, 2, 128, &m));
        TRY(check_mat(A_(q->slot2), "rope table", CODA_F32, -1, 128));
        m2 = A_(q->slot2);
        if (m2->rows < 1) return fail(CODA_ERR_SHAPE, "%s: empty RoPE table", who);
        if (m2->rows > 1 && m2->ld != 128) return fail(CODA_ERR_LAYOUT, "%s: RoPE table ld must be 128", who);
        if (!(q->fparam >= 0.0f)) return fail(CODA_ERR_VALUE, "%s: eps must be >= 0", who);
        if (at[0]->op == OP_RMS && at[0]->fparam != q->fparam)
          return fail(CODA_ERR_VALUE, "%s: the row norm and the QK-norm take one eps", who);
        e.eps = q->fparam;
        e.colvec = fptr(m);
        e.colvec2 = fptr(m) + (m->rows > 1 ? m->ld : 128);
        e.table = fptr(m2);
        e.seq_len = (int)m2->rows;
        e.region = (int)(N / 3);
        TRY(save(at[2], 2 * N / 3));
      }
      break;
    }
    case Prog::DSwiGLU:
    case Prog::DSigmoid:
    case Prog::DGelu: {
      const bool sw = c->prog == Prog::DSwiGLU;
      if (sw && N % 32 != 0) return fail(CODA_ERR_SHAPE, "%s: DSWIGLU needs N %% 32 == 0", who);
      TRY(tile(at[0]->slot, "saved pre-activation", CODA_BF16, M, sw ? 2 * N : N, &m));
      e.aux0 = m->ptr;
      e.ld_aux0 = m->ld;
      TRY(vec(at[1]->slot, "row scale", CODA_F32, M, &m2));
      e.rowvec = fptr(m2);
      TRY(partials(at[3]->slot, "dot partials", tn, &m3));
      e.partial_out = static_cast<float*>(m3->ptr);
      if (sw) d->out_cols = 2 * N;
      break;
    }
    case Prog::NormCorr: {
      const coda_epi_op* q = at[0];
      TRY(tile(q->slot, "u", CODA_BF16, M, N, &m));
      TRY(vec(q->slot2, "r", CODA_F32, M, &m2));
      TRY(partials(q->slot3, "T partials", -1, &m3));
      e.aux0 = m->ptr;
      e.ld_aux0 = m->ld;
      e.rowvec = fptr(m2);
      e.row_partials = fptr(m3);
      e.n_row_partials = (int)m3->rows;
      e.norm_dim = (int)N;
      if (m3->rows > kProloguePartials) {
        d->merge_src = fptr(m3);
        d->merge_n = (int)m3->rows;
        d->merge_dst = &e.row_partials;
      }
      TRY(dev_scale(at[1]));
      if (at[2]) {
        TRY(tile(at[2]->slot, "tile", CODA_BF16, M, N, &m));
        e.aux1 = m->ptr;
        e.ld_aux1 = m->ld;
      }
      break;
    }
    case Prog::WgradGain: {
      TRY(dev_scale(at[0]));
      const coda_epi_op* q = at[1];
      TRY(tile(q->slot, "W", CODA_BF16, M, N, &m));
      TRY(vec(q->slot2, "g", CODA_F32, M, &m2));
      TRY(partials(q->slot3, "gain partials", tn, &m3));
      e.aux0 = m->ptr;
      e.ld_aux0 = m->ld;
      e.rowvec = fptr(m2);
      e.partial_out = static_cast<float*>(m3->ptr);
      e.beta = q->fparam;
      d->out_dtype = CODA_F32;
      break;
    }
    case Prog::CrossEntropyNorm:
    case Prog::CrossEntropy: {
      const bool norm = c->prog == Prog::CrossEntropyNorm;
      if (norm) {
        TRY(row_factor(at[0]));
        TRY(row_out(at[1], &e.rowvec_out2));
      }
      const coda_epi_op* q = at[norm ? 2 : 0];
      TRY(vec(q->slot, "labels", CODA_I32, M, &m));
      TRY(partials(q->slot2, "lse partials", 2 * tn, &m2));
      TRY(vec(q->slot3, "label logit", CODA_F32, M, &m3));
      e.labels = static_cast<const int*>(m->ptr);
      e.partial_out = static_cast<float*>(m2->ptr);
      e.partial_out2 = static_cast<float*>(m2->ptr) + tn * M;
      e.rowvec_out = static_cast<float*>(m3->ptr);
      e.vocab = (int)N;
      d->out_dtype = 0;
      break;
    }
    case Prog::CrossEntropyG:
    case Prog::CrossEntropyGNorm: {
      const bool norm = c->prog == Prog::CrossEntropyGNorm;
      const coda_epi_op* q = at[norm ? 1 : 0];
      TRY(vec(q->slot, "labels", CODA_I32, M, &m));
      TRY(vec(q->slot2, "lse", CODA_F32, M, &m2));
      e.labels = static_cast<const int*>(m->ptr);
      e.rowvec = fptr(m2);
      e.vocab = (int)N;
      e.col_offset = 0;
      if (norm) {
        TRY(vec(at[0]->slot, "row scale", CODA_F32, M, &m3));
        e.rowvec2 = fptr(m3);
        TRY(partials(at[3]->slot, "dot partials", tn, &m));
        e.partial_out = static_cast<float*>(m->ptr);
      }
      break;
    }
    case Prog::StoreAlphaDev:
      TRY(dev_scale(at[0]));
      break;
    case Prog::F32AlphaDev:
      TRY(dev_scale(at[0]));
      e.beta = at[1]->fparam;
      d->out_dtype = CODA_F32;
      break;
  }
  if (dq) {
    TRY(vec(dq->slot, "row dequantisation scales", CODA_F32, M, &m));
    TRY(vec(dq->slot2, "column dequantisation scales", CODA_F32, N, &m2));
    e.rowscale = fptr(m);
    e.colscale = fptr(m2);
  }
  return CODA_OK;
}

size_t epi_ws_bytes(int64_t M) {
  Carver cv(nullptr);
  cv.take<float>((size_t)M);
  return cv.off;
}

// Checks D, carves the workspace, merges wide partials and launches.
// elem: the MX element format of the operands as the scaled MFMA codes it
// (2 = E2M3, 3 = E3M2, 4 = E2M1), 0 for bf16 / E4M3 ones.
coda_status run_decoded(Decoded& d, int64_t M, const coda_mat* D, GemmArgs g, int layout, bool fp8, int elem,
                        void* ws, size_t ws_bytes, hipStream_t s, const char* who) {
  if (d.out_dtype != 0) {
    TRY(check_mat(D, "D", d.out_dtype, M, d.out_cols));
    d.e.out = D->ptr;
    d.e.ld_out = D->ld;
    if (d.p == Prog::QKRope) {   // q | k | v are the three column thirds of D
      const int64_t w = d.out_cols / 3;
      d.e.out2 = static_cast<uint16_t*>(D->ptr) + w;
      d.e.out3 = static_cast<uint16_t*>(D->ptr) + 2 * w;
      d.e.ld_out2 = d.e.ld_out3 = D->ld;
    }
  }
  Carver cv(ws);
  float* tmp = d.merge_src ? cv.take<float>((size_t)M) : nullptr;
  TRY(ws_check(cv, ws_bytes, ws));
  if (d.merge_src) {
    const float* P = d.merge_src;
    int nP = d.merge_n;
    TRY(narrow_partials(&P, &nP, M, tmp, s));
    *d.merge_dst = P;
    d.e.n_row_partials = nP;
  }
  hipError_t err = elem == 4   ? launch_gemm_mx4(d.p, g, d.e, s)
                   : elem != 0 ? launch_gemm_mx6(d.p, elem, g, d.e, s)
                               : launch_gemm(d.p, layout, fp8, g, d.e, s);
  if (err == hipErrorInvalidValue)
    return fail(CODA_ERR_UNSUPPORTED, "%s: this epilogue chain is not compiled for these operands", who);
  return launched(err, who);
}

}  // namespace

extern "C" coda_status coda_gemm_epi_workspace(const coda_epi_program* prog, int64_t M, int64_t N, int64_t K,
                                               size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "gemm_epi_workspace: NULL bytes");
  (void)N;
  (void)K;
  const ChainDef* c;
  const coda_epi_op* at[6];
  const coda_epi_op* dq;
  TRY(find_chain(prog, "gemm_epi_workspace", &c, at, &dq));
  *bytes = (has_partial_merge(*c, at) && M > 0) ? epi_ws_bytes(M) : 0;
  return CODA_OK;
}

extern "C" coda_status coda_gemm_epi(const coda_epi_program* prog, const coda_mat* A, int32_t transA,
                                     const coda_mat* B, int32_t transB, const coda_mat* D, const coda_mat* aux,
                                     uint32_t n_aux, void* ws, size_t ws_bytes, void* stream) {
  if (!prog) return fail(CODA_ERR_NULL, "gemm_epi: NULL program");
  const bool e4m3 = prog->n_ops > 0 && prog->n_ops <= CODA_MAX_EPI_OPS && prog->ops[0].op == OP_DEQUANT;
  const int odt = e4m3 ? CODA_E4M3 : CODA_BF16;
  TRY(check_mat(A, "A", odt, -1, -1));
  TRY(check_mat(B, "B", odt, -1, -1));
  if (e4m3 && (transA != 0 || transB != 1))
    return fail(CODA_ERR_LAYOUT, "gemm_epi: E4M3 operands are A [M, K] and B [N, K] (transA 0, transB 1)");
  const int64_t M = transA ? A->cols : A->rows, K = transA ? A->rows : A->cols;
  const int64_t Kb = transB ? B->cols : B->rows, N = transB ? B->rows : B->cols;
  if (K != Kb) return fail(CODA_ERR_SHAPE, "gemm_epi: inner sizes %lld and %lld differ", (long long)K, (long long)Kb);
  const int layout = (transA ? 2 : 0) + (transB ? 1 : 0);
  Decoded d;
  TRY(decode_program(prog, M, N, K, aux, n_aux, "gemm_epi", false, &d));
  GemmArgs g = gemm_args(A->ptr, A->ld, B->ptr, B->ld, M, N, K);
  return run_decoded(d, M, D, g, layout, e4m3, 0, ws, ws_bytes, S(stream), "gemm_epi");
}

// ======================================================================== MXFP8
extern "C" coda_status coda_quantize_mxfp8(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* Sc,
                                           void* stream) {
  TRY(check_mat(X, "X", CODA_BF16, -1, -1));
  if (axis != 0 && axis != 1) return fail(CODA_ERR_VALUE, "axis must be 0 or 1");
  const int64_t R = X->rows, C = X->cols;
  const int64_t L = axis == 1 ? C : R;     // length of the blocked (contracted) axis
  if (L % 32 != 0) return fail(CODA_ERR_SHAPE, "quantize_mxfp8: the blocked axis (%lld) must be a multiple of 32",
                               (long long)L);
  const int64_t rows = axis == 1 ? R : C;
  TRY(check_mat(Q, "Q", CODA_E4M3, rows, L));
  TRY(check_scales(Sc, "S", rows, L));
  if (R == 0 || C == 0) return CODA_OK;
  const uint16_t* x = static_cast<const uint16_t*>(X->ptr);
  uint8_t* q = static_cast<uint8_t*>(Q->ptr);
  uint8_t* sc = static_cast<uint8_t*>(Sc->ptr);
  if (axis == 1)
    hipLaunchKernelGGL(quant_mx_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, S(stream), x, X->ld,
                       (int)R, (int)C, q, Q->ld, sc, Sc->ld);
  else
    hipLaunchKernelGGL(quant_mx_cols_t_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)), dim3(256),
                       0, S(stream), x, X->ld, (int)R, (int)C, q, Q->ld, sc, Sc->ld);
  return check_launch("quantize_mxfp8");
}

extern "C" coda_status coda_quantize_mxfp4(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* Sc,
                                           void* stream) {
  TRY(check_mat(X, "X", CODA_BF16, -1, -1));
  if (axis != 0 && axis != 1) return fail(CODA_ERR_VALUE, "axis must be 0 or 1");
  const int64_t R = X->rows, C = X->cols;
  const int64_t L = axis == 1 ? C : R;     // length of the blocked (contracted) axis
  if (L % 32 != 0) return fail(CODA_ERR_SHAPE, "quantize_mxfp4: the blocked axis (%lld) must be a multiple of 32",
                               (long long)L);
  const int64_t rows = axis == 1 ? R : C;
  TRY(check_mat(Q, "Q", CODA_E2M1X2, rows, L / 2));
  TRY(check_scales(Sc, "S", rows, L));
  if (R == 0 || C == 0) return CODA_OK;
  const uint16_t* x = static_cast<const uint16_t*>(X->ptr);
  uint8_t* q = static_cast<uint8_t*>(Q->ptr);
  uint8_t* sc = static_cast<uint8_t*>(Sc->ptr);
  if (axis == 1)
    hipLaunchKernelGGL(quant_mx4_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, S(stream), x, X->ld,
                       (int)R, (int)C, q, Q->ld, sc, Sc->ld);
  else
    hipLaunchKernelGGL(quant_mx4_cols_t_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)),
                       dim3(256), 0, S(stream), x, X->ld, (int)R, (int)C, q, Q->ld, sc, Sc->ld);
  return check_launch("quantize_mxfp4");
}

extern "C" coda_status coda_quantize_mxfp6(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* Sc,
                                           void* stream) {
  TRY(check_mat(X, "X", CODA_BF16, -1, -1));
  if (axis != 0 && axis != 1) return fail(CODA_ERR_VALUE, "axis must be 0 or 1");
  if (!Q) return fail(CODA_ERR_NULL, "Q: NULL");
  if (Q->dtype != CODA_E2M3 && Q->dtype != CODA_E3M2)
    return fail(CODA_ERR_DTYPE, "quantize_mxfp6: Q must be CODA_E2M3 or CODA_E3M2 (got %d)", (int)Q->dtype);
  const int f6 = Q->dtype == CODA_E2M3 ? 2 : 3;
  const int64_t R = X->rows, C = X->cols;
  const int64_t L = axis == 1 ? C : R;     // length of the blocked (contracted) axis
  if (L % 32 != 0) return fail(CODA_ERR_SHAPE, "quantize_mxfp6: the blocked axis (%lld) must be a multiple of 32",
                               (long long)L);
  const int64_t rows = axis == 1 ? R : C;
  TRY(check_mat(Q, "Q", Q->dtype, rows, L));
  TRY(check_scales(Sc, "S", rows, L));
  if (R == 0 || C == 0) return CODA_OK;
  const uint16_t* x = static_cast<const uint16_t*>(X->ptr);
  uint8_t* q = static_cast<uint8_t*>(Q->ptr);
  uint8_t* sc = static_cast<uint8_t*>(Sc->ptr);
  if (axis == 1)
    hipLaunchKernelGGL(quant_mx6_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, S(stream), x, X->ld,
                       (int)R, (int)C, q, Q->ld, sc, Sc->ld, f6);
  else
    hipLaunchKernelGGL(quant_mx6_cols_t_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)),
                       dim3(256), 0, S(stream), x, X->ld, (int)R, (int)C, q, Q->ld, sc, Sc->ld, f6);
  return check_launch("quantize_mxfp6");
}

extern "C" coda_status coda_gemm_mx(const coda_epi_program* prog, const coda_mat* A, const coda_mat* SA,
                                    const coda_mat* B, const coda_mat* SB, const coda_mat* D, const coda_mat* aux,
                                    uint32_t n_aux, void* ws, size_t ws_bytes, void* stream) {
  if (!prog) return fail(CODA_ERR_NULL, "gemm_mx: NULL program");
  // E2M1 operands (two values a byte) or FP6 ones (E2M3 / E3M2, a byte a
  // value with the block padding) when A says so; B must match
  const int odt = present(A) && (A->dtype == CODA_E2M1X2 || A->dtype == CODA_E2M3 || A->dtype == CODA_E3M2)
                      ? A->dtype : CODA_E4M3;
  const bool fp4 = odt == CODA_E2M1X2;
  const int elem = odt == CODA_E2M1X2 ? 4 : odt == CODA_E2M3 ? 2 : odt == CODA_E3M2 ? 3 : 0;
  TRY(check_mat(A, "A", odt, -1, -1));
  TRY(check_mat(B, "B", odt, -1, -1));
  const int64_t M = A->rows, Kb = A->cols, N = B->rows;
  const int64_t K = fp4 ? 2 * Kb : Kb;     // contracted length in values
  if (B->cols != Kb) return fail(CODA_ERR_SHAPE, "gemm_mx: inner sizes %lld and %lld differ", (long long)Kb,
                                 (long long)B->cols);
  if (K <= 0 || K % 128 != 0) return fail(CODA_ERR_SHAPE, "gemm_mx: K (%lld) must be a positive multiple of 128",
                                          (long long)K);
  TRY(check_scales(SA, "SA", M, K));
  TRY(check_scales(SB, "SB", N, K));
  Decoded d;
  TRY(decode_program(prog, M, N, K, aux, n_aux, "gemm_mx", true, &d));
  GemmArgs g = gemm_args(A->ptr, A->ld, B->ptr, B->ld, M, N, Kb);   // the mainloop counts bytes
  g.sA = SA->ptr;
  g.sB = SB->ptr;
  g.lds_a = SA->rows > 1 ? SA->ld : SA->cols;
  g.lds_b = SB->rows > 1 ? SB->ld : SB->cols;
  return run_decoded(d, M, D, g, LAYOUT_NT, true, elem, ws, ws_bytes, S(stream), "gemm_mx");
}

// ======================================================================== functional forward
extern "C" coda_status coda_linear_swiglu_fwd_workspace(int64_t M, int64_t K, int32_t have_partials,
                                                        int32_t precision, size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  Carver cv(nullptr);
  (void)have_partials;
  cv.take<float>(M);   // row sum of squares, or the merged partials
  if (precision != CODA_PREC_BF16) take_act(cv, M, K, 1, is_mx(precision), prec_elem(precision));
  *bytes = cv.off;
  return CODA_OK;
}

namespace {
// Sizes and carves what an fp8 activation operand of the forward needs.
size_t fwd_fp8_bytes(int64_t M, int64_t K, bool mx, int elem) {
  Carver cv(nullptr);
  take_act(cv, M, K, 1, mx, elem);
  return cv.off;
}
}  // namespace

// The pre-norm activation layers: SwiGLU over packed gate/up columns, or an
// elementwise sigmoid or GELU.
enum class Act { SwiGLU, Sigmoid, Gelu };

static coda_status swiglu_fwd_impl(const coda_mat* x, const coda_mat* P, const coda_weight* Wgu, float eps,
                                   const coda_mat* out, const coda_mat* save, const coda_mat* r_out, int precision,
                                   void* ws, size_t ws_bytes, void* stream, bool size_only, size_t* bytes,
                                   Act act = Act::SwiGLU) {
  const int64_t M = x->rows, K = x->cols, N = Wgu->w.cols, F = N / 2;
  Carver cv(size_only ? nullptr : ws);
  float* sumsq = cv.take<float>(M);
  ActQ aq{};
  if (precision != CODA_PREC_BF16) aq = take_act(cv, M, K, 1, is_mx(precision), prec_elem(precision));
  if (size_only) { *bytes = cv.off; return CODA_OK; }
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  if (!present(P)) TRY(row_sumsq_launch(x->ptr, x->ld, M, K, sumsq, s));
  EpiArgs e = epi0();
  e.out = out->ptr; e.ld_out = out->ld;
  if (present(save)) { e.save = save->ptr; e.ld_save = save->ld; }
  e.row_partials = present(P) ? fptr(P) : sumsq;
  e.n_row_partials = present(P) ? (int)P->rows : 1;
  TRY(narrow_partials(&e.row_partials, &e.n_row_partials, M, sumsq, s));
  e.norm_dim = (int)K;
  e.eps = eps;
  e.rowvec_out = present(r_out) ? static_cast<float*>(r_out->ptr) : nullptr;
  GemmArgs g;
  int layout;
  const bool fp8 = precision != CODA_PREC_BF16;
  if (fp8) {
    TRY(quant_act(aq, x->ptr, x->ld, M, K, 1, s));
    g = gemm_args(aq.q.q, aq.q.ld, Wgu->q_fwd.ptr, Wgu->q_fwd.ld, M, N, aq.elem == 4 ? K / 2 : K);
    e.rowscale = aq.q.s;
    e.colscale = fptr(&Wgu->s_fwd);
    if (aq.mx) mx_args(&g, &e, aq.e, aq.e_ld, &Wgu->s_fwd);
    layout = LAYOUT_NT;
  } else {
    g = gemm_args(x->ptr, x->ld, Wgu->w.ptr, Wgu->w.ld, M, N, K);
    layout = LAYOUT_NN;
  }
  (void)F;
  if (act == Act::Sigmoid)
    return launched(launch_fwd(Prog::Sigmoid, layout, fp8, aq.elem, g, e, s), "linear_sigmoid_fwd");
  if (act == Act::Gelu) return launched(launch_fwd(Prog::Gelu, layout, fp8, aq.elem, g, e, s), "linear_gelu_fwd");
  return launched(launch_fwd(Prog::SwiGLU, layout, fp8, aq.elem, g, e, s), "linear_swiglu_fwd");
}

static coda_status swiglu_fwd_check(const coda_mat* x, const coda_mat* P, const coda_weight* Wgu, const coda_mat* out,
                                    const coda_mat* save, const coda_mat* r_out, int precision) {
  TRY(check_precision_fwd(precision));
  TRY(check_mat(x, "x", CODA_BF16, -1, -1));
  const int64_t M = x->rows, K = x->cols;
  if (K == 0) return fail(CODA_ERR_SHAPE, "x: the normalised rows are empty (K = 0)");
  if (!Wgu) return fail(CODA_ERR_NULL, "Wgu: NULL");
  const int64_t N = Wgu->w.cols;
  TRY(check_weight(Wgu, "Wgu", K, N, precision));
  if (N % 64 != 0) return fail(CODA_ERR_SHAPE, "Wgu: 2F must be a multiple of 64");
  TRY(check_mat(P, "sumsq_partials", CODA_F32, -1, M, true));
  if (present(P) && (P->rows < 1 || P->rows > 32 || (P->rows > 1 && P->ld != M)))
    return fail(CODA_ERR_SHAPE, "sumsq_partials: 1..32 rows of M with ld == M");
  TRY(check_mat(out, "out", CODA_BF16, M, N / 2));
  TRY(check_mat(save, "save_hgu", CODA_BF16, M, N, true));
  TRY(check_vec(r_out, "r_out", CODA_F32, M, true));
  return CODA_OK;
}

extern "C" coda_status coda_linear_swiglu_fwd(const coda_mat* x, const coda_mat* sumsq_partials, const coda_weight* Wgu,
                                              float eps, const coda_mat* out, const coda_mat* save_hgu,
                                              const coda_mat* r_out, int32_t precision, void* ws, size_t ws_bytes,
                                              void* stream) {
  TRY(swiglu_fwd_check(x, sumsq_partials, Wgu, out, save_hgu, r_out, precision));
  if (!(eps >= 0.0f)) return fail(CODA_ERR_VALUE, "eps must be >= 0");
  return swiglu_fwd_impl(x, sumsq_partials, Wgu, eps, out, save_hgu, r_out, precision, ws, ws_bytes, stream, false,
                         nullptr);
}

extern "C" coda_status coda_linear_rmsnorm_residual_fwd_workspace(int64_t M, int64_t K, int64_t N, int32_t precision,
                                                                  size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  (void)N;
  *bytes = precision != CODA_PREC_BF16 ? fwd_fp8_bytes(M, K, is_mx(precision), prec_elem(precision)) : 0;
  return CODA_OK;
}

extern "C" coda_status coda_linear_rmsnorm_residual_fwd(const coda_mat* a, const coda_weight* W, const coda_mat* residual,
                                                        const coda_mat* out, const coda_mat* P_out, int32_t precision,
                                                        void* ws, size_t ws_bytes, void* stream) {
  TRY(check_precision_fwd(precision));
  TRY(check_mat(a, "a", CODA_BF16, -1, -1));
  const int64_t M = a->rows, K = a->cols;
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  const int64_t N = W->w.cols;
  TRY(check_weight(W, "W", K, N, precision));
  TRY(check_mat(residual, "residual", CODA_BF16, M, N));
  TRY(check_mat(out, "out", CODA_BF16, M, N));
  TRY(check_mat(P_out, "sumsq_partials_out", CODA_F32, coda_partials_cols(N), M, true));
  if (present(P_out) && P_out->rows > 1 && P_out->ld != M) return fail(CODA_ERR_LAYOUT, "partials: ld must be M");
  Carver cv(ws);
  ActQ aq{};
  const bool fp8 = precision != CODA_PREC_BF16;
  if (fp8) aq = take_act(cv, M, K, 1, is_mx(precision), prec_elem(precision));
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  EpiArgs e = epi0();
  e.out = out->ptr; e.ld_out = out->ld;
  e.aux0 = residual->ptr; e.ld_aux0 = residual->ld;
  const Prog prog = present(P_out) ? Prog::ResidSumsq : Prog::Resid;
  if (present(P_out)) e.partial_out = static_cast<float*>(P_out->ptr);
  GemmArgs g;
  int layout;
  if (fp8) {
    TRY(quant_act(aq, a->ptr, a->ld, M, K, 1, s));
    g = gemm_args(aq.q.q, aq.q.ld, W->q_fwd.ptr, W->q_fwd.ld, M, N, aq.elem == 4 ? K / 2 : K);
    e.rowscale = aq.q.s; e.colscale = fptr(&W->s_fwd);
    if (aq.mx) mx_args(&g, &e, aq.e, aq.e_ld, &W->s_fwd);
    layout = LAYOUT_NT;
  } else {
    g = gemm_args(a->ptr, a->ld, W->w.ptr, W->w.ld, M, N, K);
    layout = LAYOUT_NN;
  }
  return launched(launch_fwd(prog, layout, fp8, aq.elem, g, e, s), "linear_rmsnorm_residual_fwd");
}

extern "C" coda_status coda_linear_qknorm_rope_fwd_workspace(int64_t M, int64_t D, int32_t have_partials,
                                                             int32_t precision, size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  Carver cv(nullptr);
  (void)have_partials;
  cv.take<float>(M);   // row sum of squares, or the merged partials
  if (precision != CODA_PREC_BF16) take_act(cv, M, D, 1, is_mx(precision), prec_elem(precision));
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_linear_qknorm_rope_fwd(const coda_mat* x, const coda_mat* P, const coda_weight* Wqkv,
                                                   const coda_mat* gq, const coda_mat* gk, const coda_mat* rope,
                                                   int32_t seq_len, float eps, const coda_mat* q, const coda_mat* k,
                                                   const coda_mat* v, const coda_mat* save, const coda_mat* r_out,
                                                   int32_t precision, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_precision_fwd(precision));
  TRY(check_mat(x, "x", CODA_BF16, -1, -1));
  const int64_t M = x->rows, D = x->cols;
  if (D == 0) return fail(CODA_ERR_SHAPE, "x: the normalised rows are empty (D = 0)");
  if (D % 128 != 0) return fail(CODA_ERR_SHAPE, "qknorm_rope: D must be a multiple of 128");
  if (!Wqkv) return fail(CODA_ERR_NULL, "Wqkv: NULL");
  TRY(check_weight(Wqkv, "Wqkv", D, 3 * D, precision));
  TRY(check_mat(P, "sumsq_partials", CODA_F32, -1, M, true));
  if (present(P) && (P->rows < 1 || P->rows > 32 || (P->rows > 1 && P->ld != M)))
    return fail(CODA_ERR_SHAPE, "sumsq_partials: 1..32 rows of M with ld == M");
  TRY(check_vec(gq, "gq", CODA_F32, 128));
  TRY(check_vec(gk, "gk", CODA_F32, 128));
  if (seq_len <= 0) return fail(CODA_ERR_VALUE, "seq_len must be > 0");
  TRY(check_mat(rope, "rope", CODA_F32, seq_len, 128));
  if (rope->ld != 128) return fail(CODA_ERR_LAYOUT, "rope: ld must be 128");
  TRY(check_mat(q, "q", CODA_BF16, M, D));
  TRY(check_mat(k, "k", CODA_BF16, M, D));
  TRY(check_mat(v, "v", CODA_BF16, M, D));
  TRY(check_mat(save, "save_qk_pre", CODA_BF16, M, 2 * D, true));
  TRY(check_vec(r_out, "r_out", CODA_F32, M, true));
  if (!(eps >= 0.0f)) return fail(CODA_ERR_VALUE, "eps must be >= 0");
  Carver cv(ws);
  float* sumsq = cv.take<float>(M);
  const bool fp8 = precision != CODA_PREC_BF16;
  ActQ aq{};
  if (fp8) aq = take_act(cv, M, D, 1, is_mx(precision), prec_elem(precision));
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  if (!present(P)) TRY(row_sumsq_launch(x->ptr, x->ld, M, D, sumsq, s));
  EpiArgs e = epi0();
  e.out = q->ptr; e.ld_out = q->ld;
  e.out2 = k->ptr; e.ld_out2 = k->ld;
  e.out3 = v->ptr; e.ld_out3 = v->ld;
  if (present(save)) { e.save = save->ptr; e.ld_save = save->ld; }
  e.row_partials = present(P) ? fptr(P) : sumsq;
  e.n_row_partials = present(P) ? (int)P->rows : 1;
  TRY(narrow_partials(&e.row_partials, &e.n_row_partials, M, sumsq, s));
  e.norm_dim = (int)D;
  e.eps = eps;
  e.rowvec_out = present(r_out) ? static_cast<float*>(r_out->ptr) : nullptr;
  e.colvec = fptr(gq); e.colvec2 = fptr(gk);
  e.table = fptr(rope);
  e.region = (int)D;
  e.seq_len = seq_len;
  GemmArgs g;
  int layout;
  if (fp8) {
    TRY(quant_act(aq, x->ptr, x->ld, M, D, 1, s));
    g = gemm_args(aq.q.q, aq.q.ld, Wqkv->q_fwd.ptr, Wqkv->q_fwd.ld, M, 3 * D, aq.elem == 4 ? D / 2 : D);
    e.rowscale = aq.q.s; e.colscale = fptr(&Wqkv->s_fwd);
    if (aq.mx) mx_args(&g, &e, aq.e, aq.e_ld, &Wqkv->s_fwd);
    layout = LAYOUT_NT;
  } else {
    g = gemm_args(x->ptr, x->ld, Wqkv->w.ptr, Wqkv->w.ld, M, 3 * D, D);
    layout = LAYOUT_NN;
  }
  return launched(launch_fwd(Prog::QKRope, layout, fp8, aq.elem, g, e, s), "linear_qknorm_rope_fwd");
}

// ======================================================================== functional backward
namespace {
// The two GEMM forms of a backward: input gradient (dgrad) and weight gradient (wgrad).
//   dgrad: C[M, Kin] = G[M, Nout] W^T   (bf16: NT with the stored weight; fp8: NT with q_bwd)
//   wgrad: C[Kin, Nout] = X^T[Kin, M] G[M, Nout]  (bf16: TN; fp8: NT with both transposed-quantised)
struct Bwd8 {
  ActQ grow;   // G per row (dgrad A operand)
  ActQ xcol;   // X per column, transposed (wgrad A operand)
  ActQ gcol;   // G per column, transposed (wgrad B operand)
};
}  // namespace

static coda_status dgrad_args(bool fp8, const ActQ* grow, const void* G, int64_t ldG, const coda_weight* W,
                              int64_t M, int64_t Kin, int64_t Nout, GemmArgs* g, EpiArgs* e) {
  if (fp8) {
    if (!present(&W->q_bwd))
      return fail(CODA_ERR_NULL, "the weight has no input-gradient copy (q_bwd) for this precision");
    *g = gemm_args(grow->q.q, grow->q.ld, W->q_bwd.ptr, W->q_bwd.ld, M, Kin, Nout);
    e->rowscale = grow->q.s;
    e->colscale = fptr(&W->s_bwd);
    if (grow->mx) mx_args(g, e, grow->e, grow->e_ld, &W->s_bwd);
  } else {
    *g = gemm_args(G, ldG, W->w.ptr, W->w.ld, M, Kin, Nout);
  }
  return CODA_OK;
}

static void wgrad_args(bool fp8, const Bwd8& q8, const void* X, int64_t ldX, const void* G, int64_t ldG, int64_t M,
                       int64_t Kin, int64_t Nout, GemmArgs* g, EpiArgs* e, int* layout) {
  if (fp8) {
    *g = gemm_args(q8.xcol.q.q, q8.xcol.q.ld, q8.gcol.q.q, q8.gcol.q.ld, Kin, Nout, M);
    e->rowscale = q8.xcol.q.s;
    e->colscale = q8.gcol.q.s;
    if (q8.xcol.mx) {
      g->sA = q8.xcol.e; g->lds_a = q8.xcol.e_ld;
      g->sB = q8.gcol.e; g->lds_b = q8.gcol.e_ld;
      e->rowscale = nullptr; e->colscale = nullptr;
    }
    *layout = LAYOUT_NT;
  } else {
    *g = gemm_args(X, ldX, G, ldG, Kin, Nout, M);
    *layout = LAYOUT_TN;
  }
}

// Weight-gradient GEMMs contract over the tokens.  When the output has too
// few 256 x 256 tiles to fill the chip (a 2048 x 2048 weight has 64), the
// tokens are cut into up to 4 slices (a multiple of 64 each) that run as
// extra workgroups and write fp32 partial products to the workspace; a
// second pass adds the slices in order (bitwise deterministic).
struct Split {
  int n = 1;         // slices
  int64_t kchunk;    // tokens per slice
};

static Split wgrad_split(int64_t Kin, int64_t Nout, int64_t M, int64_t align = 64) {
  Split sp;
  sp.kchunk = M;
  const int64_t tiles = ((Kin + 255) / 256) * ((Nout + 255) / 256);
  int want = 1;
  if (tiles * 4 <= 256 && M >= 4096) want = 4;
  else if (tiles * 2 <= 256 && M >= 2048) want = 2;
  if (want > 1) {
    sp.kchunk = ((M + want - 1) / want + align - 1) / align * align;   // MXFP8: whole 128-token words
    sp.n = (int)((M + sp.kchunk - 1) / sp.kchunk);
  }
  return sp;
}

// Launches a weight-gradient GEMM whose epilogue writes D = beta D + value
// (fp32, e->out / e->ld_out / e->beta) and, optionally, row partials
// (e->partial_out, `pstride` floats per slice).  With sp.n > 1 the slices go
// to `part` (sp.n x Kin x Nout floats) and split_sum_kernel finishes D.
static coda_status launch_wgrad(Prog p, int layout, int prec, GemmArgs g, EpiArgs e, const Split& sp, float* part,
                                int64_t pstride, hipStream_t s, const char* what) {
  if (sp.n <= 1) return launched(launch_prec(p, layout, prec, g, e, s), what);
  float* out = static_cast<float*>(e.out);
  const int64_t ld = e.ld_out;
  const float beta = e.beta;
  const int64_t slice = (int64_t)g.M * g.N;
  e.out = part;
  e.ld_out = g.N;
  e.beta = 0.0f;
  e.split_stride = slice;
  e.split_pstride = pstride;
  g.kchunk = (int)sp.kchunk;
  TRY(launched(launch_prec(p, layout, prec, g, e, s), what));
  const int64_t quads = slice / 4;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, part, sp.n, slice, g.M,
                     g.N, beta, out, ld);
  return check_launch(what);
}

static coda_status sum_partials_launch(const float* P, int nP, int K, float beta, float* out, hipStream_t s) {
  if (K == 0) return CODA_OK;
  hipLaunchKernelGGL(sum_partials_kernel, dim3((K + 63) / 64), dim3(1024), 0, s, P, nP, K, beta, out);
  return check_launch("sum_partials");
}

// An empty token batch (M = 0) adds nothing to a gradient accumulator, so the
// backward entry points only apply D = beta D (beta 0 clears D without
// reading it, as the epilogues do) and launch no GEMM.
static coda_status scale_accum(const coda_mat* D, float beta, hipStream_t s, const char* what) {
  if (!present(D) || beta == 1.0f || D->rows == 0 || D->cols == 0) return CODA_OK;
  hipLaunchKernelGGL(scale_f32_kernel, dim3((unsigned)((D->cols + 255) / 256), (unsigned)std::min<int64_t>(D->rows, 65535)),
                     dim3(256), 0, s, static_cast<float*>(D->ptr), D->ld, (int)D->rows, (int)D->cols, beta);
  return check_launch(what);
}

static coda_status swiglu_bwd_impl(const coda_mat* dY, const coda_weight* Wd, const coda_mat* hgu, const coda_mat* r,
                                   const coda_mat* u, const coda_weight* Wgu, const coda_mat* Wunf, const coda_mat* gvec,
                                   const coda_mat* dres, const coda_mat* du, const coda_mat* dWgu, const coda_mat* dg,
                                   float beta, const coda_mat* dh_out, int precision, void* ws, size_t ws_bytes,
                                   void* stream, int64_t M, int64_t D, int64_t F, bool size_only, size_t* bytes,
                                   Act act = Act::SwiGLU) {
  // F is the width of the activation's output; the pre-activations are 2F
  // wide for SwiGLU (packed gate/up) and F wide for the elementwise maps
  const int64_t N2 = act == Act::SwiGLU ? 2 * F : F;
  const bool fp8 = precision != CODA_PREC_BF16, mx = is_mx(precision);
  const int elem = prec_elem(precision);
  if (mx && M % 128 != 0) return fail(CODA_ERR_SHAPE, "MX backward: the token count must be a multiple of 128");
  Carver cv(size_only ? nullptr : ws);
  const int nT2 = (int)coda_partials_cols(F);
  const int nTg = (int)coda_partials_cols(N2);
  float* T2 = cv.take<float>((size_t)nT2 * M);
  float* T2c = cv.take<float>(M);
  const Split sp = wgrad_split(D, N2, M, mx ? 128 : 64);
  float* dgp = cv.take<float>((size_t)sp.n * nTg * D);
  float* part = sp.n > 1 ? cv.take<float>((size_t)sp.n * D * N2) : nullptr;
  uint16_t* dh = present(dh_out) ? nullptr : cv.take<uint16_t>((size_t)M * N2);
  Bwd8 q8{};
  ActQ dYrow{};
  if (fp8) {
    dYrow = take_act(cv, M, D, 1, mx, elem);
    q8.grow = take_act(cv, M, N2, 1, mx, elem);
    q8.xcol = take_act(cv, M, D, 0, mx, elem);
    q8.gcol = take_act(cv, M, N2, 0, mx, elem);
  }
  if (size_only) { *bytes = cv.off; return CODA_OK; }
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  if (M == 0) {
    TRY(scale_accum(dWgu, beta, s, "swiglu_bwd: dW of no tokens"));
    return scale_accum(dg, beta, s, "swiglu_bwd: dg of no tokens");
  }
  void* dhp = present(dh_out) ? dh_out->ptr : dh;
  const int64_t lddh = present(dh_out) ? dh_out->ld : N2;
  // B1: da = dY Wd^T with dSwiGLU, r scale, T partials
  {
    EpiArgs e = epi0();
    e.out = dhp; e.ld_out = lddh;
    e.aux0 = hgu->ptr; e.ld_aux0 = hgu->ld;
    e.rowvec = fptr(r);
    e.partial_out = T2;
    GemmArgs g;
    if (fp8) TRY(quant_act(dYrow, dY->ptr, dY->ld, M, D, 1, s));
    dgrad_args(fp8, &dYrow, dY->ptr, dY->ld, Wd, M, F, D, &g, &e);
    const Prog back = act == Act::SwiGLU ? Prog::DSwiGLU : act == Act::Sigmoid ? Prog::DSigmoid : Prog::DGelu;
    TRY(launched(launch_prec(back, LAYOUT_NT, precision, g, e, s),
                 "swiglu_bwd: activation backward"));
  }
  // collapse the T partials (F / 256 of them) to one per row
  hipLaunchKernelGGL(rows_finish_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, T2, nT2, (int)M, 0,
                     (const float*)nullptr, 0, 0.0f, T2c);
  TRY(check_launch("swiglu_bwd: finish T"));
  if (fp8) {
    TRY(quant_act(q8.grow, dhp, lddh, M, N2, 1, s));
    TRY(quant_act(q8.xcol, u->ptr, u->ld, M, D, 0, s));
    TRY(quant_act(q8.gcol, dhp, lddh, M, N2, 0, s));
  }
  // B3: du = dh~ W~gu^T - c u + dres
  {
    EpiArgs e = epi0();
    e.out = du->ptr; e.ld_out = du->ld;
    e.aux0 = u->ptr; e.ld_aux0 = u->ld;
    if (present(dres)) { e.aux1 = dres->ptr; e.ld_aux1 = dres->ld; }
    else return fail(CODA_ERR_UNSUPPORTED, "swiglu_bwd: dres is required in this build");
    e.rowvec = fptr(r);
    e.row_partials = T2c;
    e.n_row_partials = 1;
    e.norm_dim = (int)D;
    GemmArgs g;
    dgrad_args(fp8, &q8.grow, dhp, lddh, Wgu, M, D, N2, &g, &e);
    TRY(launched(launch_prec(Prog::NormCorr, LAYOUT_NT, precision, g, e, s), "swiglu_bwd: du"));
  }
  // B4: dW = beta dW + g (u^T dh~), gain partials
  {
    EpiArgs e = epi0();
    e.out = dWgu->ptr; e.ld_out = dWgu->ld;
    e.beta = beta;
    e.aux0 = Wunf->ptr; e.ld_aux0 = Wunf->ld;
    e.rowvec = fptr(gvec);
    e.partial_out = dgp;
    GemmArgs g;
    int layout;
    wgrad_args(fp8, q8, u->ptr, u->ld, dhp, lddh, M, D, N2, &g, &e, &layout);
    TRY(launch_wgrad(Prog::WgradGain, layout, precision, g, e, sp, part, (int64_t)nTg * D, s, "swiglu_bwd: dW"));
  }
  return sum_partials_launch(dgp, sp.n * nTg, (int)D, beta, static_cast<float*>(dg->ptr), s);
}

static coda_status swiglu_bwd_check(const coda_mat* dY, const coda_weight* Wd, const coda_mat* hgu, const coda_mat* r,
                                    const coda_mat* u, const coda_weight* Wgu, const coda_mat* Wunf, const coda_mat* g,
                                    const coda_mat* dres, const coda_mat* du, const coda_mat* dWgu, const coda_mat* dg,
                                    const coda_mat* dh_out, int precision, int64_t* M, int64_t* D, int64_t* F) {
  TRY(check_precision(precision));
  TRY(check_mat(dY, "dY", CODA_BF16, -1, -1));
  *M = dY->rows; *D = dY->cols;
  if (!Wd || !Wgu) return fail(CODA_ERR_NULL, "weights: NULL");
  *F = Wd->w.rows;
  if (*F % 32 != 0) return fail(CODA_ERR_SHAPE, "F must be a multiple of 32");
  TRY(check_weight(Wd, "Wd", *F, *D, precision));
  TRY(check_weight(Wgu, "Wgu", *D, 2 * *F, precision));
  TRY(check_mat(hgu, "saved_hgu", CODA_BF16, *M, 2 * *F));
  TRY(check_vec(r, "r", CODA_F32, *M));
  TRY(check_mat(u, "u", CODA_BF16, *M, *D));
  TRY(check_mat(Wunf, "Wgu_unfolded", CODA_BF16, *D, 2 * *F));
  TRY(check_vec(g, "g", CODA_F32, *D));
  TRY(check_mat(dres, "dres", CODA_BF16, *M, *D));
  TRY(check_mat(du, "du", CODA_BF16, *M, *D));
  TRY(check_mat(dWgu, "dWgu", CODA_F32, *D, 2 * *F));
  TRY(check_vec(dg, "dg", CODA_F32, *D));
  TRY(check_mat(dh_out, "dh_gu_out", CODA_BF16, *M, 2 * *F, true));
  return CODA_OK;
}

extern "C" coda_status coda_linear_swiglu_bwd_workspace(int64_t M, int64_t D, int64_t F, int32_t precision,
                                                        size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  return swiglu_bwd_impl(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, 0.0f, nullptr, precision, nullptr, 0, nullptr, M, D, F, true, bytes);
}

extern "C" coda_status coda_linear_swiglu_bwd(const coda_mat* dY, const coda_weight* Wd, const coda_mat* saved_hgu,
                                              const coda_mat* r, const coda_mat* u, const coda_weight* Wgu,
                                              const coda_mat* Wgu_unfolded, const coda_mat* g, const coda_mat* dres,
                                              const coda_mat* du, const coda_mat* dWgu, const coda_mat* dg, float beta,
                                              const coda_mat* dh_gu_out, int32_t precision, void* ws, size_t ws_bytes,
                                              void* stream) {
  int64_t M, D, F;
  TRY(swiglu_bwd_check(dY, Wd, saved_hgu, r, u, Wgu, Wgu_unfolded, g, dres, du, dWgu, dg, dh_gu_out, precision, &M,
                       &D, &F));
  if (D == 0) return fail(CODA_ERR_SHAPE, "u: the normalised rows are empty (D = 0)");
  return swiglu_bwd_impl(dY, Wd, saved_hgu, r, u, Wgu, Wgu_unfolded, g, dres, du, dWgu, dg, beta, dh_gu_out,
                         precision, ws, ws_bytes, stream, M, D, F, false, nullptr);
}

extern "C" coda_status coda_linear_rmsnorm_residual_bwd_workspace(int64_t M, int64_t K, int64_t N, int32_t precision,
                                                                  size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  Carver cv(nullptr);
  const bool mx = is_mx(precision);
  const int elem = prec_elem(precision);
  if (precision != CODA_PREC_BF16) {
    take_act(cv, M, N, 1, mx, elem);
    take_act(cv, M, K, 0, mx, elem);
    take_act(cv, M, N, 0, mx, elem);
  }
  const Split sp = wgrad_split(K, N, M, mx ? 128 : 64);
  if (sp.n > 1) cv.take<float>((size_t)sp.n * K * N);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_linear_rmsnorm_residual_bwd(const coda_mat* d_out, const coda_mat* a, const coda_weight* W,
                                                        const coda_mat* da, const coda_mat* dW, float beta,
                                                        int32_t precision, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_precision(precision));
  TRY(check_mat(d_out, "d_out", CODA_BF16, -1, -1));
  const int64_t M = d_out->rows, N = d_out->cols;
  TRY(check_mat(a, "a", CODA_BF16, M, -1));
  const int64_t K = a->cols;
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  TRY(check_weight(W, "W", K, N, precision));
  TRY(check_mat(da, "da", CODA_BF16, M, K, true));
  TRY(check_mat(dW, "dW", CODA_F32, K, N));
  const bool fp8 = precision != CODA_PREC_BF16, mx = is_mx(precision);
  const int elem = prec_elem(precision);
  if (mx && M % 128 != 0) return fail(CODA_ERR_SHAPE, "MX backward: the token count must be a multiple of 128");
  Carver cv(ws);
  Bwd8 q8{};
  if (fp8) {
    q8.grow = take_act(cv, M, N, 1, mx, elem);
    q8.xcol = take_act(cv, M, K, 0, mx, elem);
    q8.gcol = take_act(cv, M, N, 0, mx, elem);
  }
  const Split sp = wgrad_split(K, N, M, mx ? 128 : 64);
  float* part = sp.n > 1 ? cv.take<float>((size_t)sp.n * K * N) : nullptr;
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  if (M == 0) return scale_accum(dW, beta, s, "rmsnorm_residual_bwd: dW of no tokens");
  if (fp8) {
    if (present(da)) TRY(quant_act(q8.grow, d_out->ptr, d_out->ld, M, N, 1, s));
    TRY(quant_act(q8.xcol, a->ptr, a->ld, M, K, 0, s));
    TRY(quant_act(q8.gcol, d_out->ptr, d_out->ld, M, N, 0, s));
  }
  if (present(da)) {
    EpiArgs e = epi0();
    e.out = da->ptr; e.ld_out = da->ld;
    GemmArgs g;
    dgrad_args(fp8, &q8.grow, d_out->ptr, d_out->ld, W, M, K, N, &g, &e);
    TRY(launched(launch_prec(Prog::Store, LAYOUT_NT, precision, g, e, s), "rmsnorm_residual_bwd: da"));
  }
  EpiArgs e = epi0();
  e.out = dW->ptr; e.ld_out = dW->ld;
  e.beta = beta;
  GemmArgs g;
  int layout;
  wgrad_args(fp8, q8, a->ptr, a->ld, d_out->ptr, d_out->ld, M, K, N, &g, &e, &layout);
  return launch_wgrad(Prog::StoreF32, layout, precision, g, e, sp, part, 0, s, "rmsnorm_residual_bwd: dW");
}

static coda_status qk_bwd_impl(const coda_mat* dq, const coda_mat* dk, const coda_mat* dv, const coda_mat* x,
                               const coda_mat* r, const coda_mat* qk_pre, const coda_mat* v, const coda_weight* Wqkv,
                               const coda_mat* Wunf, const coda_mat* gvec, const coda_mat* gq, const coda_mat* gk,
                               const coda_mat* rope, int seq_len, float eps, const coda_mat* dres, const coda_mat* dx,
                               const coda_mat* dW, const coda_mat* dg, const coda_mat* dgq, const coda_mat* dgk,
                               float beta, const coda_mat* dh_out, int precision, void* ws, size_t ws_bytes,
                               void* stream, int64_t M, int64_t D, bool size_only, size_t* bytes) {
  const bool fp8 = precision != CODA_PREC_BF16, mx = is_mx(precision);
  const int elem = prec_elem(precision);
  if (mx && M % 128 != 0) return fail(CODA_ERR_SHAPE, "MX backward: the token count must be a multiple of 128");
  const int64_t N3 = 3 * D;
  const int rows_per_wave = 4;
  const int nblk = (int)((M + 4 * rows_per_wave - 1) / (4 * rows_per_wave));
  Carver cv(size_only ? nullptr : ws);
  uint16_t* dh = cv.take<uint16_t>((size_t)M * N3);
  int64_t ldh = N3;
  if (!size_only && present(dh_out)) {   // the caller keeps dh~ (same traffic, its own buffer)
    dh = static_cast<uint16_t*>(dh_out->ptr);
    ldh = dh_out->ld;
  }
  float* T1 = cv.take<float>(M);
  float* pgq = cv.take<float>((size_t)std::max(nblk, 1) * 128);
  float* pgk = cv.take<float>((size_t)std::max(nblk, 1) * 128);
  const int nTg = (int)coda_partials_cols(N3);
  const Split sp = wgrad_split(D, N3, M, mx ? 128 : 64);
  float* dgp = cv.take<float>((size_t)sp.n * nTg * D);
  float* part = sp.n > 1 ? cv.take<float>((size_t)sp.n * D * N3) : nullptr;
  Bwd8 q8{};
  if (fp8) {
    q8.grow = take_act(cv, M, N3, 1, mx, elem);
    q8.xcol = take_act(cv, M, D, 0, mx, elem);
    q8.gcol = take_act(cv, M, N3, 0, mx, elem);
  }
  if (size_only) { *bytes = cv.off; return CODA_OK; }
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  if (M == 0) {
    TRY(scale_accum(dW, beta, s, "qknorm_rope_bwd: dW of no tokens"));
    TRY(scale_accum(dg, beta, s, "qknorm_rope_bwd: dg of no tokens"));
    TRY(scale_accum(dgq, beta, s, "qknorm_rope_bwd: dgq of no tokens"));
    return scale_accum(dgk, beta, s, "qknorm_rope_bwd: dgk of no tokens");
  }
  {
    hipLaunchKernelGGL(qknorm_rope_bwd_kernel, dim3(nblk), dim3(256), 0, s, static_cast<const uint16_t*>(dq->ptr),
                       static_cast<const uint16_t*>(dk->ptr), static_cast<const uint16_t*>(dv->ptr), dq->ld,
                       static_cast<const uint16_t*>(qk_pre->ptr), qk_pre->ld, static_cast<const uint16_t*>(v->ptr),
                       v->ld, fptr(r), fptr(gq), fptr(gk), fptr(rope), seq_len, eps, (int)M, (int)D, rows_per_wave,
                       dh, ldh, T1, pgq, pgk);
    TRY(check_launch("qknorm_rope_bwd: glue"));
  }
  TRY(sum_partials_launch(pgq, nblk, 128, beta, static_cast<float*>(dgq->ptr), s));
  TRY(sum_partials_launch(pgk, nblk, 128, beta, static_cast<float*>(dgk->ptr), s));
  if (fp8) {
    TRY(quant_act(q8.grow, dh, ldh, M, N3, 1, s));
    TRY(quant_act(q8.xcol, x->ptr, x->ld, M, D, 0, s));
    TRY(quant_act(q8.gcol, dh, ldh, M, N3, 0, s));
  }
  {
    EpiArgs e = epi0();
    e.out = dx->ptr; e.ld_out = dx->ld;
    e.aux0 = x->ptr; e.ld_aux0 = x->ld;
    e.aux1 = dres->ptr; e.ld_aux1 = dres->ld;
    e.rowvec = fptr(r);
    e.row_partials = T1;
    e.n_row_partials = 1;
    e.norm_dim = (int)D;
    GemmArgs g;
    dgrad_args(fp8, &q8.grow, dh, ldh, Wqkv, M, D, N3, &g, &e);
    TRY(launched(launch_prec(Prog::NormCorr, LAYOUT_NT, precision, g, e, s), "qknorm_rope_bwd: dx"));
  }
  {
    EpiArgs e = epi0();
    e.out = dW->ptr; e.ld_out = dW->ld;
    e.beta = beta;
    e.aux0 = Wunf->ptr; e.ld_aux0 = Wunf->ld;
    e.rowvec = fptr(gvec);
    e.partial_out = dgp;
    GemmArgs g;
    int layout;
    wgrad_args(fp8, q8, x->ptr, x->ld, dh, ldh, M, D, N3, &g, &e, &layout);
    TRY(launch_wgrad(Prog::WgradGain, layout, precision, g, e, sp, part, (int64_t)nTg * D, s, "qknorm_rope_bwd: dW"));
  }
  return sum_partials_launch(dgp, sp.n * nTg, (int)D, beta, static_cast<float*>(dg->ptr), s);
}

extern "C" coda_status coda_linear_qknorm_rope_bwd_workspace(int64_t M, int64_t D, int32_t precision, size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  return qk_bwd_impl(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, 1, 0.0f, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0.0f, nullptr,
                     precision, nullptr, 0, nullptr, M, D, true, bytes);
}

extern "C" coda_status coda_linear_qknorm_rope_bwd(const coda_mat* dq, const coda_mat* dk, const coda_mat* dv,
                                                   const coda_mat* x, const coda_mat* r, const coda_mat* qk_pre,
                                                   const coda_mat* v, const coda_weight* Wqkv, const coda_mat* Wunf,
                                                   const coda_mat* g, const coda_mat* gq, const coda_mat* gk,
                                                   const coda_mat* rope, int32_t seq_len, float eps, const coda_mat* dres,
                                                   const coda_mat* dx, const coda_mat* dW, const coda_mat* dg,
                                                   const coda_mat* dgq, const coda_mat* dgk, float beta,
                                                   const coda_mat* dh_qkv_out, int32_t precision, void* ws,
                                                   size_t ws_bytes, void* stream) {
  TRY(check_precision(precision));
  TRY(check_mat(x, "x", CODA_BF16, -1, -1));
  const int64_t M = x->rows, D = x->cols;
  if (D == 0) return fail(CODA_ERR_SHAPE, "x: the normalised rows are empty (D = 0)");
  if (D % 128 != 0) return fail(CODA_ERR_SHAPE, "D must be a multiple of 128");
  TRY(check_mat(dq, "dq", CODA_BF16, M, D));
  TRY(check_mat(dk, "dk", CODA_BF16, M, D));
  TRY(check_mat(dv, "dv", CODA_BF16, M, D));
  if (dk->ld != dq->ld || dv->ld != dq->ld) return fail(CODA_ERR_LAYOUT, "dq, dk, dv must share ld");
  TRY(check_vec(r, "r", CODA_F32, M));
  TRY(check_mat(qk_pre, "qk_pre", CODA_BF16, M, 2 * D));
  TRY(check_mat(v, "v", CODA_BF16, M, D));
  if (!Wqkv) return fail(CODA_ERR_NULL, "Wqkv: NULL");
  TRY(check_weight(Wqkv, "Wqkv", D, 3 * D, precision));
  TRY(check_mat(Wunf, "Wqkv_unfolded", CODA_BF16, D, 3 * D));
  TRY(check_vec(g, "g", CODA_F32, D));
  TRY(check_vec(gq, "gq", CODA_F32, 128));
  TRY(check_vec(gk, "gk", CODA_F32, 128));
  if (seq_len <= 0) return fail(CODA_ERR_VALUE, "seq_len must be > 0");
  TRY(check_mat(rope, "rope", CODA_F32, seq_len, 128));
  TRY(check_mat(dres, "dres", CODA_BF16, M, D));
  TRY(check_mat(dx, "dx", CODA_BF16, M, D));
  TRY(check_mat(dW, "dW", CODA_F32, D, 3 * D));
  TRY(check_vec(dg, "dg", CODA_F32, D));
  TRY(check_vec(dgq, "dgq", CODA_F32, 128));
  TRY(check_vec(dgk, "dgk", CODA_F32, 128));
  TRY(check_mat(dh_qkv_out, "dh_qkv_out", CODA_BF16, M, 3 * D, true));
  return qk_bwd_impl(dq, dk, dv, x, r, qk_pre, v, Wqkv, Wunf, g, gq, gk, rope, seq_len, eps, dres, dx, dW, dg, dgq, dgk,
                     beta, dh_qkv_out, precision, ws, ws_bytes, stream, M, D, false, nullptr);
}

// ======================================================================== cross-entropy
static size_t ce_fwd_layout(Carver& cv, int64_t M, int64_t V, int64_t D, int precision, float** Pm, float** Ps,
                            float** zy, float** per_row, int** status, ActQ* aq) {
  const int nT = (int)coda_partials_cols(V);
  *Pm = cv.take<float>((size_t)nT * M);
  *Ps = cv.take<float>((size_t)nT * M);
  *zy = cv.take<float>(M);
  *per_row = cv.take<float>(M);
  *status = cv.take<int>(M);
  if (precision == CODA_PREC_FP8) *aq = take_act(cv, M, D, 1);
  return cv.off;
}

static coda_status ce_fwd_impl(const coda_mat* h, const coda_weight* W, const coda_mat* labels, int32_t ignore_index,
                               const coda_mat* loss, const coda_mat* lse, const coda_mat* per_row,
                               const coda_mat* n_valid, const coda_mat* n_bad, int32_t precision, void* ws,
                               size_t ws_bytes, void* stream, const char* who);

extern "C" coda_status coda_linear_cross_entropy_fwd_workspace(int64_t M, int64_t D, int64_t V, int32_t precision,
                                                               size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  Carver cv(nullptr);
  float *a, *b, *c, *d;
  int* st;
  ActQ aq;
  ce_fwd_layout(cv, M, V, D, precision, &a, &b, &c, &d, &st, &aq);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_linear_cross_entropy_fwd(const coda_mat* h, const coda_weight* W, const coda_mat* labels,
                                                     int32_t ignore_index, const coda_mat* loss, const coda_mat* lse,
                                                     const coda_mat* per_row, const coda_mat* n_valid,
                                                     const coda_mat* n_bad, int32_t precision, void* ws,
                                                     size_t ws_bytes, void* stream) {
  return ce_fwd_impl(h, W, labels, ignore_index, loss, lse, per_row, n_valid, n_bad, precision, ws, ws_bytes, stream,
                     "cross_entropy_fwd");
}

// ---- the same forward without a workspace argument, for callers that cannot
// allocate.  Its partial (max, sum-exp) rows, label logits and row status live
// in this file-scope device array, one copy per GPU, held until the process
// ends.  Every element the forward reads there is written earlier in the same
// call (each (N tile, row) partial by its tile, each row's status by the row
// finish), so nothing needs clearing between calls; calls that overlap on one
// GPU share the array and race.
static __device__ __align__(256) char scratch[CODA_CE_FWD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the current device's copy of `scratch` (the array's
// name in host code is only a stand-in for it).
coda_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CODA_ERR_LAUNCH, "cross_entropy_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy_fwd_noalloc: device %d", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
    return fail(CODA_ERR_LAUNCH, "cross_entropy_fwd_noalloc: hipGetSymbolAddress: %s",
                hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return CODA_OK;
}
}  // namespace

extern "C" coda_status coda_linear_cross_entropy_fwd_noalloc(const coda_mat* h, const coda_weight* W,
                                                             const coda_mat* labels, int32_t ignore_index,
                                                             const coda_mat* loss, const coda_mat* lse,
                                                             const coda_mat* per_row, const coda_mat* n_valid,
                                                             const coda_mat* n_bad, void* stream) {
  TRY(check_mat(h, "h", CODA_BF16, -1, -1));
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  size_t need = 0;
  TRY(coda_linear_cross_entropy_fwd_workspace(h->rows, h->cols, W->w.cols, CODA_PREC_BF16, &need));
  if (need > sizeof(scratch))
    return fail(CODA_ERR_WORKSPACE,
                "cross_entropy_fwd_noalloc: M = %lld, V = %lld needs %zu bytes of scratch, at most %zu available",
                (long long)h->rows, (long long)W->w.cols, need, sizeof(scratch));
  void* ptr = nullptr;
  TRY(scratch_ptr(&ptr));
  return ce_fwd_impl(h, W, labels, ignore_index, loss, lse, per_row, n_valid, n_bad, CODA_PREC_BF16, ptr,
                     sizeof(scratch), stream, "cross_entropy_fwd_noalloc");
}

static coda_status ce_fwd_impl(const coda_mat* h, const coda_weight* W, const coda_mat* labels, int32_t ignore_index,
                               const coda_mat* loss, const coda_mat* lse, const coda_mat* per_row,
                               const coda_mat* n_valid, const coda_mat* n_bad, int32_t precision, void* ws,
                               size_t ws_bytes, void* stream, const char* who) {
  TRY(check_precision(precision));
  if (precision != CODA_PREC_BF16) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy: fp8 not compiled in this build");
  TRY(check_mat(h, "h", CODA_BF16, -1, -1));
  const int64_t M = h->rows, D = h->cols;
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  const int64_t V = W->w.cols;
  TRY(check_weight(W, "W", D, V, precision));
  TRY(check_vec(labels, "labels", CODA_I32, M));
  TRY(check_vec(loss, "loss", CODA_F32, 1));
  TRY(check_vec(lse, "lse", CODA_F32, M));
  TRY(check_vec(per_row, "per_row", CODA_F32, M, true));
  TRY(check_vec(n_valid, "n_valid", CODA_I32, 1));
  TRY(check_vec(n_bad, "n_bad", CODA_I32, 1, true));
  if (ignore_index >= 0 && ignore_index < V) return fail(CODA_ERR_VALUE, "ignore_index must lie outside [0, V)");
  Carver cv(ws);
  float *Pm, *Ps, *zy, *pr;
  int* st;
  ActQ aq{};
  ce_fwd_layout(cv, M, V, D, precision, &Pm, &Ps, &zy, &pr, &st, &aq);
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  float* per = present(per_row) ? static_cast<float*>(per_row->ptr) : pr;
  if (M > 0) {
    EpiArgs e = epi0();
    e.labels = static_cast<const int*>(labels->ptr);
    e.partial_out = Pm;
    e.partial_out2 = Ps;
    e.rowvec_out = zy;
    e.vocab = (int)V;
    GemmArgs g = gemm_args(h->ptr, h->ld, W->w.ptr, W->w.ld, M, V, D);
    TRY(launched(launch_gemm(Prog::CrossEntropy, LAYOUT_NN, false, g, e, s), who));
    hipLaunchKernelGGL(ce_finish_rows_kernel, dim3((unsigned)((M + 63) / 64)), dim3(256), 0, s, Pm, Ps,
                       (int)coda_partials_cols(V), (int)M, zy, static_cast<const int*>(labels->ptr), (int)V,
                       ignore_index, static_cast<float*>(lse->ptr), per, st);
    TRY(check_launch(who));
  }
  hipLaunchKernelGGL(ce_finish_loss_kernel, dim3(1), dim3(1024), 0, s, per, st, (int)M, static_cast<float*>(loss->ptr),
                     static_cast<int*>(n_valid->ptr), present(n_bad) ? static_cast<int*>(n_bad->ptr) : nullptr);
  return check_launch(who);
}

// The backward recomputes the logits into a bf16 buffer G.  With chunk_rows
// = 0 (or >= M) G holds all M x V values and one pass of three GEMMs does the
// work.  Otherwise G is bounded by chunk_rows x V values and the recompute
// runs over vocabulary slices of vc columns (a multiple of 256): each slice's
// weight-gradient GEMM writes its own columns of dW (no read-modify-write of
// dW across slices) and its dh GEMM accumulates into an fp32 [M, D] buffer,
// rounded to bf16 once at the end.
// rows of a (x, rows) grid whose kernel strides over rows by gridDim.y
static unsigned row_grid(int64_t rows) { return (unsigned)std::min<int64_t>(rows, 65535); }

static int64_t ce_slice_cols(int64_t M, int64_t V, int64_t chunk_rows) {
  if (chunk_rows <= 0 || chunk_rows >= M) return V;
  const int64_t vc = chunk_rows * V / M / 256 * 256;
  return std::min(V, std::max<int64_t>(vc, 256));
}

static size_t ce_bwd_layout(Carver& cv, int64_t M, int64_t D, int64_t V, int64_t vc, float** scale, uint16_t** G,
                            float** dh_acc) {
  *scale = cv.take<float>(1);
  *G = cv.take<uint16_t>((size_t)M * ((vc + 7) / 8 * 8));
  *dh_acc = vc < V ? cv.take<float>((size_t)M * D) : nullptr;
  return cv.off;
}

extern "C" coda_status coda_linear_cross_entropy_bwd_workspace(int64_t M, int64_t D, int64_t V, int64_t chunk_rows,
                                                               int32_t precision, size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  if (precision != CODA_PREC_BF16) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy: fp8 not compiled in this build");
  Carver cv(nullptr);
  float* sc;
  uint16_t* G;
  float* acc;
  ce_bwd_layout(cv, M, D, V, ce_slice_cols(M, V, chunk_rows), &sc, &G, &acc);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_linear_cross_entropy_bwd(const coda_mat* h, const coda_weight* W, const coda_mat* labels,
                                                     int32_t ignore_index, const coda_mat* lse, const coda_mat* n_valid,
                                                     float dloss, const coda_mat* dh, const coda_mat* dW, float beta,
                                                     int64_t chunk_rows, int32_t precision, void* ws, size_t ws_bytes,
                                                     void* stream) {
  TRY(check_precision(precision));
  if (precision != CODA_PREC_BF16) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy: fp8 not compiled in this build");
  TRY(check_mat(h, "h", CODA_BF16, -1, -1));
  const int64_t M = h->rows, D = h->cols;
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  const int64_t V = W->w.cols;
  TRY(check_weight(W, "W", D, V, precision));
  TRY(check_vec(labels, "labels", CODA_I32, M));
  TRY(check_vec(lse, "lse", CODA_F32, M));
  TRY(check_vec(n_valid, "n_valid", CODA_I32, 1));
  TRY(check_mat(dh, "dh", CODA_BF16, M, D));
  TRY(check_mat(dW, "dW", CODA_F32, D, V));
  if (ignore_index >= 0 && ignore_index < V) return fail(CODA_ERR_VALUE, "ignore_index must lie outside [0, V)");
  const int64_t vc = ce_slice_cols(M, V, chunk_rows);
  Carver cv(ws);
  float* scale;
  uint16_t* G;
  float* dh_acc;
  ce_bwd_layout(cv, M, D, V, vc, &scale, &G, &dh_acc);
  TRY(ws_check(cv, ws_bytes, ws));
  if (M == 0) return scale_accum(dW, beta, S(stream), "cross_entropy_bwd: dW of no tokens");
  hipStream_t s = S(stream);
  const int64_t ldG = (vc + 7) / 8 * 8;
  hipLaunchKernelGGL(ce_scale_kernel, dim3(1), dim3(1), 0, s, static_cast<const int*>(n_valid->ptr), dloss, scale);
  TRY(check_launch("cross_entropy_bwd: scale"));
  const uint16_t* hp = static_cast<const uint16_t*>(h->ptr);
  const uint16_t* Wp = static_cast<const uint16_t*>(W->w.ptr);
  const int* lab = static_cast<const int*>(labels->ptr);
  const float* lsep = static_cast<const float*>(lse->ptr);
  for (int64_t v0 = 0; v0 < V; v0 += vc) {
    const int64_t nv = std::min(vc, V - v0);
    {  // recompute the logits of the slice into G: G = bf16(exp(z - lse) - onehot)
      EpiArgs e = epi0();
      e.out = G; e.ld_out = ldG;
      e.labels = lab;
      e.rowvec = lsep;
      e.col_offset = (int)v0;
      e.vocab = (int)V;
      GemmArgs g = gemm_args(hp, h->ld, Wp + v0, W->w.ld, M, nv, D);
      TRY(launched(launch_gemm(Prog::CrossEntropyG, LAYOUT_NN, false, g, e, s), "cross_entropy_bwd: G"));
    }
    {  // dh = s G W^T (bf16 at once with one slice, else accumulated in fp32)
      EpiArgs e = epi0();
      e.alpha_dev = scale;
      GemmArgs g = gemm_args(G, ldG, Wp + v0, W->w.ld, M, D, nv);
      if (vc == V) {
        e.out = dh->ptr; e.ld_out = dh->ld;
        TRY(launched(launch_gemm(Prog::StoreAlphaDev, LAYOUT_NT, false, g, e, s), "cross_entropy_bwd: dh"));
      } else {
        e.out = dh_acc; e.ld_out = D;
        e.beta = v0 == 0 ? 0.0f : 1.0f;
        TRY(launched(launch_gemm(Prog::F32AlphaDev, LAYOUT_NT, false, g, e, s), "cross_entropy_bwd: dh"));
      }
    }
    {  // dW[:, v0 : v0 + nv] = beta dW + s h^T G
      EpiArgs e = epi0();
      e.out = static_cast<float*>(dW->ptr) + v0; e.ld_out = dW->ld;
      e.beta = beta;
      e.alpha_dev = scale;
      GemmArgs g = gemm_args(hp, h->ld, G, ldG, D, nv, M);
      TRY(launched(launch_gemm(Prog::F32AlphaDev, LAYOUT_TN, false, g, e, s), "cross_entropy_bwd: dW"));
    }
  }
  if (vc < V) {
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)((D / 4 + 255) / 256), row_grid(M)), dim3(256), 0, s,
                       dh_acc, D, static_cast<uint16_t*>(dh->ptr), dh->ld, (int)M, (int)D);
    TRY(check_launch("cross_entropy_bwd: dh"));
  }
  return CODA_OK;
}

// ======================================================================== final RMSNorm -> LM head -> CE
// The third GEMM-residual-RMSNorm-GEMM occurrence of the CODA paper
// (§3.2.1): the final norm's r is a row scale of the logits, its gain is
// folded into W_vocab (W~ = bf16(g W)), and the cross-entropy epilogues of
// coda_linear_cross_entropy run on z = r (y W~).
static size_t nce_fwd_layout(Carver& cv, int64_t M, int64_t V, bool need_sumsq, float** Pm, float** Ps, float** zy,
                             float** per_row, int** status, float** P1, float** r) {
  const int nT = (int)coda_partials_cols(V);
  *Pm = cv.take<float>((size_t)nT * M);
  *Ps = cv.take<float>((size_t)nT * M);
  *zy = cv.take<float>(M);
  *per_row = cv.take<float>(M);
  *status = cv.take<int>(M);
  (void)need_sumsq;
  *P1 = cv.take<float>(M);   // row sum of squares, or the merged partials
  *r = cv.take<float>(M);
  return cv.off;
}

extern "C" coda_status coda_linear_rmsnorm_cross_entropy_fwd_workspace(int64_t M, int64_t D, int64_t V,
                                                                       int32_t have_partials, int32_t precision,
                                                                       size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  (void)D;
  if (precision != CODA_PREC_BF16) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy: fp8 not compiled in this build");
  Carver cv(nullptr);
  float *a, *b, *c, *d, *e, *f;
  int* st;
  nce_fwd_layout(cv, M, V, !have_partials, &a, &b, &c, &d, &st, &e, &f);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_linear_rmsnorm_cross_entropy_fwd(
    const coda_mat* y, const coda_mat* sumsq_partials, const coda_weight* W, float eps, const coda_mat* labels,
    int32_t ignore_index, const coda_mat* loss, const coda_mat* lse, const coda_mat* per_row, const coda_mat* n_valid,
    const coda_mat* n_bad, const coda_mat* r_out, int32_t precision, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_precision(precision));
  if (precision != CODA_PREC_BF16) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy: fp8 not compiled in this build");
  TRY(check_mat(y, "y", CODA_BF16, -1, -1));
  const int64_t M = y->rows, D = y->cols;
  if (D == 0) return fail(CODA_ERR_SHAPE, "y: the normalised rows are empty (D = 0)");
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  const int64_t V = W->w.cols;
  TRY(check_weight(W, "W", D, V, precision));
  const coda_mat* P = sumsq_partials;
  if (present(P)) {
    TRY(check_mat(P, "sumsq_partials", CODA_F32, -1, M));
    if (P->rows < 1 || P->rows > 32 || P->ld != M)
      return fail(CODA_ERR_SHAPE, "sumsq_partials: 1..32 rows of M, ld == M");
  }
  TRY(check_vec(labels, "labels", CODA_I32, M));
  TRY(check_vec(loss, "loss", CODA_F32, 1));
  TRY(check_vec(lse, "lse", CODA_F32, M));
  TRY(check_vec(per_row, "per_row", CODA_F32, M, true));
  TRY(check_vec(n_valid, "n_valid", CODA_I32, 1));
  TRY(check_vec(n_bad, "n_bad", CODA_I32, 1, true));
  TRY(check_vec(r_out, "r_out", CODA_F32, M, true));
  if (ignore_index >= 0 && ignore_index < V) return fail(CODA_ERR_VALUE, "ignore_index must lie outside [0, V)");
  Carver cv(ws);
  float *Pm, *Ps, *zy, *pr, *P1, *rws;
  int* st;
  nce_fwd_layout(cv, M, V, !present(P), &Pm, &Ps, &zy, &pr, &st, &P1, &rws);
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  float* per = present(per_row) ? static_cast<float*>(per_row->ptr) : pr;
  if (M > 0) {
    const float* parts = present(P) ? static_cast<const float*>(P->ptr) : P1;
    const int nP = present(P) ? (int)P->rows : 1;
    if (!present(P)) {
      hipLaunchKernelGGL(row_sumsq_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s,
                         static_cast<const uint16_t*>(y->ptr), y->ld, (int)M, (int)D, P1);
      TRY(check_launch("rmsnorm_cross_entropy_fwd: sumsq"));
    }
    EpiArgs e = epi0();
    e.labels = static_cast<const int*>(labels->ptr);
    e.partial_out = Pm;
    e.partial_out2 = Ps;
    e.rowvec_out = zy;
    e.rowvec_out2 = present(r_out) ? static_cast<float*>(r_out->ptr) : rws;
    e.row_partials = parts;
    e.n_row_partials = nP;
    TRY(narrow_partials(&e.row_partials, &e.n_row_partials, M, P1, s));
    e.norm_dim = (int)D;
    e.eps = eps;
    e.vocab = (int)V;
    GemmArgs g = gemm_args(y->ptr, y->ld, W->w.ptr, W->w.ld, M, V, D);
    TRY(launched(launch_gemm(Prog::CrossEntropyNorm, LAYOUT_NN, false, g, e, s), "rmsnorm_cross_entropy_fwd: logits"));
    hipLaunchKernelGGL(ce_finish_rows_kernel, dim3((unsigned)((M + 63) / 64)), dim3(256), 0, s, Pm, Ps,
                       (int)coda_partials_cols(V), (int)M, zy, static_cast<const int*>(labels->ptr), (int)V,
                       ignore_index, static_cast<float*>(lse->ptr), per, st);
    TRY(check_launch("rmsnorm_cross_entropy_fwd: rows"));
  }
  hipLaunchKernelGGL(ce_finish_loss_kernel, dim3(1), dim3(1024), 0, s, per, st, (int)M, static_cast<float*>(loss->ptr),
                     static_cast<int*>(n_valid->ptr), present(n_bad) ? static_cast<int*>(n_bad->ptr) : nullptr);
  return check_launch("rmsnorm_cross_entropy_fwd: loss");
}

static size_t nce_bwd_layout(Carver& cv, int64_t M, int64_t D, int64_t V, int64_t vc, float** scale, uint16_t** G,
                             float** Tp, float** Tc, float** dgp, float** dy_acc) {
  *scale = cv.take<float>(1);
  *G = cv.take<uint16_t>((size_t)M * ((vc + 7) / 8 * 8));
  *Tp = cv.take<float>((size_t)coda_partials_cols(V) * M);
  *Tc = cv.take<float>(M);
  *dgp = cv.take<float>((size_t)coda_partials_cols(V) * D);
  *dy_acc = vc < V ? cv.take<float>((size_t)M * D) : nullptr;
  return cv.off;
}

extern "C" coda_status coda_linear_rmsnorm_cross_entropy_bwd_workspace(int64_t M, int64_t D, int64_t V,
                                                                       int64_t chunk_rows, int32_t precision,
                                                                       size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  if (precision != CODA_PREC_BF16) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy: fp8 not compiled in this build");
  Carver cv(nullptr);
  float *sc, *Tp, *Tc, *dgp, *acc;
  uint16_t* G;
  nce_bwd_layout(cv, M, D, V, ce_slice_cols(M, V, chunk_rows), &sc, &G, &Tp, &Tc, &dgp, &acc);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_linear_rmsnorm_cross_entropy_bwd(
    const coda_mat* y, const coda_mat* r, const coda_weight* W, const coda_mat* W_unfolded, const coda_mat* gvec,
    const coda_mat* labels, int32_t ignore_index, const coda_mat* lse, const coda_mat* n_valid, float dloss,
    const coda_mat* dres, const coda_mat* dy, const coda_mat* dW, const coda_mat* dg, float beta, int64_t chunk_rows,
    int32_t precision, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_precision(precision));
  if (precision != CODA_PREC_BF16) return fail(CODA_ERR_UNSUPPORTED, "cross_entropy: fp8 not compiled in this build");
  TRY(check_mat(y, "y", CODA_BF16, -1, -1));
  const int64_t M = y->rows, D = y->cols;
  if (D == 0) return fail(CODA_ERR_SHAPE, "y: the normalised rows are empty (D = 0)");
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  const int64_t V = W->w.cols;
  TRY(check_weight(W, "W", D, V, precision));
  TRY(check_mat(W_unfolded, "W_unfolded", CODA_BF16, D, V));
  TRY(check_vec(gvec, "g", CODA_F32, D));
  TRY(check_vec(r, "r", CODA_F32, M));
  TRY(check_vec(labels, "labels", CODA_I32, M));
  TRY(check_vec(lse, "lse", CODA_F32, M));
  TRY(check_vec(n_valid, "n_valid", CODA_I32, 1));
  TRY(check_mat(dres, "dres", CODA_BF16, M, D, true));
  TRY(check_mat(dy, "dy", CODA_BF16, M, D));
  TRY(check_mat(dW, "dW", CODA_F32, D, V));
  TRY(check_vec(dg, "dg", CODA_F32, D));
  if (ignore_index >= 0 && ignore_index < V) return fail(CODA_ERR_VALUE, "ignore_index must lie outside [0, V)");
  const int64_t vc = ce_slice_cols(M, V, chunk_rows);
  Carver cv(ws);
  float *scale, *Tp, *Tc, *dgp, *dy_acc;
  uint16_t* G;
  nce_bwd_layout(cv, M, D, V, vc, &scale, &G, &Tp, &Tc, &dgp, &dy_acc);
  TRY(ws_check(cv, ws_bytes, ws));
  if (M == 0) {
    TRY(scale_accum(dW, beta, S(stream), "rmsnorm_cross_entropy_bwd: dW of no tokens"));
    return scale_accum(dg, beta, S(stream), "rmsnorm_cross_entropy_bwd: dg of no tokens");
  }
  hipStream_t s = S(stream);
  const int64_t ldG = (vc + 7) / 8 * 8;
  const int nT = (int)coda_partials_cols(V);
  hipLaunchKernelGGL(ce_scale_kernel, dim3(1), dim3(1), 0, s, static_cast<const int*>(n_valid->ptr), dloss, scale);
  TRY(check_launch("rmsnorm_cross_entropy_bwd: scale"));
  const uint16_t* yp = static_cast<const uint16_t*>(y->ptr);
  const uint16_t* Wp = static_cast<const uint16_t*>(W->w.ptr);
  const uint16_t* Wu = static_cast<const uint16_t*>(W_unfolded->ptr);
  const int* lab = static_cast<const int*>(labels->ptr);
  const float* lsep = static_cast<const float*>(lse->ptr);
  const float* rp = static_cast<const float*>(r->ptr);
  const uint16_t* dresp = present(dres) ? static_cast<const uint16_t*>(dres->ptr) : nullptr;
  // One pass when the whole G~ fits: the dy GEMM then needs T complete first.
  // Over vocabulary slices (vc a multiple of the 256-column partial tiles),
  // each slice adds its share of s G~ W~^T into an fp32 [M, D] buffer and
  // writes its own columns of dW and its own T and gain partial columns; T
  // and the correction come after the last slice.
  for (int64_t v0 = 0; v0 < V; v0 += vc) {
    const int64_t nv = std::min(vc, V - v0);
    const int64_t pc = v0 / kBN;   // first partial column of the slice
    {  // recompute z = r (y W~) for the slice: G~ = bf16(r (p - onehot)), T partials
      EpiArgs e = epi0();
      e.out = G; e.ld_out = ldG;
      e.labels = lab;
      e.rowvec = lsep;
      e.rowvec2 = rp;
      e.col_offset = (int)v0;
      e.vocab = (int)V;
      e.partial_out = Tp + pc * M;
      GemmArgs g = gemm_args(yp, y->ld, Wp + v0, W->w.ld, M, nv, D);
      TRY(launched(launch_gemm(Prog::CrossEntropyGNorm, LAYOUT_NN, false, g, e, s), "rmsnorm_cross_entropy_bwd: G"));
    }
    if (vc == V) {
      hipLaunchKernelGGL(rows_finish_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, Tp, nT, (int)M, 0,
                         (const float*)nullptr, 0, 0.0f, Tc);
      TRY(check_launch("rmsnorm_cross_entropy_bwd: finish T"));
      // dy = s (G~ W~^T - (r T / D) y) + dres
      EpiArgs e = epi0();
      e.out = dy->ptr; e.ld_out = dy->ld;
      e.aux0 = yp; e.ld_aux0 = y->ld;
      if (dresp) { e.aux1 = dresp; e.ld_aux1 = dres->ld; }
      e.rowvec = rp;
      e.row_partials = Tc;
      e.n_row_partials = 1;
      e.norm_dim = (int)D;
      e.alpha_dev = scale;
      GemmArgs g = gemm_args(G, ldG, Wp, W->w.ld, M, D, V);
      TRY(launched(launch_gemm(Prog::NormCorr, LAYOUT_NT, false, g, e, s), "rmsnorm_cross_entropy_bwd: dy"));
    } else {  // dy_acc (+)= s G~ W~^T over the slice
      EpiArgs e = epi0();
      e.out = dy_acc; e.ld_out = D;
      e.beta = v0 == 0 ? 0.0f : 1.0f;
      e.alpha_dev = scale;
      GemmArgs g = gemm_args(G, ldG, Wp + v0, W->w.ld, M, D, nv);
      TRY(launched(launch_gemm(Prog::F32AlphaDev, LAYOUT_NT, false, g, e, s), "rmsnorm_cross_entropy_bwd: dy"));
    }
    {  // dW[:, v0 : v0 + nv] = beta dW + s g (y^T G~), gain partials s sum_v W (y^T G~)
      EpiArgs e = epi0();
      e.out = static_cast<float*>(dW->ptr) + v0; e.ld_out = dW->ld;
      e.beta = beta;
      e.aux0 = Wu + v0; e.ld_aux0 = W_unfolded->ld;
      e.rowvec = fptr(gvec);
      e.partial_out = dgp + pc * D;
      e.alpha_dev = scale;
      GemmArgs g = gemm_args(yp, y->ld, G, ldG, D, nv, M);
      TRY(launched(launch_gemm(Prog::WgradGain, LAYOUT_TN, false, g, e, s), "rmsnorm_cross_entropy_bwd: dW"));
    }
  }
  if (vc < V && M > 0) {
    // c = r T / D, then dy = dy_acc - s c y + dres
    hipLaunchKernelGGL(rows_finish_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, Tp, nT, (int)M, 2, rp,
                       (int)D, 0.0f, Tc);
    TRY(check_launch("rmsnorm_cross_entropy_bwd: finish T"));
    hipLaunchKernelGGL(norm_corr_finish_kernel, dim3((unsigned)((D / 4 + 255) / 256), row_grid(M)), dim3(256), 0, s,
                       dy_acc, D, yp, y->ld, Tc, scale, dresp, dresp ? dres->ld : 0, static_cast<uint16_t*>(dy->ptr),
                       dy->ld, (int)M, (int)D);
    TRY(check_launch("rmsnorm_cross_entropy_bwd: dy"));
  }
  return sum_partials_launch(dgp, nT, (int)D, beta, static_cast<float*>(dg->ptr), s);
}

// ======================================================================== RMSNorm -> Linear -> sigmoid | GELU
static coda_status map_fwd_check(const coda_mat* x, const coda_mat* P, const coda_weight* W, const coda_mat* out,
                                 const coda_mat* save, const coda_mat* r_out, int precision) {
  TRY(check_precision_fwd(precision));
  TRY(check_mat(x, "x", CODA_BF16, -1, -1));
  const int64_t M = x->rows, K = x->cols;
  if (K == 0) return fail(CODA_ERR_SHAPE, "x: the normalised rows are empty (K = 0)");
  if (!W) return fail(CODA_ERR_NULL, "W: NULL");
  const int64_t N = W->w.cols;
  TRY(check_weight(W, "W", K, N, precision));
  TRY(check_mat(P, "sumsq_partials", CODA_F32, -1, M, true));
  if (present(P) && (P->rows < 1 || P->rows > 32 || (P->rows > 1 && P->ld != M)))
    return fail(CODA_ERR_SHAPE, "sumsq_partials: 1..32 rows of M with ld == M");
  TRY(check_mat(out, "out", CODA_BF16, M, N));
  TRY(check_mat(save, "save_h", CODA_BF16, M, N, true));
  TRY(check_vec(r_out, "r_out", CODA_F32, M, true));
  return CODA_OK;
}

static coda_status map_fwd(const coda_mat* x, const coda_mat* P, const coda_weight* W, float eps, const coda_mat* out,
                           const coda_mat* save_h, const coda_mat* r_out, int32_t precision, void* ws,
                           size_t ws_bytes, void* stream, Act act) {
  TRY(map_fwd_check(x, P, W, out, save_h, r_out, precision));
  if (!(eps >= 0.0f)) return fail(CODA_ERR_VALUE, "eps must be >= 0");
  return swiglu_fwd_impl(x, P, W, eps, out, save_h, r_out, precision, ws, ws_bytes, stream, false, nullptr, act);
}

static coda_status map_bwd_workspace(int64_t M, int64_t D, int64_t N, int32_t precision, size_t* bytes, Act act) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  return swiglu_bwd_impl(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, 0.0f, nullptr, precision, nullptr, 0, nullptr, M, D, N, true, bytes, act);
}

static coda_status map_bwd(const coda_mat* dY, const coda_weight* Wn, const coda_mat* saved_h, const coda_mat* r,
                           const coda_mat* u, const coda_weight* W, const coda_mat* W_unfolded, const coda_mat* g,
                           const coda_mat* dres, const coda_mat* du, const coda_mat* dW, const coda_mat* dg, float beta,
                           const coda_mat* dh_out, int32_t precision, void* ws, size_t ws_bytes, void* stream,
                           Act act) {
  TRY(check_precision(precision));
  TRY(check_mat(dY, "dY", CODA_BF16, -1, -1));
  const int64_t M = dY->rows, D = dY->cols;
  if (D == 0) return fail(CODA_ERR_SHAPE, "u: the normalised rows are empty (D = 0)");
  if (!Wn || !W) return fail(CODA_ERR_NULL, "weights: NULL");
  const int64_t N = Wn->w.rows;
  TRY(check_weight(Wn, "Wn", N, D, precision));
  TRY(check_weight(W, "W", D, N, precision));
  TRY(check_mat(saved_h, "saved_h", CODA_BF16, M, N));
  TRY(check_vec(r, "r", CODA_F32, M));
  TRY(check_mat(u, "u", CODA_BF16, M, D));
  TRY(check_mat(W_unfolded, "W_unfolded", CODA_BF16, D, N));
  TRY(check_vec(g, "g", CODA_F32, D));
  TRY(check_mat(dres, "dres", CODA_BF16, M, D));
  TRY(check_mat(du, "du", CODA_BF16, M, D));
  TRY(check_mat(dW, "dW", CODA_F32, D, N));
  TRY(check_vec(dg, "dg", CODA_F32, D));
  TRY(check_mat(dh_out, "dh_out", CODA_BF16, M, N, true));
  return swiglu_bwd_impl(dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta, dh_out, precision, ws,
                         ws_bytes, stream, M, D, N, false, nullptr, act);
}

extern "C" coda_status coda_linear_sigmoid_fwd_workspace(int64_t M, int64_t K, int32_t have_partials,
                                                         int32_t precision, size_t* bytes) {
  return coda_linear_swiglu_fwd_workspace(M, K, have_partials, precision, bytes);
}

extern "C" coda_status coda_linear_sigmoid_fwd(const coda_mat* x, const coda_mat* sumsq_partials, const coda_weight* W,
                                               float eps, const coda_mat* out, const coda_mat* save_h,
                                               const coda_mat* r_out, int32_t precision, void* ws, size_t ws_bytes,
                                               void* stream) {
  return map_fwd(x, sumsq_partials, W, eps, out, save_h, r_out, precision, ws, ws_bytes, stream, Act::Sigmoid);
}

extern "C" coda_status coda_linear_sigmoid_bwd_workspace(int64_t M, int64_t D, int64_t N, int32_t precision,
                                                         size_t* bytes) {
  return map_bwd_workspace(M, D, N, precision, bytes, Act::Sigmoid);
}

extern "C" coda_status coda_linear_sigmoid_bwd(const coda_mat* dY, const coda_weight* Wn, const coda_mat* saved_h,
                                               const coda_mat* r, const coda_mat* u, const coda_weight* W,
                                               const coda_mat* W_unfolded, const coda_mat* g, const coda_mat* dres,
                                               const coda_mat* du, const coda_mat* dW, const coda_mat* dg, float beta,
                                               const coda_mat* dh_out, int32_t precision, void* ws, size_t ws_bytes,
                                               void* stream) {
  return map_bwd(dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta, dh_out, precision, ws, ws_bytes,
                 stream, Act::Sigmoid);
}

extern "C" coda_status coda_linear_gelu_fwd_workspace(int64_t M, int64_t K, int32_t have_partials, int32_t precision,
                                                      size_t* bytes) {
  return coda_linear_swiglu_fwd_workspace(M, K, have_partials, precision, bytes);
}

extern "C" coda_status coda_linear_gelu_fwd(const coda_mat* x, const coda_mat* sumsq_partials, const coda_weight* W,
                                            float eps, const coda_mat* out, const coda_mat* save_h,
                                            const coda_mat* r_out, int32_t precision, void* ws, size_t ws_bytes,
                                            void* stream) {
  return map_fwd(x, sumsq_partials, W, eps, out, save_h, r_out, precision, ws, ws_bytes, stream, Act::Gelu);
}

extern "C" coda_status coda_linear_gelu_bwd_workspace(int64_t M, int64_t D, int64_t N, int32_t precision,
                                                      size_t* bytes) {
  return map_bwd_workspace(M, D, N, precision, bytes, Act::Gelu);
}

extern "C" coda_status coda_linear_gelu_bwd(const coda_mat* dY, const coda_weight* Wn, const coda_mat* saved_h,
                                            const coda_mat* r, const coda_mat* u, const coda_weight* W,
                                            const coda_mat* W_unfolded, const coda_mat* g, const coda_mat* dres,
                                            const coda_mat* du, const coda_mat* dW, const coda_mat* dg, float beta,
                                            const coda_mat* dh_out, int32_t precision, void* ws, size_t ws_bytes,
                                            void* stream) {
  return map_bwd(dY, Wn, saved_h, r, u, W, W_unfolded, g, dres, du, dW, dg, beta, dh_out, precision, ws, ws_bytes,
                 stream, Act::Gelu);
}
