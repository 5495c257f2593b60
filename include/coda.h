/*
 * coda.h - C ABI of the MI355X (gfx950) GEMM+epilogue library.
 *
 * The method: the CODA paper "Rewriting Transformer Blocks as GEMM-Epilogue
 * Programs" (arXiv 2605.19269).  §2.2 splits a GEMM into a fixed mainloop and
 * a programmable epilogue that runs on each output tile while it is still on
 * chip; §3.1 lists five epilogue primitive classes (elementwise / pairwise
 * maps, rank-1 vector loads and stores, rank-2 tile loads and stores, tile
 * row reductions merged later, running state such as online log-sum-exp);
 * §3.2 writes the non-attention parts of a Transformer block as
 * GEMM + epilogue programs, and §3.2.1 gives the reparameterisation
 *     RMSNorm(x W0 + z, g) W1 = (r (x W0 + z) * g) W1,   r = 1 / rms(x W0 + z),
 * whose per-row factor r is applied behind the second GEMM (the "delayed r"
 * described in the KuCoin news summary of CODA, section on the epilogue).
 * The functional entry points follow the kernel-granular API named by the
 * papers.ananclaw.com CODA guide (section on the functional API):
 * linear_swiglu, linear_cross_entropy, linear_qknorm_rope, plus
 * linear_rmsnorm_residual for the O- and down-projections.
 *
 * Conventions for every entry point
 *  - Matrices are described by coda_mat: a DEVICE pointer, an element type,
 *    rows, cols and a leading dimension `ld` in elements (row-major: element
 *    (i, j) lives at ptr + i * ld + j).  Vectors are 1 x n coda_mats.
 *  - Weights are stored [K_in, N_out] row-major.
 *  - The caller owns all device memory (inputs, outputs, workspace).  The
 *    library never allocates, frees or synchronises; every call enqueues
 *    kernels on `stream` (a hipStream_t, NULL = default stream) and returns.
 *  - Validation (null pointers, dtypes, shapes, ld, 16-byte alignment,
 *    workspace size) runs on the host BEFORE any HIP call; a failed check
 *    returns a status code and leaves device memory untouched.
 *    coda_last_error() gives a human-readable message (thread-local).
 *  - A kernel launch failure returns CODA_ERR_LAUNCH.  Data errors that only
 *    the device can see (a label outside [0, V) that is not the ignore index)
 *    are reported through a device-side counter output.
 *  - Contiguous rows: bf16 matrices need cols % 8 == 0 and ld % 8 == 0,
 *    fp32 matrices cols % 4 == 0 and ld % 4 == 0, E4M3 matrices
 *    cols % 16 == 0 and ld % 16 == 0; every pointer 16-byte aligned.
 *    A matrix with more than one row needs a row stride (ld x element size)
 *    below 16 MiB: the kernels address a tile's rows by 32-bit offsets.
 *  - Results are bitwise deterministic: reductions run in a fixed order.
 *  - Empty token batches (M = 0 rows of activations) are valid: a forward
 *    call writes nothing, and a backward call applies D = beta D to its
 *    fp32 gradient accumulators (beta 0 clears them without reading them)
 *    and launches no GEMM.  A normalised row of width 0 (the K or D that an
 *    RMSNorm divides by) has no root mean square: CODA_ERR_SHAPE.
 */
#ifndef CODA_H_
#define CODA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CODA_ABI_VERSION 2

typedef enum coda_status {
  CODA_OK = 0,
  CODA_ERR_NULL = 1,        /* a required pointer is NULL */
  CODA_ERR_DTYPE = 2,       /* wrong element type */
  CODA_ERR_SHAPE = 3,       /* inconsistent or unsupported sizes */
  CODA_ERR_LAYOUT = 4,      /* ld smaller than cols, or not a multiple of the vector width */
  CODA_ERR_ALIGN = 5,       /* pointer not 16-byte aligned */
  CODA_ERR_WORKSPACE = 6,   /* workspace missing or too small */
  CODA_ERR_UNSUPPORTED = 7, /* epilogue program or option not compiled in */
  CODA_ERR_LAUNCH = 8,      /* a kernel launch failed */
  CODA_ERR_VALUE = 9        /* an invalid scalar argument */
} coda_status;

/* CODA_E8M0: one byte 2^(code - 127) (code 255 = NaN, never written here),
 * the shared block scale of the OCP Microscaling (MX) formats.
 * CODA_E2M1X2: two FP4 E2M1 codes a byte (the MX specification's FP4
 * element: sign, 2 exponent bits with bias 1, 1 mantissa bit; values 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6), element 2i in the low nibble of byte i; a matrix of
 * them counts cols and ld in bytes.
 * CODA_E2M3 / CODA_E3M2: the MX specification's FP6 elements (sign, 2
 * exponent bits with bias 1 and 3 mantissa bits, largest 7.5; or 3 exponent
 * bits with bias 3 and 2 mantissa bits, largest 28).  Each block of 32
 * consecutive values of a row is 32 bytes: the 32 six-bit codes packed into
 * the first 24 (code v at bits [6 v, 6 v + 6) of the block read as one
 * little-endian 192-bit number), then 8 zero bytes; a matrix of them counts
 * cols and ld in bytes, which equal values. */
typedef enum coda_dtype {
  CODA_BF16 = 1, CODA_F32 = 2, CODA_E4M3 = 3, CODA_I32 = 4, CODA_E8M0 = 5, CODA_E2M1X2 = 6,
  CODA_E2M3 = 7, CODA_E3M2 = 8
} coda_dtype;

/* GEMM operand precision of the functional entry points. */
typedef enum coda_precision {
  CODA_PREC_BF16 = 0, /* bf16 operands, fp32 accumulate */
  CODA_PREC_FP8 = 1,  /* OCP E4M3 operands with amax scales, fp32 accumulate */
  CODA_PREC_MXFP8 = 2, /* E4M3 operands with one E8M0 scale per 32 values of the
                          contracted axis (OCP MX), fp32 accumulate; every
                          contracted size (hidden, MLP width, tokens of a
                          backward) a multiple of 128 */
  CODA_PREC_MXFP4 = 3, /* E2M1 operands (two a byte) with one E8M0 scale per 32
                          values of the contracted axis, fp32 accumulate; the
                          forward entry points need w, q_fwd (E2M1X2 [N, K/2])
                          and s_fwd (word layout), the backward ones also
                          q_bwd (E2M1X2 [K, N/2]) and s_bwd (blocks along
                          N_out); every contracted size a multiple of 128;
                          the cross-entropy entry points refuse it */
  CODA_PREC_MXFP6_E2M3 = 4, /* FP6 E2M3 operands (CODA_E2M3, a byte a value with
                               the block padding) under the same exponents;
                               q_fwd [N, K] and q_bwd [K, N] of dtype
                               CODA_E2M3, otherwise as MXFP4 */
  CODA_PREC_MXFP6_E3M2 = 5  /* the same with FP6 E3M2 operands (CODA_E3M2) */
} coda_precision;

typedef struct coda_mat {
  void* ptr;       /* device pointer (NULL = absent where optional) */
  int32_t dtype;   /* coda_dtype */
  int32_t reserved;
  int64_t rows, cols, ld;
} coda_mat;

/* A weight W [K_in, N_out] and, for fp8 precision, its two E4M3 copies made
 * by coda_quantize_weight: q_fwd [N_out, K_in] with one scale per output
 * channel (forward GEMM, contracted axis K_in contiguous) and q_bwd
 * [K_in, N_out] with one scale per input channel (input-gradient GEMM).
 * For MXFP8 precision the same two copies carry E8M0 block exponents in
 * word layout instead (see coda_quantize_mxfp8): s_fwd [K_in / 128,
 * 4 N_out] (blocks along K_in) and s_bwd [N_out / 128, 4 K_in] (blocks
 * along N_out); coda_quantize_weight makes them when s_fwd has dtype E8M0.
 * bf16 precision reads only `w`. */
typedef struct coda_weight {
  coda_mat w;
  coda_mat q_fwd, s_fwd;
  coda_mat q_bwd, s_bwd;
} coda_weight;

int coda_abi_version(void);
const char* coda_status_string(int status);
const char* coda_last_error(void);

/* Launch schedule of the bf16 gate/up GEMM with the SwiGLU epilogue (the
 * generic entry point's SwiGLU chain on NN operands and the bf16
 * coda_linear_swiglu_fwd).  The CODA paper (arXiv 2605.19269), §1, hides a
 * tile's epilogue under other tiles' mainloops (ping-pong warp groups,
 * tensor memory); the co-resident schedule is that overlap on this chip:
 *   CODA_SCHED_PINGPONG   (default) one 256 x 256 tile a workgroup, two
 *                         8-wave groups alternating copies and matrix work,
 *                         one workgroup a compute unit; every tile's
 *                         epilogue runs after its own mainloop.
 *   CODA_SCHED_CORESIDENT 128 x 256 tiles, 4-wave workgroups, three LDS
 *                         stages, two workgroups a compute unit, so one's
 *                         epilogue and stores overlap the other's matrix
 *                         instructions.  Same results up to the order of
 *                         fp32 sums; slower on this chip (the smaller tile
 *                         copies 1.5 times the operand bytes a flop).
 * The setting is process-wide and read at each launch; changing it while
 * another thread launches is a race.  CODA_ERR_VALUE for an unknown value. */
typedef enum coda_schedule {
  CODA_SCHED_PINGPONG = 0,
  CODA_SCHED_CORESIDENT = 1
} coda_schedule;
coda_status coda_set_schedule(int32_t schedule);
int32_t coda_get_schedule(void);

/* ===================================================================== prep */

/* W_out[k, n] = bf16(g[k] * W[k, n]): the RMSNorm gain folded into the weight
 * of the GEMM that consumes the norm (the §3.2.1 identity with g moved onto
 * W1).  W, W_out: bf16 [K, N] (may alias); g: fp32 1 x K. */
coda_status coda_fold_gain(const coda_mat* W, const coda_mat* g, const coda_mat* W_out, void* stream);

/* Packs the gate and up weights [K, F] into W_gu [K, 2F]: each 64-column
 * block holds 32 gate columns then the matching 32 up columns, so one lane
 * of the SwiGLU epilogue holds gate_f and up_f.  g (fp32 1 x K) is folded
 * when non-NULL.  F % 32 == 0. */
coda_status coda_pack_gate_up(const coda_mat* Wg, const coda_mat* Wu, const coda_mat* g_or_null,
                              const coda_mat* Wgu_out, void* stream);

/* RoPE table [seq_len, head_dim/2, 2] fp32 (out is seq_len x head_dim):
 * (cos, sin) of p * theta^(-2i/head_dim), angles in float64.  head_dim = 128. */
coda_status coda_rope_table(int32_t seq_len, int32_t head_dim, double theta, const coda_mat* out,
                            void* stream);

/* out[m] = sum_k x[m, k]^2 (fp32 1 x M): one row partial, usable wherever an
 * entry point takes sum-of-squares partials (with n = 1). */
coda_status coda_row_sumsq(const coda_mat* x, const coda_mat* out, void* stream);

/* E4M3 quantisation of a bf16 matrix X [R, C] with the amax taken over the
 * contracted axis `axis`:
 *   axis = 1: Q [R, C], scale fp32 1 x R   (Q = e4m3(clamp(X * 448/amax_r)))
 *   axis = 0: Q [C, R] (written transposed), scale fp32 1 x C
 * scale = amax / 448 (1 when amax = 0); dequantised value Q * scale.
 * Workspace (axis 0 only): coda_quantize_e4m3_workspace. */
coda_status coda_quantize_e4m3_workspace(const coda_mat* X, int32_t axis, size_t* bytes);
coda_status coda_quantize_e4m3(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* scale,
                               void* ws, size_t ws_bytes, void* stream);

/* Fills the quantised copies of wt->w that the precision of q_fwd / s_fwd
 * selects: E4M3 with fp32 scales (per output channel, Q transposed, and per
 * input channel), MXFP8 (E8M0 scales: blocks along K_in for q_fwd [N, K],
 * along N_out for q_bwd [K, N]) or MXFP4 (q_fwd of dtype CODA_E2M1X2: the same
 * blocks, two codes a byte; q_bwd is optional, NULL for a forward-only weight)
 * or MXFP6 (q_fwd of dtype CODA_E2M3 or CODA_E3M2: the same blocks in that
 * format, a byte a value; q_bwd optional as for MXFP4). */
coda_status coda_quantize_weight_workspace(const coda_weight* wt, size_t* bytes);
coda_status coda_quantize_weight(const coda_weight* wt, void* ws, size_t ws_bytes, void* stream);

/* ===================================================================== generic GEMM + epilogue */

/* The generic entry point: one GEMM whose output tile passes through an
 * epilogue program before (or instead of) its store.
 *
 * The CODA paper (§3.1) builds every epilogue from five primitive classes:
 *   P1 elementwise and pairwise maps, P2 rank-1 vector loads and stores,
 *   P3 rank-2 tile loads and stores, P4 tile row reductions written as
 *   partials and merged later, P5 running state (online log-sum-exp);
 * §2.2 confines an epilogue to its tile, its accumulator and auxiliaries
 * indexed like it.  A program is an ordered chain of such primitives.  The
 * library compiles a fixed set of chains (each one instantiation of the
 * fixed mainloop with a fused epilogue, no run-time code generation), checks
 * a program against that set op by op before any HIP call, and returns
 * CODA_ERR_UNSUPPORTED for any other chain or for a chain not compiled for
 * the given operand layout or type.
 *
 * An op names its primitive, up to three operands by index into the `aux`
 * array (slot, slot2, slot3; unused ones are ignored) and one float
 * parameter.  M, N, K are the product's sizes; tiles_n = ceil(N / 256)
 * (coda_partials_cols(N)); a partials operand [n, M] is fp32 with ld == M.
 *
 *   op                     class  operands                                   meaning
 *   STORE_BF16             P3     -                                          store the tile in bf16 to D
 *   ACCUM_F32              P3     fparam = beta                              D (fp32) = beta D + value
 *   ROW_SCALE              P2     slot: fp32 1 x M (r)                       value *= r[m]
 *   COL_SCALE              P2     slot: fp32 1 x N                           value *= c[n]
 *   ADD_TILE               P3     slot: bf16 [M, N]                          value += Z[m, n]
 *   ROW_SUMSQ_PARTIAL      P4     slot: partials [tiles_n, M]                sum over the tile's columns of bf16(stored)^2
 *   SWIGLU                 P1     -                                          SiLU(gate) * up over packed column pairs
 *   ROW_RMS_FROM_PARTIALS  P2+P4  slot: partials [n, M] (n <= 32);           r = (sum_t P[t, m] / K + eps)^-1/2 finished in
 *                                 fparam = eps                               the prologue (n > 8: merged in the workspace);
 *                                                                            value *= r[m]
 *   STORE_ROW_VEC          P2     slot: fp32 1 x M                           store the row factor r just finished or given
 *   SAVE_PRE               P3     slot: bf16 tile                            store the values as they stand (pre-activation)
 *   QKNORM_ROPE            P1     slot: fp32 [2, 128] gains (q, k);          per 128-column head of the q and k thirds:
 *                                 slot2: fp32 [seq_len, 128] RoPE table      RMSNorm (eps, gain), then rotation of the
 *                                 (coda_rope_table); fparam = eps            adjacent pairs at position m mod seq_len
 *   DSWIGLU                P3+P1  slot: bf16 [M, 2N] saved gate/up (packed)  dhg = da hu s (1 + hg (1 - s)), dhu = da hg s,
 *                                                                            s = sigmoid(hg); D [M, 2N] packed
 *   ROW_DOT_PARTIAL        P4     slot: partials [tiles_n, M]                sum over the tile of stored * the map's input
 *                                                                            (the saved pre-activation, or the logit)
 *   NORM_CORRECTION        P2+P3  slot: bf16 u [M, N]; slot2: fp32 r 1 x M; value = acc - (r[m] T[m] / N) u[m, n],
 *                                 slot3: partials T [n, M] (n <= 32)         T = sum_t P[t, m] (RMSNorm backward)
 *   WGRAD_GAIN             P2+P3+ slot: bf16 W [M, N] (unfolded weight);     D (fp32) = beta D + g[m] value,
 *                          P4     slot2: fp32 g 1 x M; slot3: partials       P[tn, m] = sum over the tile of W value
 *                                 [tiles_n, M]; fparam = beta                (the folded gain's gradient)
 *   CE_LSE_PARTIAL         P5     slot: int32 labels 1 x M; slot2: partials  per (N tile, row): max and sum of exp(z - max)
 *                                 [2 tiles_n, M] (max rows, then sum rows);  over the columns < N, and the logit of
 *                                 slot3: fp32 1 x M label logit              column labels[m] gathered; nothing stored to D
 *   CE_GRAD                P1     slot: int32 labels 1 x M; slot2: fp32      value = exp(z - lse[m]) - [n == labels[m]] on
 *                                 lse 1 x M                                  rows with a label in [0, N), else 0
 *   SIGMOID                P1     -                                          value = sigmoid(value)
 *   DSIGMOID               P3+P1  slot: bf16 [M, N] saved h                  value = da s (1 - s), s = sigmoid(h)
 *   GELU                   P1     -                                          value = GELU(value) = value Phi(value),
 *                                                                            Phi the normal CDF (erf form)
 *   DGELU                  P3+P1  slot: bf16 [M, N] saved h                  value = da (Phi(h) + h phi(h)), phi the
 *                                                                            normal density
 *   SCALE_DEV              P2     slot: fp32 1 x 1 device scalar             value *= s
 *   DEQUANT_E4M3           P2     slot: fp32 1 x M; slot2: fp32 1 x N        E4M3 operands: value = acc sA[m] sB[n]
 *
 * Compiled chains ([x] optional, a|b alternatives), and the operand forms
 * each is compiled for (bf16 layouts NN, NT, TN, TT as transA/transB; E4M3:
 * A [M, K], B [N, K] with DEQUANT_E4M3 as the program's first op; MX:
 * coda_gemm_mx):
 *   STORE_BF16                                              NN NT TN TT E4M3 MX
 *   ACCUM_F32                                               NN NT TN TT E4M3 MX
 *   ROW_SCALE COL_SCALE STORE_BF16                          NN MX
 *   ADD_TILE STORE_BF16 [ROW_SUMSQ_PARTIAL]                 NN E4M3 MX        residual + next-norm partials
 *   ROW_SCALE|ROW_RMS_FROM_PARTIALS [STORE_ROW_VEC] [SAVE_PRE] SWIGLU STORE_BF16
 *                                                           NN E4M3 MX        D [M, N/2], N % 64 == 0
 *   ROW_SCALE|ROW_RMS_FROM_PARTIALS [STORE_ROW_VEC] [SAVE_PRE] SIGMOID|GELU STORE_BF16
 *                                                           NN E4M3 MX
 *   ROW_SCALE|ROW_RMS_FROM_PARTIALS [STORE_ROW_VEC] [SAVE_PRE] QKNORM_ROPE STORE_BF16
 *                                                           NN E4M3 MX        D [M, N] = q | k | v, N % 384 == 0;
 *                                                                             SAVE_PRE [M, 2N/3] = q | k before the norm
 *   DSWIGLU ROW_SCALE STORE_BF16 ROW_DOT_PARTIAL            NT E4M3 MX        N % 32 == 0
 *   DSIGMOID|DGELU ROW_SCALE STORE_BF16 ROW_DOT_PARTIAL     NT E4M3 MX
 *   NORM_CORRECTION [SCALE_DEV] [ADD_TILE] STORE_BF16       NT E4M3 MX        value = s (acc - c u) + Z
 *   [SCALE_DEV] WGRAD_GAIN                                  TN E4M3 MX        s scales D's new term and P
 *   ROW_RMS_FROM_PARTIALS [STORE_ROW_VEC] CE_LSE_PARTIAL    NN                z = r acc (final norm folded)
 *   CE_LSE_PARTIAL                                          NN E4M3
 *   CE_GRAD STORE_BF16                                      NN E4M3
 *   ROW_SCALE CE_GRAD STORE_BF16 ROW_DOT_PARTIAL            NN                z = r acc, stored r (p - onehot),
 *                                                                             T = sum stored * z
 *   SCALE_DEV STORE_BF16                                    NT E4M3
 *   SCALE_DEV ACCUM_F32                                     NT TN E4M3
 * In a chain with ROW_RMS_FROM_PARTIALS and QKNORM_ROPE both eps must be
 * equal (one eps per epilogue).  Errors: CODA_ERR_UNSUPPORTED (chain or
 * form not compiled), CODA_ERR_SHAPE / DTYPE / LAYOUT / ALIGN on an operand,
 * CODA_ERR_VALUE on a parameter, CODA_ERR_WORKSPACE when the workspace is
 * smaller than coda_gemm_epi_workspace asks. */
typedef enum coda_epi_opcode {
  CODA_EPI_STORE_BF16 = 1,
  CODA_EPI_ACCUM_F32 = 2,
  CODA_EPI_ROW_SCALE = 3,
  CODA_EPI_COL_SCALE = 4,
  CODA_EPI_ADD_TILE = 5,
  CODA_EPI_ROW_SUMSQ_PARTIAL = 6,
  CODA_EPI_SWIGLU = 7,
  CODA_EPI_ROW_RMS_FROM_PARTIALS = 8,
  CODA_EPI_STORE_ROW_VEC = 9,
  CODA_EPI_SAVE_PRE = 10,
  CODA_EPI_QKNORM_ROPE = 11,
  CODA_EPI_DSWIGLU = 12,
  CODA_EPI_ROW_DOT_PARTIAL = 13,
  CODA_EPI_NORM_CORRECTION = 14,
  CODA_EPI_WGRAD_GAIN = 15,
  CODA_EPI_CE_LSE_PARTIAL = 16,
  CODA_EPI_CE_GRAD = 17,
  CODA_EPI_SIGMOID = 18,
  CODA_EPI_DSIGMOID = 19,
  CODA_EPI_SCALE_DEV = 20,
  CODA_EPI_DEQUANT_E4M3 = 21,
  CODA_EPI_GELU = 22,
  CODA_EPI_DGELU = 23
} coda_epi_opcode;

typedef struct coda_epi_op {
  uint16_t op;     /* coda_epi_opcode */
  uint16_t slot;   /* first aux operand */
  uint16_t slot2;  /* second aux operand */
  uint16_t slot3;  /* third aux operand */
  float fparam;
} coda_epi_op;

#define CODA_MAX_EPI_OPS 8
typedef struct coda_epi_program {
  uint32_t n_ops;
  coda_epi_op ops[CODA_MAX_EPI_OPS];
} coda_epi_program;

/* Number of N tiles (partial rows) an epilogue reduction writes for N columns. */
int64_t coda_partials_cols(int64_t N);

/* Workspace bytes coda_gemm_epi and coda_gemm_mx need for `prog` at M x N
 * x K: room to merge more than 8 partial rows (ROW_RMS_FROM_PARTIALS,
 * NORM_CORRECTION) to one before the GEMM; 0 for other chains.
 * CODA_ERR_UNSUPPORTED for a chain outside the compiled set. */
coda_status coda_gemm_epi_workspace(const coda_epi_program* prog, int64_t M, int64_t N, int64_t K, size_t* bytes);

/* D = epilogue(op(A) op(B)).  A: bf16 [M, K] (transA 0) or [K, M] (transA
 * 1), or E4M3 [M, K] when the program starts with DEQUANT_E4M3; B: bf16
 * [K, N] (transB 0) or [N, K] (transB 1), or E4M3 [N, K].  D as the chain
 * says (NULL for CE_LSE_PARTIAL chains).  aux: the operands the ops name.
 * ws: caller-owned device workspace of at least coda_gemm_epi_workspace
 * bytes (256-byte aligned; NULL when 0).  Asynchronous on `stream`. */
coda_status coda_gemm_epi(const coda_epi_program* prog, const coda_mat* A, int32_t transA,
                          const coda_mat* B, int32_t transB, const coda_mat* D,
                          const coda_mat* aux, uint32_t n_aux, void* ws, size_t ws_bytes, void* stream);

/* ===================================================================== MXFP8 block-scaled operands */

/* The CODA paper (§1) names the move of GEMM operands to 8- and 4-bit types
 * as one reason epilogue work grows in relative cost; gfx950's scaled MFMA
 * takes the block-scaled form of the OCP Microscaling Formats (MX) v1.0
 * specification, MXFP8 with E4M3 elements: every block of 32 consecutive
 * values along the contracted axis shares one E8M0 scale 2^e, and the
 * value the block stands for is 2^e * E4M3 element.
 *
 * Exponent layout ("word layout").  The exponents of an operand with n rows
 * and a contracted axis of L values form an E8M0 matrix S of
 * ceil(L / 128) x 4n bytes: word row g holds one 4-byte word per operand
 * row r, whose bytes j = 0..3 are the exponents of blocks 4 g + j (values
 * 128 g + 32 j .. 128 g + 32 j + 31) of row r:  S[g, 4 r + j].  The words of
 * consecutive rows are contiguous, so the GEMM copies the exponents of 64
 * rows for 128 K values with one 256-byte read.  S needs a 4-byte aligned
 * pointer and ld % 4 == 0 (it may be a uint8 tensor).  S byte = e + 127.
 *
 * Quantiser.  X: bf16 [R, C].  For each block with absolute max a:
 *   e = floor(log2 a) - 8, clamped to [-127, 127] (-127 when a is 0 or an
 *   fp32 subnormal);  element = E4M3(x / 2^e), round to nearest even,
 *   saturated at +-448.
 *   axis = 1: blocks along C:  Q E4M3 [R, C], S of R rows and L = C;  C % 32 == 0
 *   axis = 0: blocks along R, written transposed (the contracted axis
 *             contiguous):     Q E4M3 [C, R], S of C rows and L = R;  R % 32 == 0
 * When L is not a multiple of 128 the bytes of the last word row past the
 * last block are not written.  Q follows the E4M3 rules above.  No
 * workspace.  Errors: CODA_ERR_SHAPE when the blocked axis is not a
 * multiple of 32 or S is not ceil(L / 128) x 4n. */
coda_status coda_quantize_mxfp8(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* S,
                                void* stream);

/* MXFP4 copy of X (bf16 [R, C]), OCP MX v1.0 FP4: blocks of 32 values along
 * the contracted axis share the E8M0 exponent e = floor(log2 max|v|) - 2
 * (2 = the exponent of E2M1's largest power of two, 6 = 1.5 * 2^2), clamped
 * to [-127, 127] (-127 for an all-zero block); an element is the nearest
 * E2M1 value to v / 2^e, ties to the even mantissa, saturated at +-6; a
 * value that rounds to zero is stored as code 0 (+0).
 *   axis 1: Q [R, C / 2] (E2M1X2), exponents of R rows (C % 32 == 0);
 *   axis 0: Q [C, R / 2] (E2M1X2, written transposed), exponents of C rows
 *           (R % 32 == 0).
 * S: E8M0 in word layout as for coda_quantize_mxfp8, [ceil(L / 128), 4 rows].
 * Errors: CODA_ERR_SHAPE when the blocked axis is not a multiple of 32 or a
 * shape does not match; CODA_ERR_LAYOUT / CODA_ERR_ALIGN as for matrices. */
coda_status coda_quantize_mxfp4(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* S,
                                void* stream);

/* MXFP6 copy of X (bf16 [R, C]), OCP MX v1.0 FP6 with the element format
 * Q's dtype names (CODA_E2M3 or CODA_E3M2): blocks of 32 values along the
 * contracted axis share the E8M0 exponent e = floor(log2 max|v|) - emax
 * (emax = 2 for E2M3, 4 for E3M2: the exponent of the format's largest
 * power of two), clamped to [-127, 127] (-127 for an all-zero block); an
 * element is the nearest FP6 value to v / 2^e, ties to the even mantissa,
 * saturated at the largest (7.5 or 28); a value that rounds to zero is code
 * 0 (+0).  Blocks are packed as the dtype comment above says.
 *   axis 1: Q [R, C], exponents of R rows (C % 32 == 0);
 *   axis 0: Q [C, R] (written transposed), exponents of C rows (R % 32 == 0).
 * S: E8M0 in word layout as for coda_quantize_mxfp8, [ceil(L / 128), 4 rows].
 * Errors: CODA_ERR_DTYPE when Q is neither FP6 dtype; otherwise as
 * coda_quantize_mxfp4. */
coda_status coda_quantize_mxfp6(const coda_mat* X, int32_t axis, const coda_mat* Q, const coda_mat* S,
                                void* stream);

/* D = epilogue(sum_k A~[m, k] B~[n, k]) with MXFP8 operands
 *   A~ = A (E4M3 [M, K]) scaled by SA (E8M0 [K / 128, 4 M], word layout),
 *   B~ = B (E4M3 [N, K], i.e. the second operand stored with K contiguous)
 *        scaled by SB (E8M0 [K / 128, 4 N], word layout);
 * products and sums in fp32 on the matrix cores, the block scales applied
 * by the scaled MFMA.  K must be a positive multiple of 128 (the exponents
 * of 128 K values travel as one 4-byte word).  The epilogue program is any
 * chain coda_gemm_epi compiles for MX operands (its table, column MX), with
 * D and the aux operands shaped as there, and the same workspace
 * (coda_gemm_epi_workspace).  Errors as coda_gemm_epi, plus CODA_ERR_DTYPE
 * / CODA_ERR_SHAPE / CODA_ERR_ALIGN / CODA_ERR_LAYOUT for the scale
 * matrices.
 * MXFP4: with A of dtype CODA_E2M1X2 the operands are E2M1 (as written by
 * coda_quantize_mxfp4), A [M, K / 2 bytes] and B [N, K / 2 bytes], same
 * exponent layout and K rule (K counts values), and every chain of the MX
 * column.
 * MXFP6: with A of dtype CODA_E2M3 or CODA_E3M2 (as written by
 * coda_quantize_mxfp6) the operands are FP6 of that format, A [M, K] and
 * B [N, K] in bytes, B of the same dtype (CODA_ERR_DTYPE otherwise), same
 * exponent layout and K rule, and every chain of the MX column. */
coda_status coda_gemm_mx(const coda_epi_program* prog, const coda_mat* A, const coda_mat* SA,
                         const coda_mat* B, const coda_mat* SB, const coda_mat* D, const coda_mat* aux,
                         uint32_t n_aux, void* ws, size_t ws_bytes, void* stream);

/* ===================================================================== functional: forward */

/* Precision of the functional entry points (forward and backward alike):
 *   CODA_PREC_BF16   bf16 GEMM operands;
 *   CODA_PREC_FP8    E4M3 operands, one amax scale per row of each operand's
 *                    non-contracted axis, applied by the epilogue; the weight
 *                    carries coda_quantize_weight's two per-channel copies;
 *   CODA_PREC_MXFP8  E4M3 operands, one E8M0 exponent per 32 values of the
 *                    contracted axis, applied by the scaled MFMA; the weight
 *                    carries the two block-scaled copies; every contracted
 *                    size must be a multiple of 128 (CODA_ERR_SHAPE otherwise);
 *   CODA_PREC_MXFP4  E2M1 operands under the same exponents; the weight
 *                    carries the forward copy and, for the backward entry
 *                    points, the input-gradient copy (a weight without it is
 *                    refused with CODA_ERR_NULL there);
 *   CODA_PREC_MXFP6_E2M3, CODA_PREC_MXFP6_E3M2  FP6 operands of that format
 *                    under the same exponents, every activation quantised in
 *                    the weight's format; weight copies as for MXFP4 with the
 *                    FP6 dtype (one byte a value).
 * Activations are quantised per call into the workspace (the *_workspace
 * queries size it for the given precision).  The cross-entropy entry points
 * take CODA_PREC_BF16 only (CODA_ERR_UNSUPPORTED otherwise). */

/* RMSNorm -> Linear -> SwiGLU (config-1 op and the block's gate/up GEMM).
 * Passages: the CODA paper §3.2.1 and Fig. 4 (the GEMM-residual-RMSNorm-GEMM
 * identity: the norm's per-row factor r moves behind the next GEMM as a row
 * scale, its gain folds into the weight) and §3.1 item 1 (a pairwise map, here
 * SiLU(gate) * up; the papers.ananclaw.com guide lists it as linear_swiglu):
 *   r = (sum_t P[t, m] / K + eps)^(-1/2),  h = r * (x W~_gu),
 *   out = SiLU(h_gate) * h_up
 * x: bf16 [M, K].  sumsq_partials: fp32 [n, M] sum-of-squares partials of x
 * (n <= 32) or NULL (the library computes them).  More than 8 partial rows
 * are first merged to one by a small kernel.  The workspace (always needed,
 * sized by the query; have_partials is accepted for compatibility and does
 * not change the size) holds that row.
 * Wgu: packed, gain-folded weight (coda_pack_gate_up).  out: bf16 [M, F].
 * save_hgu (bf16 [M, 2F], packed order) and r_out (fp32 1 x M) are optional
 * saves for the backward. */
coda_status coda_linear_swiglu_fwd_workspace(int64_t M, int64_t K, int32_t have_partials, int32_t precision,
                                             size_t* bytes);
coda_status coda_linear_swiglu_fwd(const coda_mat* x, const coda_mat* sumsq_partials, const coda_weight* Wgu,
                                   float eps, const coda_mat* out, const coda_mat* save_hgu,
                                   const coda_mat* r_out, int32_t precision, void* ws, size_t ws_bytes,
                                   void* stream);

/* Residual linear (O-projection, down-projection).  Passage: the CODA paper
 * §3.2.1 (the residual add is tile-local and the next norm's statistic is a
 * row reduction written as per-tile partials, §3.1 item 4; the guide's
 * linear_rmsnorm_residual): out = residual + a W, stored bf16, plus the
 * sum-of-squares partials of the stored out for the next RMSNorm
 * (fp32 [coda_partials_cols(N), M], optional). */
coda_status coda_linear_rmsnorm_residual_fwd_workspace(int64_t M, int64_t K, int64_t N, int32_t precision,
                                                       size_t* bytes);
coda_status coda_linear_rmsnorm_residual_fwd(const coda_mat* a, const coda_weight* W, const coda_mat* residual,
                                             const coda_mat* out, const coda_mat* sumsq_partials_out,
                                             int32_t precision, void* ws, size_t ws_bytes, void* stream);

/* QKV projection with the delayed RMSNorm factor, per-head QK-RMSNorm and
 * RoPE (MHA, head_dim 128, D = heads * 128).  Passages: the CODA paper
 * §3.2.1 (delayed r) and §3.1 item 1 (pairwise maps: the RoPE rotation of
 * adjacent column pairs); the guide lists it as linear_qknorm_rope:
 *   h = r1 * (x W~_qkv) [M, 3D];  q = RoPE(QKnorm(h_q; gq)), k likewise, v = h_v
 * positions p = m mod seq_len.  rope: coda_rope_table output.  Optional
 * saves: qk_pre bf16 [M, 2D] (pre-norm q | k), r_out fp32 1 x M.
 * sumsq_partials and the workspace as in coda_linear_swiglu_fwd. */
coda_status coda_linear_qknorm_rope_fwd_workspace(int64_t M, int64_t D, int32_t have_partials,
                                                  int32_t precision, size_t* bytes);
coda_status coda_linear_qknorm_rope_fwd(const coda_mat* x, const coda_mat* sumsq_partials,
                                        const coda_weight* Wqkv, const coda_mat* gq, const coda_mat* gk,
                                        const coda_mat* rope, int32_t seq_len, float eps, const coda_mat* q,
                                        const coda_mat* k, const coda_mat* v, const coda_mat* save_qk_pre,
                                        const coda_mat* r_out, int32_t precision, void* ws, size_t ws_bytes,
                                        void* stream);

/* ===================================================================== functional: backward */

/* Backward of RMSNorm -> gate/up Linear -> SwiGLU, fused behind the GEMM
 * that produces the SwiGLU output gradient da = dY Wd^T (never materialised).
 * Passages: the CODA paper §3.2 (a tile-local forward keeps the
 * GEMM-epilogue form in the backward) and the KuCoin news summary's results
 * section (the SwiGLU backward among the fused kernels); the formulas are
 * the analytic gradients of the reparameterised forward:
 *   dSwiGLU with the saved (packed) hg/hu, dh~ = bf16(r * [dhg, dhu]),
 *   T = sum_j dh~ h,  c = r T / D,
 *   du = dh~ W~_gu^T - c u + dres          (bf16 [M, D]; dres optional)
 *   dW_gu = beta dW_gu + g * (u^T dh~)     (fp32 [D, 2F], packed order)
 *   dg = beta dg + sum_n W_gu * (u^T dh~)  (fp32 1 x D)
 * Wd: down weight [F, D]; Wgu: folded packed weight; Wgu_unfolded: the same
 * packing without the gain; u: the norm input (h1).  dh_gu_out: optional
 * bf16 [M, 2F] copy of dh~ (else held in the workspace). */
coda_status coda_linear_swiglu_bwd_workspace(int64_t M, int64_t D, int64_t F, int32_t precision,
                                             size_t* bytes);
coda_status coda_linear_swiglu_bwd(const coda_mat* dY, const coda_weight* Wd, const coda_mat* saved_hgu,
                                   const coda_mat* r, const coda_mat* u, const coda_weight* Wgu,
                                   const coda_mat* Wgu_unfolded, const coda_mat* g, const coda_mat* dres,
                                   const coda_mat* du, const coda_mat* dWgu, const coda_mat* dg, float beta,
                                   const coda_mat* dh_gu_out, int32_t precision, void* ws, size_t ws_bytes,
                                   void* stream);

/* Backward of a residual linear out = residual + a W (the CODA paper §3.2;
 * the fp32 weight-gradient accumulation is an epilogue store, §3.1 item 3):
 *   dW = beta dW + a^T d_out (fp32 [K, N]);  da = d_out W^T (bf16 [M, K], optional). */
coda_status coda_linear_rmsnorm_residual_bwd_workspace(int64_t M, int64_t K, int64_t N, int32_t precision,
                                                       size_t* bytes);
coda_status coda_linear_rmsnorm_residual_bwd(const coda_mat* d_out, const coda_mat* a, const coda_weight* W,
                                             const coda_mat* da, const coda_mat* dW, float beta,
                                             int32_t precision, void* ws, size_t ws_bytes, void* stream);

/* Backward of the QKV projection with QK-norm and RoPE (the CODA paper §3.2
 * and §3.2.1, as for coda_linear_swiglu_bwd), given the attention gradients
 * dq, dk (of the rotated q, k) and dv:
 *   inverse RoPE, per-head RMSNorm backward from the saved pre-norm q, k,
 *   dh~ = bf16(r1 [dq_pre, dk_pre, dv]),  T = sum_j dh~ h,  c = r1 T / D,
 *   dx = dh~ W~^T - c x + dres (bf16 [M, D]),
 *   dW = beta dW + g1 * (x^T dh~) (fp32 [D, 3D]),  dg1 = beta dg1 + sum_n W * (x^T dh~),
 *   dgq, dgk = beta dg + per-head gain gradients (fp32 1 x 128).
 * dh_qkv_out: optional bf16 [M, 3D] that receives dh~ (else it is held in
 * the workspace). */
coda_status coda_linear_qknorm_rope_bwd_workspace(int64_t M, int64_t D, int32_t precision, size_t* bytes);
coda_status coda_linear_qknorm_rope_bwd(const coda_mat* dq, const coda_mat* dk, const coda_mat* dv,
                                        const coda_mat* x, const coda_mat* r, const coda_mat* qk_pre,
                                        const coda_mat* v, const coda_weight* Wqkv, const coda_mat* Wqkv_unfolded,
                                        const coda_mat* g, const coda_mat* gq, const coda_mat* gk,
                                        const coda_mat* rope, int32_t seq_len, float eps, const coda_mat* dres,
                                        const coda_mat* dx, const coda_mat* dW, const coda_mat* dg,
                                        const coda_mat* dgq, const coda_mat* dgk, float beta,
                                        const coda_mat* dh_qkv_out, int32_t precision, void* ws, size_t ws_bytes,
                                        void* stream);

/* ===================================================================== cross-entropy */

/* Linear + cross-entropy forward without materialising the logits (the
 * running-state primitive of the CODA paper, §3.1 item 5: an online
 * log-sum-exp carried across N tiles, finished by a light merge step):
 *   z = h W (per N tile: online max / sum-exp partials, label-logit gather),
 *   lse[m], per-row loss, loss = sum_valid / n_valid (NaN if n_valid = 0).
 * h: bf16 [M, D]; W: [D, V]; labels: int32 1 x M.  A row is valid when its
 * label lies in [0, V); rows whose label equals ignore_index (which must lie
 * outside [0, V), else CODA_ERR_VALUE) are skipped, and any other label
 * outside [0, V) is a data error: the row is skipped too and counted in
 * n_bad.  Outputs: loss fp32 1 x 1, lse fp32 1 x M, per_row fp32 1 x M
 * (optional, 0 on skipped rows), n_valid int32 1 x 1 (required), n_bad int32
 * 1 x 1 (optional). */
coda_status coda_linear_cross_entropy_fwd_workspace(int64_t M, int64_t D, int64_t V, int32_t precision,
                                                    size_t* bytes);
coda_status coda_linear_cross_entropy_fwd(const coda_mat* h, const coda_weight* W, const coda_mat* labels,
                                          int32_t ignore_index, const coda_mat* loss, const coda_mat* lse,
                                          const coda_mat* per_row, const coda_mat* n_valid,
                                          const coda_mat* n_bad, int32_t precision, void* ws, size_t ws_bytes,
                                          void* stream);

/* The same forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument, bf16 operands only.  The partials live
 * in a library-owned device array of CODA_CE_FWD_NOALLOC_SCRATCH_BYTES, one
 * copy per GPU, held until the process ends; the call allocates nothing.
 * Shapes whose partials need more (2 ceil(V / 256) M + 3 M floats, about
 * 33 MB at M = 8192, V = 128256) return CODA_ERR_WORKSPACE.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (several
 * streams, several host threads) race and must be serialised by the
 * caller.  Arguments, outputs and errors otherwise as in
 * coda_linear_cross_entropy_fwd; the results are bitwise those of it. */
#define CODA_CE_FWD_NOALLOC_SCRATCH_BYTES (48u << 20)
coda_status coda_linear_cross_entropy_fwd_noalloc(const coda_mat* h, const coda_weight* W, const coda_mat* labels,
                                                  int32_t ignore_index, const coda_mat* loss, const coda_mat* lse,
                                                  const coda_mat* per_row, const coda_mat* n_valid,
                                                  const coda_mat* n_bad, void* stream);

/* Backward: recompute z, G = bf16(exp(z - lse) - onehot(label)) on valid
 * rows, exactly 0 on every row whose label lies outside [0, V) (ignored or
 * bad, as counted by the forward), s = dloss / n_valid,
 *   dh = bf16(s * G W^T) [M, D],  dW = beta dW + s * h^T G (fp32 [D, V]).
 * chunk_rows bounds the recomputed logits: 0 (or >= M) recomputes all M x V
 * at once; otherwise the buffer holds about chunk_rows x V values and the
 * recompute runs over vocabulary slices of that many values (a multiple of
 * 256 columns), each slice writing its own columns of dW, with dh summed in
 * fp32 over the slices and rounded to bf16 once (the workspace then also
 * holds an fp32 [M, D] buffer).  ignore_index must lie outside [0, V) as in
 * the forward. */
coda_status coda_linear_cross_entropy_bwd_workspace(int64_t M, int64_t D, int64_t V, int64_t chunk_rows,
                                                    int32_t precision, size_t* bytes);
coda_status coda_linear_cross_entropy_bwd(const coda_mat* h, const coda_weight* W, const coda_mat* labels,
                                          int32_t ignore_index, const coda_mat* lse, const coda_mat* n_valid,
                                          float dloss, const coda_mat* dh, const coda_mat* dW, float beta,
                                          int64_t chunk_rows, int32_t precision, void* ws, size_t ws_bytes,
                                          void* stream);

/* ===================================================================== RMSNorm -> Linear -> sigmoid */

/* The elementwise-map primitive of the CODA paper (§3.1 item 1) with the
 * delayed RMSNorm of §3.2.1, as in coda_linear_swiglu but with a sigmoid on
 * every column (the linear_sigmoid of the papers.ananclaw.com CODA guide):
 *   r = (sum_t P[t, m] / K + eps)^(-1/2),  h = r (x W~),  out = sigmoid(h)
 * x: bf16 [M, K]; W: the gain-folded weight [K, N]; out: bf16 [M, N];
 * save_h (bf16 [M, N]) and r_out (fp32 1 x M) are optional saves for the
 * backward.  Partials and workspace as in coda_linear_swiglu_fwd. */
coda_status coda_linear_sigmoid_fwd_workspace(int64_t M, int64_t K, int32_t have_partials, int32_t precision,
                                              size_t* bytes);
coda_status coda_linear_sigmoid_fwd(const coda_mat* x, const coda_mat* sumsq_partials, const coda_weight* W,
                                    float eps, const coda_mat* out, const coda_mat* save_h, const coda_mat* r_out,
                                    int32_t precision, void* ws, size_t ws_bytes, void* stream);

/* Backward fused behind the consumer GEMM da = dY Wn^T (Wn [N, D], never
 * materialising da): with s = sigmoid(saved h),
 *   dh~ = bf16(r da s (1 - s)),  T = sum_j dh~ h,  c = r T / D,
 *   du = dh~ W~^T - c u + dres (bf16 [M, D]),
 *   dW = beta dW + g (u^T dh~) (fp32 [D, N]),  dg = beta dg + sum_n W (u^T dh~).
 * Arguments as in coda_linear_swiglu_bwd with N in place of 2F. */
coda_status coda_linear_sigmoid_bwd_workspace(int64_t M, int64_t D, int64_t N, int32_t precision, size_t* bytes);
coda_status coda_linear_sigmoid_bwd(const coda_mat* dY, const coda_weight* Wn, const coda_mat* saved_h,
                                    const coda_mat* r, const coda_mat* u, const coda_weight* W,
                                    const coda_mat* W_unfolded, const coda_mat* g, const coda_mat* dres,
                                    const coda_mat* du, const coda_mat* dW, const coda_mat* dg, float beta,
                                    const coda_mat* dh_out, int32_t precision, void* ws, size_t ws_bytes,
                                    void* stream);

/* ===================================================================== RMSNorm -> Linear -> GELU */

/* The same layer with GELU as the elementwise map (the guide's linear_sigmoid
 * names one member of a family of activation epilogues; GELU is taken as the
 * second, in its exact form):
 *   r = (sum_t P[t, m] / K + eps)^(-1/2),  h = r (x W~),
 *   out = GELU(h) = h Phi(h),  Phi(h) = (1 + erf(h / sqrt 2)) / 2.
 * Arguments, shapes, precisions, workspace and errors as in
 * coda_linear_sigmoid_fwd. */
coda_status coda_linear_gelu_fwd_workspace(int64_t M, int64_t K, int32_t have_partials, int32_t precision,
                                           size_t* bytes);
coda_status coda_linear_gelu_fwd(const coda_mat* x, const coda_mat* sumsq_partials, const coda_weight* W,
                                 float eps, const coda_mat* out, const coda_mat* save_h, const coda_mat* r_out,
                                 int32_t precision, void* ws, size_t ws_bytes, void* stream);

/* Backward fused behind the consumer GEMM da = dY Wn^T, as
 * coda_linear_sigmoid_bwd with GELU'(h) = Phi(h) + h phi(h) (phi the normal
 * density) in place of s (1 - s):
 *   dh~ = bf16(r da GELU'(h)),  T = sum_j dh~ h,  c = r T / D,
 *   du = dh~ W~^T - c u + dres,  dW = beta dW + g (u^T dh~),
 *   dg = beta dg + sum_n W (u^T dh~).
 * Arguments as in coda_linear_sigmoid_bwd. */
coda_status coda_linear_gelu_bwd_workspace(int64_t M, int64_t D, int64_t N, int32_t precision, size_t* bytes);
coda_status coda_linear_gelu_bwd(const coda_mat* dY, const coda_weight* Wn, const coda_mat* saved_h,
                                 const coda_mat* r, const coda_mat* u, const coda_weight* W,
                                 const coda_mat* W_unfolded, const coda_mat* g, const coda_mat* dres,
                                 const coda_mat* du, const coda_mat* dW, const coda_mat* dg, float beta,
                                 const coda_mat* dh_out, int32_t precision, void* ws, size_t ws_bytes,
                                 void* stream);

/* ===================================================================== final RMSNorm -> LM head -> CE */

/* The third GEMM-residual-RMSNorm-GEMM occurrence of the CODA paper (§3.2.1,
 * final down-projection -> residual -> final RMSNorm -> LM head), fused with
 * the cross-entropy above:
 *   r = (sum_t P[t, m] / D + eps)^(-1/2),  z = r (y W~),  W~ = bf16(g W)
 *   (coda_fold_gain), then lse, per-row loss and the mean loss as in
 *   coda_linear_cross_entropy_fwd.
 * y: bf16 [M, D] (the final residual stream); sumsq_partials: fp32 [n, M]
 * (n <= 32) sum-of-squares partials of y (the last down-projection's
 * coda_linear_rmsnorm_residual_fwd output) or NULL (computed here).  More
 * than 8 partial rows are merged to one first, in the workspace.  W: the
 * folded weight [D, V].  r_out: optional fp32 1 x M
 * (needed by the backward).  Other outputs as in the plain cross-entropy.
 * bf16 only (fp8 returns CODA_ERR_UNSUPPORTED). */
coda_status coda_linear_rmsnorm_cross_entropy_fwd_workspace(int64_t M, int64_t D, int64_t V, int32_t have_partials,
                                                            int32_t precision, size_t* bytes);
coda_status coda_linear_rmsnorm_cross_entropy_fwd(const coda_mat* y, const coda_mat* sumsq_partials,
                                                  const coda_weight* W, float eps, const coda_mat* labels,
                                                  int32_t ignore_index, const coda_mat* loss, const coda_mat* lse,
                                                  const coda_mat* per_row, const coda_mat* n_valid,
                                                  const coda_mat* n_bad, const coda_mat* r_out, int32_t precision,
                                                  void* ws, size_t ws_bytes, void* stream);

/* Backward, recomputing z:
 *   G~ = bf16(r (exp(z - lse) - onehot)) (0 on rows whose label lies outside
 *   [0, V)), s = dloss / n_valid,
 *   T = s sum_v G~ z,  dy = bf16(s G~ W~^T - (r T / D) y + dres),
 *   dW = beta dW + s g (y^T G~) (fp32 [D, V]),  dg = beta dg + s sum_v W (y^T G~) (fp32 1 x D).
 * r: the forward's r_out; W_unfolded: W without the gain; g: fp32 1 x D;
 * dres: optional bf16 [M, D] gradient arriving along the residual stream.
 * chunk_rows bounds the recomputed logits as in coda_linear_cross_entropy_bwd:
 * 0 (or >= M) recomputes all M x V at once; otherwise the recompute runs over
 * vocabulary slices of about chunk_rows x V values (a multiple of 256
 * columns), each writing its own columns of dW, with s G~ W~^T summed in
 * fp32 over the slices and the correction and rounding applied once after
 * the last (the workspace then also holds an fp32 [M, D] buffer).
 * With M = 0, dW and dg are left unchanged.  ignore_index must lie outside
 * [0, V) as in the forward. */
coda_status coda_linear_rmsnorm_cross_entropy_bwd_workspace(int64_t M, int64_t D, int64_t V, int64_t chunk_rows,
                                                            int32_t precision, size_t* bytes);
coda_status coda_linear_rmsnorm_cross_entropy_bwd(const coda_mat* y, const coda_mat* r, const coda_weight* W,
                                                  const coda_mat* W_unfolded, const coda_mat* g,
                                                  const coda_mat* labels, int32_t ignore_index, const coda_mat* lse,
                                                  const coda_mat* n_valid, float dloss, const coda_mat* dres,
                                                  const coda_mat* dy, const coda_mat* dW, const coda_mat* dg,
                                                  float beta, int64_t chunk_rows, int32_t precision, void* ws,
                                                  size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CODA_H_ */
