// Light HBM-bound kernels around the GEMMs: weight preparation, row
// statistics, the finishers that merge per-tile partials, the RoPE / QK-norm
// backward glue and the cross-entropy finishers.
//
// The CODA paper (arXiv 2605.19269), §3.1 item 4, merges tile partials with
// lightweight auxiliary kernels; the KuCoin news summary of CODA (section on
// the epilogue) describes the tiny reduction that combines the partial RMS
// values.  All reductions here run in a fixed order (no float atomics).
#pragma once
#include "coda_device.hpp"

namespace coda {

// W~[k, n] = bf16(g[k] * W[k, n]): the RMSNorm gain folded into the next weight.
__global__ void fold_gain_kernel(const uint16_t* W, int64_t ldw, const float* g, uint16_t* out,
                                 int64_t ldo, int K, int N);
// Packs W_gate, W_up [K, F] into [K, 2F]: every 64-column block holds 32 gate
// columns then the matching 32 up columns; optionally folds the gain g[k].
__global__ void pack_gate_up_kernel(const uint16_t* Wg, int64_t ldg, const uint16_t* Wu, int64_t ldu,
                                    const float* g, uint16_t* out, int64_t ldo, int K, int F);
// out[p][i] = (cos, sin)(p * theta^(-2 i / head_dim)), angle in float64.
__global__ void rope_table_kernel(int seq_len, int head_dim, double theta, float* out);
// out[m] = sum_k x[m, k]^2 (fp32), one wave per row.
__global__ void row_sumsq_kernel(const uint16_t* x, int64_t ld, int M, int K, float* out);
// out[m] = sum_{t < nP} P[t][m]                 (mode 0)
//        = (sum / D + eps)^(-1/2)               (mode 1)
//        = rowvec[m] * sum / D                  (mode 2)
__global__ void rows_finish_kernel(const float* P, int nP, int M, int mode, const float* rowvec,
                                   int D, float eps, float* out);
// Split-K finish: out[r][c] = beta out[r][c] + sum_{s < nslices} P[s * slice + r * cols + c],
// slices added in ascending order; cols % 4 == 0, 16-byte aligned rows.
__global__ __launch_bounds__(256) void split_sum_kernel(const float* P, int nslices, int64_t slice, int rows, int cols,
                                                        float beta, float* out, int64_t ld);
// out[k] = beta * out[k] + sum_{t < nP} P[t][k]
__global__ __launch_bounds__(1024) void sum_partials_kernel(const float* P, int nP, int K, float beta, float* out);
// Backward glue between attention and the QKV dgrad / wgrad GEMMs: inverse
// RoPE of dq, dk, per-head RMSNorm backward (from the saved pre-norm q, k),
// r1 row scale -> dh~_qkv (bf16 [M, 3D]); T1[m] = sum_j dh~ h; gain-gradient
// partials for g_q and g_k per block.  r1 == nullptr means r1 = 1.
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(const uint16_t* dq, const uint16_t* dk, const uint16_t* dv,
                                       int64_t ld_g, const uint16_t* qk_pre, int64_t ld_pre,
                                       const uint16_t* v, int64_t ld_v, const float* r1,
                                       const float* gq, const float* gk, const float* table,
                                       int seq_len, float eps, int M, int D, int rows_per_wave,
                                       uint16_t* dh, int64_t ld_dh, float* T1,
                                       float* pgq, float* pgk);
// Per-row cross-entropy finish: lse from the (max, sum-exp) tile partials,
// per-row loss, and a status per row (0 valid, 1 ignored, 2 bad label).
__global__ void ce_finish_rows_kernel(const float* Pm, const float* Ps, int nT, int M,
                                      const float* zy, const int* labels, int V, int ignore_index,
                                      float* lse, float* per_row, int* status);
// Single-workgroup mean over valid rows: loss = sum / n_valid, n_valid, and
// the count of bad labels.
__global__ void ce_finish_loss_kernel(const float* per_row, const int* status, int M, float* loss,
                                      int* n_valid, int* n_bad);
// scale[0] = dloss / n_valid (0 when n_valid == 0)
__global__ void ce_scale_kernel(const int* n_valid, float dloss, float* scale);
// out = bf16(X), fp32 [R, C] -> bf16 (C % 4 == 0); grid (x, R)
__global__ void f32_to_bf16_kernel(const float* X, int64_t ldx, uint16_t* out, int64_t ldo, int R, int C);
// out[i] = v for i < n
__global__ void fill_f32_kernel(float* out, int n, float v);
// out[r][c] = beta out[r][c] (beta 0 writes zeros without reading); grid (x, R)
__global__ void scale_f32_kernel(float* out, int64_t ld, int R, int C, float beta);
// RMSNorm backward correction after a product accumulated in fp32 over
// slices: out[r][c] = bf16(acc[r][c] - (*scale) cr[r] y[r][c] + res[r][c])
// (res optional), with acc already scaled; grid (x, R), C % 4 == 0.
__global__ void norm_corr_finish_kernel(const float* acc, int64_t lda, const uint16_t* y, int64_t ldy, const float* cr,
                                        const float* scale, const uint16_t* res, int64_t ldr, uint16_t* out,
                                        int64_t ldo, int R, int C);
// E4M3 quantisation with amax over the contracted axis.
//   axis 1: Q[r, c] with one scale per row  r  (Q keeps the [R, C] layout),
//           amax and codes in one kernel (a wave a row)
//   axis 0: Q^T[c, r] with one scale per column c (Q written transposed, so the
//           GEMM's contracted axis is contiguous)
__global__ void amax_cols_partial_kernel(const uint16_t* X, int64_t ld, int R, int C, int rows_per_block,
                                         float* part);
__global__ void amax_cols_finish_kernel(const float* part, int nparts, int C, float* amax);
__global__ void quant_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                  float* scale);
__global__ void quant_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, const float* amax,
                                    uint8_t* QT, int64_t ldq, float* scale);
// MXFP8 quantisation (E4M3 elements, one E8M0 scale per 32 values of the
// contracted axis): blocks along the columns, or along the rows written
// transposed.
__global__ void quant_mx_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                     uint8_t* S, int64_t lds);
__global__ void quant_mx_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* QT, int64_t ldq,
                                       uint8_t* S, int64_t lds);
// MXFP4 (E2M1 elements, packed two a byte, element 2i in the low nibble)
// with E8M0 exponents in word layout; same shapes and launches as the MXFP8
// quantisers above, with Q holding C / 2 (or R / 2) bytes a row.
__global__ void quant_mx4_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                      uint8_t* S, int64_t lds);
__global__ void quant_mx4_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* QT, int64_t ldq,
                                        uint8_t* S, int64_t lds);
// MXFP6 (f6 = 2: E2M3, f6 = 3: E3M2), a 32-value block packed into 24 bytes
// then 8 zero bytes, so Q rows hold as many bytes as values; same shapes and
// launches as the MXFP8 quantisers.
__global__ void quant_mx6_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                      uint8_t* S, int64_t lds, int f6);
__global__ void quant_mx6_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* QT, int64_t ldq,
                                        uint8_t* S, int64_t lds, int f6);

}  // namespace coda
