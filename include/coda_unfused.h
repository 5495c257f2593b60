/*
 * coda_unfused.h - the unfused baseline of the GEMM+epilogue library.
 *
 * The CODA paper (arXiv 2605.19269, §1 and §2.1) contrasts GEMM+epilogue
 * programs with the usual operator sequence, where every normalisation,
 * activation and residual update is its own memory-bound kernel.  These entry
 * points are that sequence, built from the library's own GEMM (coda_gemm_epi
 * with a plain STORE_BF16 / ACCUM_F32 program) plus the separate elementwise
 * kernels below, so the fused path can be timed against it on the same GPU.
 *
 * Same conventions as coda.h: device pointers in coda_mat descriptors,
 * caller-owned memory, asynchronous on `stream`, host-side validation before
 * any HIP call, status codes.
 */
#ifndef CODA_UNFUSED_H_
#define CODA_UNFUSED_H_

#include "coda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out = bf16(x * r * g) with r = (mean(x^2) + eps)^(-1/2) per row (canonical
 * RMSNorm); x, out bf16 [M, D]; g fp32 1 x D; r_out fp32 1 x M (optional). */
coda_status coda_unfused_rmsnorm_fwd(const coda_mat* x, const coda_mat* g, float eps, const coda_mat* out,
                                     const coda_mat* r_out, void* stream);

/* RMSNorm backward given dy = d(out): t = g dy, du = r t - (r^3 / D) u sum(u t)
 * (+ dres when given), stored bf16; dg = beta dg + sum over rows of r u dy.
 * u: the norm input, r: its saved inverse RMS. */
coda_status coda_unfused_rmsnorm_bwd_workspace(int64_t M, int64_t D, size_t* bytes);
coda_status coda_unfused_rmsnorm_bwd(const coda_mat* u, const coda_mat* g, const coda_mat* r, const coda_mat* dy,
                                     const coda_mat* dres, const coda_mat* du, const coda_mat* dg, float beta,
                                     void* ws, size_t ws_bytes, void* stream);

/* out = a + b (bf16, same shape). */
coda_status coda_unfused_add(const coda_mat* a, const coda_mat* b, const coda_mat* out, void* stream);

/* SwiGLU on the packed gate/up product h [M, 2F] -> out [M, F], and its
 * backward: dh (packed [M, 2F]) from da [M, F] and h. */
coda_status coda_unfused_swiglu_fwd(const coda_mat* h, const coda_mat* out, void* stream);
coda_status coda_unfused_swiglu_bwd(const coda_mat* da, const coda_mat* h, const coda_mat* dh, void* stream);

/* QK-norm + RoPE on the QKV product qkv [M, 3D] (q | k | v): q, k bf16 [M, D]. */
coda_status coda_unfused_qknorm_rope_fwd(const coda_mat* qkv, const coda_mat* gq, const coda_mat* gk,
                                         const coda_mat* rope, int32_t seq_len, float eps, const coda_mat* q,
                                         const coda_mat* k, void* stream);

/* Backward of QK-norm + RoPE: dqkv [M, 3D] = (d q_pre | d k_pre | dv) from the
 * attention gradients and the saved product qkv; dgq, dgk = beta dg + ... */
coda_status coda_unfused_qknorm_rope_bwd_workspace(int64_t M, int64_t D, size_t* bytes);
coda_status coda_unfused_qknorm_rope_bwd(const coda_mat* dq, const coda_mat* dk, const coda_mat* dv,
                                         const coda_mat* qkv, const coda_mat* gq, const coda_mat* gk,
                                         const coda_mat* rope, int32_t seq_len, float eps, const coda_mat* dqkv,
                                         const coda_mat* dgq, const coda_mat* dgk, float beta, void* ws,
                                         size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CODA_UNFUSED_H_ */
