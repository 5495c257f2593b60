// The unfused baseline: separate memory-bound kernels for RMSNorm (forward and
// backward), residual add, SwiGLU (forward and backward) and QK-norm + RoPE,
// to run around the library's plain-store GEMMs (contract in coda_unfused.h).
#include "../../include/coda_unfused.h"
#include "aux_kernels.hpp"
#include "capi_util.hpp"

using namespace coda;

namespace {

__global__ void unf_rmsnorm_fwd_kernel(const uint16_t* x, int64_t ldx, int M, int D, const float* g, float eps,
                                       uint16_t* out, int64_t ldo, float* r_out) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (m >= M) return;
  const uint16_t* row = x + (int64_t)m * ldx;
  float s = 0.0f;
  for (int k = lane * 8; k < D; k += 512) {
    uint4 w = *reinterpret_cast<const uint4*>(row + k);
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) s += bf_lo(ws[t]) * bf_lo(ws[t]) + bf_hi(ws[t]) * bf_hi(ws[t]);
  }
  s = wave_sum(s);
  const float r = rsqrtf(s / (float)D + eps);
  if (r_out && lane == 0) r_out[m] = r;
  for (int k = lane * 8; k < D; k += 512) {
    uint4 w = *reinterpret_cast<const uint4*>(row + k);
    uint32_t ws[4] = {w.x, w.y, w.z, w.w}, o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      o[t] = pack_bf2(bf_lo(ws[t]) * r * g[k + 2 * t], bf_hi(ws[t]) * r * g[k + 2 * t + 1]);
    *reinterpret_cast<uint4*>(out + (int64_t)m * ldo + k) = uint4{o[0], o[1], o[2], o[3]};
  }
}

__global__ void unf_rmsnorm_bwd_kernel(const uint16_t* u, int64_t ldu, const float* g, const float* r,
                                       const uint16_t* dy, int64_t lddy, const uint16_t* dres, int64_t ldres,
                                       int M, int D, uint16_t* du, int64_t lddu) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (m >= M) return;
  float s = 0.0f;
  for (int k = lane * 8; k < D; k += 512) {
    uint4 uw = *reinterpret_cast<const uint4*>(u + (int64_t)m * ldu + k);
    uint4 dw = *reinterpret_cast<const uint4*>(dy + (int64_t)m * lddy + k);
    uint32_t ua[4] = {uw.x, uw.y, uw.z, uw.w}, da[4] = {dw.x, dw.y, dw.z, dw.w};
#pragma unroll
    for (int t = 0; t < 4; ++t)
      s += bf_lo(ua[t]) * (g[k + 2 * t] * bf_lo(da[t])) + bf_hi(ua[t]) * (g[k + 2 * t + 1] * bf_hi(da[t]));
  }
  s = wave_sum(s);
  const float rr = r[m];
  const float c = rr * rr * rr / (float)D * s;
  for (int k = lane * 8; k < D; k += 512) {
    uint4 uw = *reinterpret_cast<const uint4*>(u + (int64_t)m * ldu + k);
    uint4 dw = *reinterpret_cast<const uint4*>(dy + (int64_t)m * lddy + k);
    uint4 rw = dres ? *reinterpret_cast<const uint4*>(dres + (int64_t)m * ldres + k) : uint4{0, 0, 0, 0};
    uint32_t ua[4] = {uw.x, uw.y, uw.z, uw.w}, da[4] = {dw.x, dw.y, dw.z, dw.w}, ra[4] = {rw.x, rw.y, rw.z, rw.w};
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float t0 = g[k + 2 * t] * bf_lo(da[t]), t1 = g[k + 2 * t + 1] * bf_hi(da[t]);
      const float v0 = rr * t0 - c * bf_lo(ua[t]) + bf_lo(ra[t]);
      const float v1 = rr * t1 - c * bf_hi(ua[t]) + bf_hi(ra[t]);
      o[t] = pack_bf2(v0, v1);
    }
    *reinterpret_cast<uint4*>(du + (int64_t)m * lddu + k) = uint4{o[0], o[1], o[2], o[3]};
  }
}

// column partial sums of r u dy over blocks of rows (gain gradient)
__global__ void unf_rmsnorm_dg_kernel(const uint16_t* u, int64_t ldu, const float* r, const uint16_t* dy,
                                      int64_t lddy, int M, int D, int rows_per_block, float* part) {
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 2;
  if (c >= D) return;
  const int r0 = blockIdx.y * rows_per_block;
  float s0 = 0.0f, s1 = 0.0f;
  for (int m = r0; m < min(M, r0 + rows_per_block); ++m) {
    const uint32_t uw = *reinterpret_cast<const uint32_t*>(u + (int64_t)m * ldu + c);
    const uint32_t dw = *reinterpret_cast<const uint32_t*>(dy + (int64_t)m * lddy + c);
    s0 += r[m] * bf_lo(uw) * bf_lo(dw);
    s1 += r[m] * bf_hi(uw) * bf_hi(dw);
  }
  part[(int64_t)blockIdx.y * D + c] = s0;
  part[(int64_t)blockIdx.y * D + c + 1] = s1;
}

__global__ void unf_add_kernel(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, uint16_t* out,
                               int64_t ldo, int M, int N) {
  const int m = blockIdx.y;
  for (int n = (blockIdx.x * blockDim.x + threadIdx.x) * 8; n < N; n += gridDim.x * blockDim.x * 8) {
    uint4 x = *reinterpret_cast<const uint4*>(a + (int64_t)m * lda + n);
    uint4 y = *reinterpret_cast<const uint4*>(b + (int64_t)m * ldb + n);
    uint32_t xa[4] = {x.x, x.y, x.z, x.w}, ya[4] = {y.x, y.y, y.z, y.w}, o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = pack_bf2(bf_lo(xa[t]) + bf_lo(ya[t]), bf_hi(xa[t]) + bf_hi(ya[t]));
    *reinterpret_cast<uint4*>(out + (int64_t)m * ldo + n) = uint4{o[0], o[1], o[2], o[3]};
  }
}

// packed h [M, 2F]: 64-column blocks of 32 gate then 32 up columns
__global__ void unf_swiglu_fwd_kernel(const uint16_t* h, int64_t ldh, uint16_t* out, int64_t ldo, int M, int F) {
  const int m = blockIdx.y;
  for (int f = (blockIdx.x * blockDim.x + threadIdx.x) * 8; f < F; f += gridDim.x * blockDim.x * 8) {
    const int pg = (f >> 5) * 64 + (f & 31);
    uint4 gw = *reinterpret_cast<const uint4*>(h + (int64_t)m * ldh + pg);
    uint4 uw = *reinterpret_cast<const uint4*>(h + (int64_t)m * ldh + pg + 32);
    uint32_t ga[4] = {gw.x, gw.y, gw.z, gw.w}, ua[4] = {uw.x, uw.y, uw.z, uw.w}, o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float g0 = bf_lo(ga[t]), g1 = bf_hi(ga[t]);
      o[t] = pack_bf2(g0 * sigmoidf_(g0) * bf_lo(ua[t]), g1 * sigmoidf_(g1) * bf_hi(ua[t]));
    }
    *reinterpret_cast<uint4*>(out + (int64_t)m * ldo + f) = uint4{o[0], o[1], o[2], o[3]};
  }
}

__global__ void unf_swiglu_bwd_kernel(const uint16_t* da, int64_t ldda, const uint16_t* h, int64_t ldh,
                                      uint16_t* dh, int64_t lddh, int M, int F) {
  const int m = blockIdx.y;
  for (int f = (blockIdx.x * blockDim.x + threadIdx.x) * 8; f < F; f += gridDim.x * blockDim.x * 8) {
    const int pg = (f >> 5) * 64 + (f & 31);
    uint4 aw = *reinterpret_cast<const uint4*>(da + (int64_t)m * ldda + f);
    uint4 gw = *reinterpret_cast<const uint4*>(h + (int64_t)m * ldh + pg);
    uint4 uw = *reinterpret_cast<const uint4*>(h + (int64_t)m * ldh + pg + 32);
    uint32_t aa[4] = {aw.x, aw.y, aw.z, aw.w}, ga[4] = {gw.x, gw.y, gw.z, gw.w}, ua[4] = {uw.x, uw.y, uw.z, uw.w};
    uint32_t og[4], ou[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float dg[2], du[2];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const float a = hlf ? bf_hi(aa[t]) : bf_lo(aa[t]);
        const float g = hlf ? bf_hi(ga[t]) : bf_lo(ga[t]);
        const float u = hlf ? bf_hi(ua[t]) : bf_lo(ua[t]);
        const float s = sigmoidf_(g);
        dg[hlf] = a * u * s * (1.0f + g * (1.0f - s));
        du[hlf] = a * g * s;
      }
      og[t] = pack_bf2(dg[0], dg[1]);
      ou[t] = pack_bf2(du[0], du[1]);
    }
    *reinterpret_cast<uint4*>(dh + (int64_t)m * lddh + pg) = uint4{og[0], og[1], og[2], og[3]};
    *reinterpret_cast<uint4*>(dh + (int64_t)m * lddh + pg + 32) = uint4{ou[0], ou[1], ou[2], ou[3]};
  }
}

// one wave per (row, head); lane l owns the RoPE pair (2l, 2l+1)
__global__ void unf_qknorm_rope_fwd_kernel(const uint16_t* qkv, int64_t ld, const float* gq, const float* gk,
                                           const float* table, int seq_len, float eps, int M, int D,
                                           uint16_t* q, int64_t ldq, uint16_t* k, int64_t ldk) {
  const int lane = threadIdx.x & 63;
  const int H = D / 128;
  const int item = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);   // (row, region, head)
  if (item >= M * 2 * H) return;
  const int m = item / (2 * H), reg = (item / H) % 2, h = item % H;
  const int col = h * 128 + 2 * lane;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(qkv + (int64_t)m * ld + reg * D + col);
  const float u0 = bf_lo(w), u1 = bf_hi(w);
  const float rho = rsqrtf(wave_sum(u0 * u0 + u1 * u1) / 128.0f + eps);
  const float* g = reg == 0 ? gq : gk;
  const float y0 = u0 * rho * g[2 * lane], y1 = u1 * rho * g[2 * lane + 1];
  const int pos = m % seq_len;
  const float c = table[((int64_t)pos * 64 + lane) * 2], s = table[((int64_t)pos * 64 + lane) * 2 + 1];
  const uint32_t o = pack_bf2(y0 * c - y1 * s, y0 * s + y1 * c);
  uint16_t* dst = reg == 0 ? q + (int64_t)m * ldq : k + (int64_t)m * ldk;
  *reinterpret_cast<uint32_t*>(dst + col) = o;
}

}  // namespace

extern "C" coda_status coda_unfused_rmsnorm_fwd(const coda_mat* x, const coda_mat* g, float eps, const coda_mat* out,
                                                const coda_mat* r_out, void* stream) {
  TRY(check_mat(x, "x", CODA_BF16, -1, -1));
  const int64_t M = x->rows, D = x->cols;
  TRY(check_vec(g, "g", CODA_F32, D));
  TRY(check_mat(out, "out", CODA_BF16, M, D));
  TRY(check_vec(r_out, "r_out", CODA_F32, M, true));
  if (M == 0) return CODA_OK;
  hipLaunchKernelGGL(unf_rmsnorm_fwd_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, S(stream),
                     static_cast<const uint16_t*>(x->ptr), x->ld, (int)M, (int)D, fptr(g), eps,
                     static_cast<uint16_t*>(out->ptr), out->ld,
                     present(r_out) ? static_cast<float*>(r_out->ptr) : nullptr);
  return check_launch("unfused_rmsnorm_fwd");
}

static const int kDgRows = 256;

extern "C" coda_status coda_unfused_rmsnorm_bwd_workspace(int64_t M, int64_t D, size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  Carver cv(nullptr);
  cv.take<float>((size_t)((M + kDgRows - 1) / kDgRows) * D);
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_unfused_rmsnorm_bwd(const coda_mat* u, const coda_mat* g, const coda_mat* r,
                                                const coda_mat* dy, const coda_mat* dres, const coda_mat* du,
                                                const coda_mat* dg, float beta, void* ws, size_t ws_bytes,
                                                void* stream) {
  TRY(check_mat(u, "u", CODA_BF16, -1, -1));
  const int64_t M = u->rows, D = u->cols;
  TRY(check_vec(g, "g", CODA_F32, D));
  TRY(check_vec(r, "r", CODA_F32, M));
  TRY(check_mat(dy, "dy", CODA_BF16, M, D));
  TRY(check_mat(dres, "dres", CODA_BF16, M, D, true));
  TRY(check_mat(du, "du", CODA_BF16, M, D));
  TRY(check_vec(dg, "dg", CODA_F32, D));
  Carver cv(ws);
  const int nblk = (int)((M + kDgRows - 1) / kDgRows);
  float* part = cv.take<float>((size_t)nblk * D);
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  if (M > 0) {
    hipLaunchKernelGGL(unf_rmsnorm_bwd_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(u->ptr), u->ld, fptr(g), fptr(r),
                       static_cast<const uint16_t*>(dy->ptr), dy->ld,
                       present(dres) ? static_cast<const uint16_t*>(dres->ptr) : nullptr,
                       present(dres) ? dres->ld : 0, (int)M, (int)D, static_cast<uint16_t*>(du->ptr), du->ld);
    hipLaunchKernelGGL(unf_rmsnorm_dg_kernel, dim3((unsigned)((D / 2 + 255) / 256), nblk), dim3(256), 0, s,
                       static_cast<const uint16_t*>(u->ptr), u->ld, fptr(r), static_cast<const uint16_t*>(dy->ptr),
                       dy->ld, (int)M, (int)D, kDgRows, part);
    TRY(check_launch("unfused_rmsnorm_bwd"));
  }
  hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)((D + 63) / 64)), dim3(1024), 0, s, part, nblk, (int)D, beta,
                     static_cast<float*>(dg->ptr));
  return check_launch("unfused_rmsnorm_bwd: dg");
}

extern "C" coda_status coda_unfused_add(const coda_mat* a, const coda_mat* b, const coda_mat* out, void* stream) {
  TRY(check_mat(a, "a", CODA_BF16, -1, -1));
  TRY(check_mat(b, "b", CODA_BF16, a->rows, a->cols));
  TRY(check_mat(out, "out", CODA_BF16, a->rows, a->cols));
  if (a->rows == 0 || a->cols == 0) return CODA_OK;
  hipLaunchKernelGGL(unf_add_kernel, dim3((unsigned)((a->cols / 8 + 255) / 256), (unsigned)a->rows), dim3(256), 0,
                     S(stream), static_cast<const uint16_t*>(a->ptr), a->ld, static_cast<const uint16_t*>(b->ptr),
                     b->ld, static_cast<uint16_t*>(out->ptr), out->ld, (int)a->rows, (int)a->cols);
  return check_launch("unfused_add");
}

extern "C" coda_status coda_unfused_swiglu_fwd(const coda_mat* h, const coda_mat* out, void* stream) {
  TRY(check_mat(h, "h", CODA_BF16, -1, -1));
  if (h->cols % 64 != 0) return fail(CODA_ERR_SHAPE, "swiglu: 2F must be a multiple of 64");
  TRY(check_mat(out, "out", CODA_BF16, h->rows, h->cols / 2));
  if (h->rows == 0) return CODA_OK;
  const int F = (int)(h->cols / 2);
  hipLaunchKernelGGL(unf_swiglu_fwd_kernel, dim3((unsigned)((F / 8 + 255) / 256), (unsigned)h->rows), dim3(256), 0,
                     S(stream), static_cast<const uint16_t*>(h->ptr), h->ld, static_cast<uint16_t*>(out->ptr),
                     out->ld, (int)h->rows, F);
  return check_launch("unfused_swiglu_fwd");
}

extern "C" coda_status coda_unfused_swiglu_bwd(const coda_mat* da, const coda_mat* h, const coda_mat* dh,
                                               void* stream) {
  TRY(check_mat(h, "h", CODA_BF16, -1, -1));
  if (h->cols % 64 != 0) return fail(CODA_ERR_SHAPE, "swiglu: 2F must be a multiple of 64");
  TRY(check_mat(da, "da", CODA_BF16, h->rows, h->cols / 2));
  TRY(check_mat(dh, "dh", CODA_BF16, h->rows, h->cols));
  if (h->rows == 0) return CODA_OK;
  const int F = (int)(h->cols / 2);
  hipLaunchKernelGGL(unf_swiglu_bwd_kernel, dim3((unsigned)((F / 8 + 255) / 256), (unsigned)h->rows), dim3(256), 0,
                     S(stream), static_cast<const uint16_t*>(da->ptr), da->ld, static_cast<const uint16_t*>(h->ptr),
                     h->ld, static_cast<uint16_t*>(dh->ptr), dh->ld, (int)h->rows, F);
  return check_launch("unfused_swiglu_bwd");
}

extern "C" coda_status coda_unfused_qknorm_rope_fwd(const coda_mat* qkv, const coda_mat* gq, const coda_mat* gk,
                                                    const coda_mat* rope, int32_t seq_len, float eps,
                                                    const coda_mat* q, const coda_mat* k, void* stream) {
  TRY(check_mat(qkv, "qkv", CODA_BF16, -1, -1));
  const int64_t M = qkv->rows, D = qkv->cols / 3;
  if (qkv->cols % 384 != 0) return fail(CODA_ERR_SHAPE, "qkv: 3D with D a multiple of 128");
  TRY(check_vec(gq, "gq", CODA_F32, 128));
  TRY(check_vec(gk, "gk", CODA_F32, 128));
  if (seq_len <= 0) return fail(CODA_ERR_VALUE, "seq_len must be > 0");
  TRY(check_mat(rope, "rope", CODA_F32, seq_len, 128));
  TRY(check_mat(q, "q", CODA_BF16, M, D));
  TRY(check_mat(k, "k", CODA_BF16, M, D));
  const int64_t items = M * 2 * (D / 128);
  if (items == 0) return CODA_OK;
  hipLaunchKernelGGL(unf_qknorm_rope_fwd_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, S(stream),
                     static_cast<const uint16_t*>(qkv->ptr), qkv->ld, fptr(gq), fptr(gk), fptr(rope), seq_len, eps,
                     (int)M, (int)D, static_cast<uint16_t*>(q->ptr), q->ld, static_cast<uint16_t*>(k->ptr), k->ld);
  return check_launch("unfused_qknorm_rope_fwd");
}

static const int kQkRowsPerWave = 4;

extern "C" coda_status coda_unfused_qknorm_rope_bwd_workspace(int64_t M, int64_t D, size_t* bytes) {
  if (!bytes) return fail(CODA_ERR_NULL, "NULL bytes");
  const int64_t nblk = (M + 4 * kQkRowsPerWave - 1) / (4 * kQkRowsPerWave);
  Carver cv(nullptr);
  cv.take<float>(M);
  cv.take<float>((size_t)std::max<int64_t>(nblk, 1) * 128);
  cv.take<float>((size_t)std::max<int64_t>(nblk, 1) * 128);
  (void)D;
  *bytes = cv.off;
  return CODA_OK;
}

extern "C" coda_status coda_unfused_qknorm_rope_bwd(const coda_mat* dq, const coda_mat* dk, const coda_mat* dv,
                                                    const coda_mat* qkv, const coda_mat* gq, const coda_mat* gk,
                                                    const coda_mat* rope, int32_t seq_len, float eps,
                                                    const coda_mat* dqkv, const coda_mat* dgq, const coda_mat* dgk,
                                                    float beta, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_mat(qkv, "qkv", CODA_BF16, -1, -1));
  const int64_t M = qkv->rows, D = qkv->cols / 3;
  if (qkv->cols % 384 != 0) return fail(CODA_ERR_SHAPE, "qkv: 3D with D a multiple of 128");
  TRY(check_mat(dq, "dq", CODA_BF16, M, D));
  TRY(check_mat(dk, "dk", CODA_BF16, M, D));
  TRY(check_mat(dv, "dv", CODA_BF16, M, D));
  if (dk->ld != dq->ld || dv->ld != dq->ld) return fail(CODA_ERR_LAYOUT, "dq, dk, dv must share ld");
  TRY(check_vec(gq, "gq", CODA_F32, 128));
  TRY(check_vec(gk, "gk", CODA_F32, 128));
  if (seq_len <= 0) return fail(CODA_ERR_VALUE, "seq_len must be > 0");
  TRY(check_mat(rope, "rope", CODA_F32, seq_len, 128));
  TRY(check_mat(dqkv, "dqkv", CODA_BF16, M, 3 * D));
  TRY(check_vec(dgq, "dgq", CODA_F32, 128));
  TRY(check_vec(dgk, "dgk", CODA_F32, 128));
  const int nblk = (int)((M + 4 * kQkRowsPerWave - 1) / (4 * kQkRowsPerWave));
  Carver cv(ws);
  float* T = cv.take<float>(M);
  float* pgq = cv.take<float>((size_t)std::max(nblk, 1) * 128);
  float* pgk = cv.take<float>((size_t)std::max(nblk, 1) * 128);
  TRY(ws_check(cv, ws_bytes, ws));
  hipStream_t s = S(stream);
  const uint16_t* base = static_cast<const uint16_t*>(qkv->ptr);
  if (M > 0) {
    hipLaunchKernelGGL(qknorm_rope_bwd_kernel, dim3(nblk), dim3(256), 0, s, static_cast<const uint16_t*>(dq->ptr),
                       static_cast<const uint16_t*>(dk->ptr), static_cast<const uint16_t*>(dv->ptr), dq->ld, base,
                       qkv->ld, base + 2 * D, qkv->ld, (const float*)nullptr, fptr(gq), fptr(gk), fptr(rope),
                       seq_len, eps, (int)M, (int)D, kQkRowsPerWave, static_cast<uint16_t*>(dqkv->ptr), dqkv->ld,
                       T, pgq, pgk);
    TRY(check_launch("unfused_qknorm_rope_bwd"));
  }
  hipLaunchKernelGGL(sum_partials_kernel, dim3(2), dim3(1024), 0, s, pgq, nblk, 128, beta, static_cast<float*>(dgq->ptr));
  hipLaunchKernelGGL(sum_partials_kernel, dim3(2), dim3(1024), 0, s, pgk, nblk, 128, beta, static_cast<float*>(dgk->ptr));
  return check_launch("unfused_qknorm_rope_bwd: dg");
}
