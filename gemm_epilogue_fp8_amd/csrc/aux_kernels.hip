// Auxiliary kernels (see aux_kernels.hpp for the contract of each).
#include "aux_kernels.hpp"

namespace coda {

__global__ void fold_gain_kernel(const uint16_t* W, int64_t ldw, const float* g, uint16_t* out,
                                 int64_t ldo, int K, int N) {
  const int k = blockIdx.y;
  const float gk = g[k];
  for (int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4; n < N; n += gridDim.x * blockDim.x * 4) {
    uint2 w = *reinterpret_cast<const uint2*>(W + (int64_t)k * ldw + n);
    uint2 o = {pack_bf2(gk * bf_lo(w.x), gk * bf_hi(w.x)), pack_bf2(gk * bf_lo(w.y), gk * bf_hi(w.y))};
    *reinterpret_cast<uint2*>(out + (int64_t)k * ldo + n) = o;
  }
}

__global__ void pack_gate_up_kernel(const uint16_t* Wg, int64_t ldg, const uint16_t* Wu, int64_t ldu,
                                    const float* g, uint16_t* out, int64_t ldo, int K, int F) {
  const int k = blockIdx.y;
  const float gk = g ? g[k] : 1.0f;
  const int N = 2 * F;
  for (int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4; n < N; n += gridDim.x * blockDim.x * 4) {
    const int b = n >> 6, t = n & 63;
    const bool up = t >= 32;
    const int f = b * 32 + (t & 31);
    const uint16_t* src = up ? Wu + (int64_t)k * ldu : Wg + (int64_t)k * ldg;
    uint2 w = *reinterpret_cast<const uint2*>(src + f);
    uint2 o = w;
    if (g) o = uint2{pack_bf2(gk * bf_lo(w.x), gk * bf_hi(w.x)), pack_bf2(gk * bf_lo(w.y), gk * bf_hi(w.y))};
    *reinterpret_cast<uint2*>(out + (int64_t)k * ldo + n) = o;
  }
}

__global__ void rope_table_kernel(int seq_len, int head_dim, double theta, float* out) {
  const int half = head_dim / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= seq_len * half) return;
  const int p = idx / half, i = idx % half;
  const double ang = (double)p * pow(theta, -2.0 * (double)i / (double)head_dim);
  out[2 * idx] = (float)cos(ang);
  out[2 * idx + 1] = (float)sin(ang);
}

__global__ void row_sumsq_kernel(const uint16_t* x, int64_t ld, int M, int K, float* out) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (m >= M) return;
  const uint16_t* row = x + (int64_t)m * ld;
  float s = 0.0f;
  for (int k = lane * 8; k < K; k += 512) {
    uint4 w = *reinterpret_cast<const uint4*>(row + k);
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float a = bf_lo(ws[t]), b = bf_hi(ws[t]);
      s += a * a + b * b;
    }
  }
  s = wave_sum(s);
  if (lane == 0) out[m] = s;
}

__global__ void rows_finish_kernel(const float* P, int nP, int M, int mode, const float* rowvec,
                                   int D, float eps, float* out) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int t = 0;
  for (; t + 8 <= nP; t += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += P[(int64_t)(t + u) * M + m];
  for (; t < nP; ++t) acc[0] += P[(int64_t)t * M + m];
  float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  if (mode == 1) s = rsqrtf(s / (float)D + eps);
  else if (mode == 2) s = rowvec[m] * s / (float)D;
  out[m] = s;
}

__global__ __launch_bounds__(256) void split_sum_kernel(const float* P, int nslices, int64_t slice, int rows, int cols,
                                                        float beta, float* out, int64_t ld) {
  // out[r][c..c+3] = beta out + sum over s (ascending) of P[s][r][c..c+3]
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cq = cols / 4;
  if (q >= (int64_t)rows * cq) return;
  const int r = (int)(q / cq), c = (int)(q % cq) * 4;
  const float* p = P + (int64_t)r * cols + c;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(p);
  for (int s = 1; s < nslices; ++s) acc = acc + *reinterpret_cast<const f32x4_t*>(p + s * slice);
  f32x4_t* o = reinterpret_cast<f32x4_t*>(out + (int64_t)r * ld + c);
  if (beta != 0.0f) acc = acc + beta * *o;
  *o = acc;
}

__global__ __launch_bounds__(1024) void sum_partials_kernel(const float* P, int nP, int K, float beta, float* out) {
  // block of 1024 threads: 64 columns x 16 partial groups; group j adds
  // partials j, j + 16, ...
  // and the 16 group sums are combined in a fixed tree
  __shared__ float red[16][64];
  const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cl;
  float s = 0.0f;
  if (c < K) {
#pragma unroll 4
    for (int t = grp; t < nP; t += 16) s += P[(int64_t)t * K + c];
  }
  red[grp][cl] = s;
  __syncthreads();
  if (grp == 0 && c < K) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = red[2 * j][cl] + red[2 * j + 1][cl];
    const float w = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    out[c] = (beta != 0.0f ? beta * out[c] : 0.0f) + w;
  }
}

__device__ __forceinline__ float sum16(float v) {   // sum over the 16-lane group of this lane
  v += __shfl_xor(v, 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

__device__ __forceinline__ void unpack8(uint4 w, float (&x)[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) { x[2 * t] = bf_lo(a[t]); x[2 * t + 1] = bf_hi(a[t]); }
}

__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(
    const uint16_t* dq, const uint16_t* dk, const uint16_t* dv, int64_t ld_g, const uint16_t* qk_pre,
    int64_t ld_pre, const uint16_t* v, int64_t ld_v, const float* r1, const float* gq, const float* gk,
    const float* table, int seq_len, float eps, int M, int D, int rows_per_wave, uint16_t* dh, int64_t ld_dh,
    float* T1, float* pgq, float* pgk) {
  // One wave per row.  A head (128 columns) is handled by 16 lanes, 8
  // consecutive columns (4 RoPE pairs) a lane, so a wave covers 4 heads per
  // 16-byte access; per-head sums reduce over the 16-lane group.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 15, slot = lane >> 4;
  const int H = D / 128;
  float g[2][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { g[0][e] = gq[8 * sub + e]; g[1][e] = gk[8 * sub + e]; }
  float dgacc[2][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dgacc[0][e] = dgacc[1][e] = 0.0f;
  for (int rr = 0; rr < rows_per_wave; ++rr) {
    const int m = (blockIdx.x * 4 + wave) * rows_per_wave + rr;
    if (m >= M) break;
    const float r = r1 ? r1[m] : 1.0f;     // no r1: plain (unfused) QK-norm backward
    const int pos = m % seq_len;
    // (cos, sin) of the lane's 4 frequencies 4 sub .. 4 sub + 3
    const float4 cs01 = *reinterpret_cast<const float4*>(table + ((int64_t)pos * 64 + 4 * sub) * 2);
    const float4 cs23 = *reinterpret_cast<const float4*>(table + ((int64_t)pos * 64 + 4 * sub) * 2 + 4);
    const float cs[4][2] = {{cs01.x, cs01.y}, {cs01.z, cs01.w}, {cs23.x, cs23.y}, {cs23.z, cs23.w}};
    float T = 0.0f;
#pragma unroll
    for (int reg = 0; reg < 2; ++reg) {
      const uint16_t* G = reg == 0 ? dq : dk;
      for (int h0 = 0; h0 < H; h0 += 4) {
        const int h = h0 + slot;
        const bool on = h < H;                 // whole 16-lane groups switch off together
        const int col = h * 128 + 8 * sub;
        float d[8], u[8];
        if (on) {
          unpack8(*reinterpret_cast<const uint4*>(G + (int64_t)m * ld_g + col), d);
          unpack8(*reinterpret_cast<const uint4*>(qk_pre + (int64_t)m * ld_pre + reg * D + col), u);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) d[e] = u[e] = 0.0f;
        }
        // inverse rotation (transpose of the forward RoPE matrix)
        float n[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          n[2 * p] = d[2 * p] * cs[p][0] + d[2 * p + 1] * cs[p][1];
          n[2 * p + 1] = -d[2 * p] * cs[p][1] + d[2 * p + 1] * cs[p][0];
        }
        float ss = 0.0f, st = 0.0f, t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          t[e] = g[reg][e] * n[e];
          ss += u[e] * u[e];
          st += u[e] * t[e];
        }
        ss = sum16(ss);
        st = sum16(st);
        const float rho = rsqrtf(ss / 128.0f + eps);
        const float k3 = rho * rho * rho / 128.0f * st;
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[q] = pack_bf2(r * (rho * t[2 * q] - k3 * u[2 * q]), r * (rho * t[2 * q + 1] - k3 * u[2 * q + 1]));
          T += bf_lo(o[q]) * u[2 * q] + bf_hi(o[q]) * u[2 * q + 1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) dgacc[reg][e] += rho * u[e] * n[e];
        if (on) *reinterpret_cast<uint4*>(dh + (int64_t)m * ld_dh + reg * D + col) = uint4{o[0], o[1], o[2], o[3]};
      }
    }
    for (int col = lane * 8; col < D; col += 512) {
      uint4 gw = *reinterpret_cast<const uint4*>(dv + (int64_t)m * ld_g + col);
      uint4 vw = *reinterpret_cast<const uint4*>(v + (int64_t)m * ld_v + col);
      uint32_t ga[4] = {gw.x, gw.y, gw.z, gw.w}, va[4] = {vw.x, vw.y, vw.z, vw.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[q] = pack_bf2(r * bf_lo(ga[q]), r * bf_hi(ga[q]));
        T += bf_lo(o[q]) * bf_lo(va[q]) + bf_hi(o[q]) * bf_hi(va[q]);
      }
      *reinterpret_cast<uint4*>(dh + (int64_t)m * ld_dh + 2 * D + col) = uint4{o[0], o[1], o[2], o[3]};
    }
    T = wave_sum(T);
    if (lane == 0) T1[m] = T;
  }
  // gain-gradient partials of this block, in a fixed order: the 4 head slots
  // of a wave (lanes sub, sub + 16, sub + 32, sub + 48), then the 4 waves
#pragma unroll
  for (int reg = 0; reg < 2; ++reg)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = dgacc[reg][e];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      dgacc[reg][e] = x;
    }
  __shared__ float red[4][2][128];
  if (slot == 0)
#pragma unroll
    for (int reg = 0; reg < 2; ++reg)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][reg][8 * sub + e] = dgacc[reg][e];
  __syncthreads();
  const int tt = threadIdx.x;   // 256 threads: (region, column)
  const int reg = tt >> 7, cidx = tt & 127;
  float sacc = (red[0][reg][cidx] + red[1][reg][cidx]) + (red[2][reg][cidx] + red[3][reg][cidx]);
  (reg == 0 ? pgq : pgk)[(int64_t)blockIdx.x * 128 + cidx] = sacc;
}

__device__ __forceinline__ void lse_merge_(float& m, float& s, float m2, float s2) {
  float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
  m = mm;
}

__global__ void ce_finish_rows_kernel(const float* Pm, const float* Ps, int nT, int M,
                                      const float* zy, const int* labels, int V, int ignore_index,
                                      float* lse, float* per_row, int* status) {
  // 256 threads = 64 rows x 4 partial groups
  __shared__ float rm[4][64], rs[4][64];
  const int rloc = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int m = blockIdx.x * 64 + rloc;
  float mx = -INFINITY, s = 0.0f;
  if (m < M)
    for (int t = grp; t < nT; t += 4) lse_merge_(mx, s, Pm[(int64_t)t * M + m], Ps[(int64_t)t * M + m]);
  rm[grp][rloc] = mx;
  rs[grp][rloc] = s;
  __syncthreads();
  if (grp == 0 && m < M) {
    for (int g = 1; g < 4; ++g) lse_merge_(mx, s, rm[g][rloc], rs[g][rloc]);
    const float l = mx + __logf(s);
    lse[m] = l;
    const int y = labels[m];
    int st = 0;
    float pr = 0.0f;
    if (y == ignore_index) st = 1;
    else if (y < 0 || y >= V) st = 2;
    else pr = l - zy[m];
    per_row[m] = pr;
    status[m] = st;
  }
}

__global__ void ce_finish_loss_kernel(const float* per_row, const int* status, int M, float* loss,
                                      int* n_valid, int* n_bad) {
  __shared__ float rsum[1024];
  __shared__ int rcnt[1024], rbad[1024];
  const int t = threadIdx.x;
  float s = 0.0f;
  int cnt = 0, bad = 0;
  for (int m = t; m < M; m += blockDim.x) {
    const int st = status[m];
    if (st == 0) { s += per_row[m]; ++cnt; }
    else if (st == 2) ++bad;
  }
  rsum[t] = s; rcnt[t] = cnt; rbad[t] = bad;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (t < w) { rsum[t] += rsum[t + w]; rcnt[t] += rcnt[t + w]; rbad[t] += rbad[t + w]; }
    __syncthreads();
  }
  if (t == 0) {
    *loss = rsum[0] / (float)rcnt[0];   // 0 / 0 = NaN for an empty batch
    *n_valid = rcnt[0];
    if (n_bad) *n_bad = rbad[0];
  }
}

// out[r, c] = bf16(X[r, c]) for fp32 X (C % 4 == 0), 4 values a thread
__global__ void f32_to_bf16_kernel(const float* X, int64_t ldx, uint16_t* out, int64_t ldo, int R, int C) {
  for (int r = blockIdx.y; r < R; r += gridDim.y)
    for (int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4; c < C; c += gridDim.x * blockDim.x * 4) {
      const float4 v = *reinterpret_cast<const float4*>(X + (int64_t)r * ldx + c);
      *reinterpret_cast<uint2*>(out + (int64_t)r * ldo + c) = uint2{pack_bf2(v.x, v.y), pack_bf2(v.z, v.w)};
    }
}

__global__ void fill_f32_kernel(float* out, int n, float v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) out[i] = v;
}

__global__ void scale_f32_kernel(float* out, int64_t ld, int R, int C, float beta) {
  for (int r = blockIdx.y; r < R; r += gridDim.y)
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < C; c += gridDim.x * blockDim.x) {
      float* p = out + (int64_t)r * ld + c;
      *p = beta != 0.0f ? beta * *p : 0.0f;
    }
}

__global__ void norm_corr_finish_kernel(const float* acc, int64_t lda, const uint16_t* y, int64_t ldy, const float* cr,
                                        const float* scale, const uint16_t* res, int64_t ldr, uint16_t* out,
                                        int64_t ldo, int R, int C) {
  for (int r = blockIdx.y; r < R; r += gridDim.y) {
    const float sc = *scale * cr[r];
    for (int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4; c < C; c += gridDim.x * blockDim.x * 4) {
      const float4 a = *reinterpret_cast<const float4*>(acc + (int64_t)r * lda + c);
      const uint2 yw = *reinterpret_cast<const uint2*>(y + (int64_t)r * ldy + c);
      float v[4] = {a.x - sc * bf_lo(yw.x), a.y - sc * bf_hi(yw.x), a.z - sc * bf_lo(yw.y), a.w - sc * bf_hi(yw.y)};
      if (res) {
        const uint2 rw = *reinterpret_cast<const uint2*>(res + (int64_t)r * ldr + c);
        v[0] += bf_lo(rw.x); v[1] += bf_hi(rw.x); v[2] += bf_lo(rw.y); v[3] += bf_hi(rw.y);
      }
      *reinterpret_cast<uint2*>(out + (int64_t)r * ldo + c) = uint2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
    }
  }
}

__global__ void ce_scale_kernel(const int* n_valid, float dloss, float* scale) {
  const int n = *n_valid;
  *scale = n > 0 ? dloss / (float)n : 0.0f;
}

// ---------------------------------------------------------------- fp8 quantisation
__device__ __forceinline__ float absmax_bf2(uint32_t w, float m) {
  return fmaxf(m, fmaxf(fabsf(bf_lo(w)), fabsf(bf_hi(w))));
}
__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }
// 4 floats -> 4 E4M3 bytes (round to nearest even by the hardware convert)
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return (uint32_t)w;
}

__global__ void amax_cols_partial_kernel(const uint16_t* X, int64_t ld, int R, int C, int rows_per_block,
                                         float* part) {
  // thread owns 2 columns; block covers 512 columns x rows_per_block rows
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 2;
  const int r0 = blockIdx.y * rows_per_block;
  if (c >= C) return;
  float m0 = 0.0f, m1 = 0.0f;
  for (int r = r0; r < min(R, r0 + rows_per_block); ++r) {
    uint32_t v = *reinterpret_cast<const uint32_t*>(X + (int64_t)r * ld + c);
    m0 = fmaxf(m0, fabsf(bf_lo(v)));
    m1 = fmaxf(m1, fabsf(bf_hi(v)));
  }
  part[(int64_t)blockIdx.y * C + c] = m0;
  part[(int64_t)blockIdx.y * C + c + 1] = m1;
}

__global__ void amax_cols_finish_kernel(const float* part, int nparts, int C, float* amax) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float m = 0.0f;
  for (int t = 0; t < nparts; ++t) m = fmaxf(m, part[(int64_t)t * C + c]);
  amax[c] = m;
}

__global__ void quant_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                  float* scale) {
  // one wave a row: the row's amax, then its codes; the second read of the
  // row comes from cache, not from a second pass over the whole matrix
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (r >= R) return;
  const uint16_t* x = X + (int64_t)r * ld;
  float m = 0.0f;
  for (int c = lane * 8; c < C; c += 512) {
    uint4 w = *reinterpret_cast<const uint4*>(x + c);
    m = absmax_bf2(w.x, absmax_bf2(w.y, absmax_bf2(w.z, absmax_bf2(w.w, m))));
  }
  float a = wave_max(m);
  if (!(a > 0.0f)) a = 448.0f;
  const float mult = 448.0f / a;
  if (lane == 0) scale[r] = a / 448.0f;
  for (int c = lane * 8; c < C; c += 512) {
    uint4 w = *reinterpret_cast<const uint4*>(x + c);
    uint32_t lo = cvt4_e4m3(bf_lo(w.x) * mult, bf_hi(w.x) * mult, bf_lo(w.y) * mult, bf_hi(w.y) * mult);
    uint32_t hi = cvt4_e4m3(bf_lo(w.z) * mult, bf_hi(w.z) * mult, bf_lo(w.w) * mult, bf_hi(w.w) * mult);
    *reinterpret_cast<uint2*>(Q + (int64_t)r * ldq + c) = uint2{lo, hi};
  }
  // C is a multiple of 8: zero the bytes up to the row's next 16-byte
  // boundary, which the GEMM's last 16-byte K chunk reads (ldq >= that
  // boundary: ldq is a multiple of 16)
  if ((C & 15) != 0 && lane == 0) *reinterpret_cast<uint2*>(Q + (int64_t)r * ldq + C) = uint2{0u, 0u};
}

// The 64 x 64 bf16 tile X[r0 .., c0 ..] as floats in LDS (positions outside
// the matrix read 0), for the transposing quantisers: 16-byte loads along X's
// rows (C % 8 == 0, so a chunk of 8 is wholly in or out), two a thread of
// 256.  Thread i fills row i / 8, columns 8 (i % 8) .. + 7; with a row stride
// of 65 floats the 64 lanes of one store instruction hit 64 distinct banks.
__device__ __forceinline__ void load_tile_t(const uint16_t* X, int64_t ld, int R, int C, int r0, int c0,
                                            float (*tile)[65]) {
  for (int i = threadIdx.x; i < 512; i += blockDim.x) {
    const int rr = i >> 3, cc = (i & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    uint4 w = {0u, 0u, 0u, 0u};
    if (r < R && c < C) w = *reinterpret_cast<const uint4*>(X + (int64_t)r * ld + c);
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[rr][cc + 2 * j] = bf_lo(v[j]);
      tile[rr][cc + 2 * j + 1] = bf_hi(v[j]);
    }
  }
  __syncthreads();
}

__global__ void quant_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, const float* amax,
                                    uint8_t* QT, int64_t ldq, float* scale) {
  // 64 x 64 tile through LDS: read X[r0.., c0..] rows, write QT[c][r0..r0+63]
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  load_tile_t(X, ld, R, C, r0, c0, tile);
  // thread -> (column cc, 16 consecutive rows)
  const int cc = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int c = c0 + cc;
  if (c >= C) return;
  float a = amax[c];
  if (!(a > 0.0f)) a = 448.0f;
  const float mult = 448.0f / a;
  if (blockIdx.y == 0 && part == 0) scale[c] = a / 448.0f;
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = part * 16 + 4 * k;
    w[k] = cvt4_e4m3(tile[rr][cc] * mult, tile[rr + 1][cc] * mult, tile[rr + 2][cc] * mult, tile[rr + 3][cc] * mult);
  }
  // Rows at or past R were loaded as 0 and encode as byte 0, so the last
  // 16-byte group of a QT row also zeroes the bytes between R and the next
  // 16-byte boundary, which the GEMM's last 16-byte K chunk reads (ldq is a
  // multiple of 16, so that boundary lies inside the row).
  const int rbase = r0 + part * 16;
  if (rbase < R) *reinterpret_cast<uint4*>(QT + (int64_t)c * ldq + rbase) = uint4{w[0], w[1], w[2], w[3]};
}

// ---------------------------------------------------------------- MXFP8 (block-scaled E4M3)
// OCP Microscaling Formats (MX) v1.0, MXFP8 with E4M3 elements: a block of 32
// consecutive values along the contracted axis shares one E8M0 scale 2^e.
// e = floor(log2(max |v|)) - 8 (8 = the exponent of E4M3's largest power of
// two), clamped to [-127, 127]; a block whose max is zero or an fp32
// subnormal takes -127.  Elements are E4M3(v / 2^e), round to nearest even,
// saturated at +-448.
__device__ __forceinline__ int mx_exponent(float amax) {
  const int be = (int)((__float_as_uint(amax) >> 23) & 0xFF);   // biased exponent, 0 for zero / subnormal
  return be == 0 ? -127 : min(max(be - 127 - 8, -127), 127);
}

// 4 floats scaled by 2^-e (exact) -> 4 E4M3 bytes
__device__ __forceinline__ uint32_t cvt4_mx(float a, float b, float c, float d, int e) {
  return cvt4_e4m3(ldexpf(a, -e), ldexpf(b, -e), ldexpf(c, -e), ldexpf(d, -e));
}

// Exponents go to word layout: block b of operand row r is byte
// S[(b / 4) lds + 4 r + b % 4], so the words of one 128-value K range of
// consecutive rows are contiguous.
// Blocks along the columns: X [R, C] -> Q [R, C], exponents of R rows
// (C % 32 == 0).  One wave a row, 8 values a lane, a block = 4 consecutive
// lanes.
__global__ void quant_mx_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                     uint8_t* S, int64_t lds) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (r >= R) return;                      // r is uniform over the wave
  for (int c = lane * 8; c < C; c += 512) {
    // C % 32 == 0: the 4 lanes of a block run the same iterations
    const uint4 w = *reinterpret_cast<const uint4*>(X + (int64_t)r * ld + c);
    float m = absmax_bf2(w.x, absmax_bf2(w.y, absmax_bf2(w.z, absmax_bf2(w.w, 0.0f))));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    const int e = mx_exponent(m);
    const uint32_t lo = cvt4_mx(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), e);
    const uint32_t hi = cvt4_mx(bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w), e);
    *reinterpret_cast<uint2*>(Q + (int64_t)r * ldq + c) = uint2{lo, hi};
    const int b = c / 32;
    if ((lane & 3) == 0) S[(int64_t)(b >> 2) * lds + 4 * r + (b & 3)] = (uint8_t)(e + 127);
  }
}

// Blocks along the rows, written transposed: X [R, C] -> Q^T [C, R],
// exponents of C rows (R % 32 == 0).  A 64 x 64 tile goes through LDS; thread
// (column cc, part) encodes rows [16 part, 16 part + 16) of its column, and
// a block is the two parts of one lane pair.
__global__ void quant_mx_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* QT, int64_t ldq,
                                       uint8_t* S, int64_t lds) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  load_tile_t(X, ld, R, C, r0, c0, tile);
  const int cc = threadIdx.x >> 2, part = threadIdx.x & 3;
  float v[16];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    v[k] = tile[part * 16 + k][cc];
    m = fmaxf(m, fabsf(v[k]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));      // every lane is still active here
  const int e = mx_exponent(m);
  const int c = c0 + cc, rbase = r0 + part * 16;
  if (c >= C || rbase >= R) return;        // R % 32 == 0: rows rbase .. rbase + 15 all exist
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = cvt4_mx(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3], e);
  *reinterpret_cast<uint4*>(QT + (int64_t)c * ldq + rbase) = uint4{w[0], w[1], w[2], w[3]};
  const int b = rbase / 32;
  if ((part & 1) == 0) S[(int64_t)(b >> 2) * lds + 4 * c + (b & 3)] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------- MXFP4 (block-scaled E2M1)
// OCP MX v1.0 FP4 E2M1 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
// negatives) under one E8M0 exponent per 32 values:
// e = floor(log2(max |v|)) - 2 (2 = the exponent of 4, E2M1's largest power
// of two), clamped to [-127, 127], -127 for a zero or subnormal maximum.
__device__ __forceinline__ int mx4_exponent(float amax) {
  const int be = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  return be == 0 ? -127 : min(max(be - 127 - 2, -127), 127);
}

// E2M1 code of v (already divided by the block scale): the nearest value,
// ties to the even mantissa, saturated at 6; a value that rounds to zero is
// code 0.  Each comparison climbs one step of the value ladder; its
// threshold is the midpoint of the two neighbours, passed strictly (>) when
// the lower neighbour has the even mantissa and inclusively (>=) when the
// upper one has.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((v < 0.0f && c != 0u) ? 8u : 0u);
}

// 8 values scaled by 2^-e (exact) -> 8 packed codes, value k in nibble k
__device__ __forceinline__ uint32_t pack8_e2m1(const float* v, int e) {
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) w |= e2m1_code(ldexpf(v[k], -e)) << (4 * k);
  return w;
}

// Blocks along the columns: X [R, C] -> Q [R, C / 2] bytes, exponents of R
// rows in word layout (C % 32 == 0).  One wave a row, 8 values a lane, a
// block = 4 consecutive lanes.
__global__ void quant_mx4_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                      uint8_t* S, int64_t lds) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (r >= R) return;                      // r is uniform over the wave
  for (int c = lane * 8; c < C; c += 512) {
    // C % 32 == 0: the 4 lanes of a block run the same iterations
    const uint4 w = *reinterpret_cast<const uint4*>(X + (int64_t)r * ld + c);
    float m = absmax_bf2(w.x, absmax_bf2(w.y, absmax_bf2(w.z, absmax_bf2(w.w, 0.0f))));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    const int e = mx4_exponent(m);
    const float v[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
    *reinterpret_cast<uint32_t*>(Q + (int64_t)r * ldq + c / 2) = pack8_e2m1(v, e);
    const int b = c / 32;
    if ((lane & 3) == 0) S[(int64_t)(b >> 2) * lds + 4 * r + (b & 3)] = (uint8_t)(e + 127);
  }
}

// Blocks along the rows, written transposed: X [R, C] -> Q^T [C, R / 2]
// bytes, exponents of C rows (R % 32 == 0).  As quant_mx_cols_t_kernel: a
// 64 x 64 tile through LDS, thread (column cc, part) encodes rows
// [16 part, 16 part + 16) of its column, a block is one lane pair.
__global__ void quant_mx4_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* QT, int64_t ldq,
                                        uint8_t* S, int64_t lds) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  load_tile_t(X, ld, R, C, r0, c0, tile);
  const int cc = threadIdx.x >> 2, part = threadIdx.x & 3;
  float v[16];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    v[k] = tile[part * 16 + k][cc];
    m = fmaxf(m, fabsf(v[k]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));      // every lane is still active here
  const int e = mx4_exponent(m);
  const int c = c0 + cc, rbase = r0 + part * 16;
  if (c >= C || rbase >= R) return;        // R % 32 == 0: rows rbase .. rbase + 15 all exist
  *reinterpret_cast<uint2*>(QT + (int64_t)c * ldq + rbase / 2) = uint2{pack8_e2m1(v, e), pack8_e2m1(v + 8, e)};
  const int b = rbase / 32;
  if ((part & 1) == 0) S[(int64_t)(b >> 2) * lds + 4 * c + (b & 3)] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------- MXFP6 (block-scaled E2M3 / E3M2)
// OCP MX v1.0 FP6 elements under one E8M0 exponent per 32 values: E2M3 (bias
// 1, largest 7.5 = 1.875 * 2^2) and E3M2 (bias 3, largest 28 = 1.75 * 2^4),
// e = floor(log2(max |v|)) - emax with emax = 2 or 4, clamped to
// [-127, 127], -127 for a zero or subnormal maximum.  A block's 32 codes are
// packed into 24 bytes, code v at bits [6 v, 6 v + 6) of one little-endian
// 192-bit number, followed by 8 zero bytes: a row of L values is L bytes and
// every block starts on a 32-byte boundary.
template <int EB, int MB>
struct Fp6Fmt {
  static constexpr int BIAS = (1 << (EB - 1)) - 1;
  static constexpr int EMAX = (1 << EB) - 1 - BIAS;
};

template <int EB, int MB>
__device__ __forceinline__ int mx6_exponent(float amax) {
  const int be = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  return be == 0 ? -127 : min(max(be - 127 - Fp6Fmt<EB, MB>::EMAX, -127), 127);
}

// FP6 code of v (already divided by the block scale): nearest value, ties to
// the even mantissa, saturated at the largest.  With k = floor(log2 |v|),
// raised to the exponent of the smallest normal so that subnormals share the
// lowest binade's step 2^(k - MB), r = |v| / 2^(k - MB) rounded half to even
// is the significand in units of that step; the code's magnitude is then
// (k + BIAS - 1) 2^MB + r, which carries into the next binade when r reaches
// 2^(MB + 1) and is the plain subnormal code when k is the lowest exponent.
template <int EB, int MB>
__device__ __forceinline__ uint32_t fp6_code(float v) {
  constexpr int B = Fp6Fmt<EB, MB>::BIAS;
  const float a = fabsf(v);
  const int k = max((int)((__float_as_uint(a) >> 23) & 0xFF) - 127, 1 - B);
  const int r = (int)rintf(ldexpf(a, MB - k));
  const uint32_t c = (uint32_t)min(((k + B - 1) << MB) + r, 31);
  return c | ((v < 0.0f && c != 0u) ? 32u : 0u);
}

// 8 values scaled by 2^-e (exact) -> 48 bits, value k at bits [6 k, 6 k + 6)
template <int EB, int MB>
__device__ __forceinline__ uint64_t pack8_fp6(const float* v, int e) {
  uint64_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) w |= (uint64_t)fp6_code<EB, MB>(ldexpf(v[k], -e)) << (6 * k);
  return w;
}

// two 48-bit groups (lo first) -> the three words of their 96 bits
__device__ __forceinline__ void store96(uint8_t* dst, uint64_t lo, uint64_t hi) {
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  d[0] = (uint32_t)lo;
  d[1] = (uint32_t)(lo >> 32) | (uint32_t)(hi << 16);
  d[2] = (uint32_t)(hi >> 16);
}

// Blocks along the columns: X [R, C] -> Q [R, C] bytes.  One wave a row, 8
// values a lane, a block = 4 consecutive lanes; lane q of a block packs
// values 8 q .. 8 q + 7 into 48 bits, and the even lane of each pair stores
// the pair's 96 bits (bytes 12 (q / 2) .. of the block).
template <int EB, int MB>
__device__ __forceinline__ void quant_mx6_rows(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                               uint8_t* S, int64_t lds) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (r >= R) return;                      // r is uniform over the wave
  for (int c = lane * 8; c < C; c += 512) {
    // C % 32 == 0: the 4 lanes of a block run the same iterations
    const uint4 w = *reinterpret_cast<const uint4*>(X + (int64_t)r * ld + c);
    float m = absmax_bf2(w.x, absmax_bf2(w.y, absmax_bf2(w.z, absmax_bf2(w.w, 0.0f))));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    const int e = mx6_exponent<EB, MB>(m);
    const float v[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
    const uint64_t p = pack8_fp6<EB, MB>(v, e);
    const uint32_t nlo = __shfl_xor((uint32_t)p, 1, 64), nhi = __shfl_xor((uint32_t)(p >> 32), 1, 64);
    const int q = lane & 3;
    uint8_t* blk = Q + (int64_t)r * ldq + (c - 8 * q);
    if ((q & 1) == 0) store96(blk + 12 * (q >> 1), p, ((uint64_t)nhi << 32) | nlo);
    if (q == 3) *reinterpret_cast<uint2*>(blk + 24) = uint2{0u, 0u};
    const int b = c / 32;
    if (q == 0) S[(int64_t)(b >> 2) * lds + 4 * r + (b & 3)] = (uint8_t)(e + 127);
  }
}

// Blocks along the rows, written transposed: X [R, C] -> Q^T [C, R] bytes.
// As quant_mx_cols_t_kernel: a 64 x 64 tile through LDS, thread (column cc,
// part) encodes rows [16 part, 16 part + 16) of its column into 96 bits, a
// block is one lane pair, and the odd part also writes the block's padding.
template <int EB, int MB>
__device__ __forceinline__ void quant_mx6_cols_t(const uint16_t* X, int64_t ld, int R, int C, uint8_t* QT,
                                                 int64_t ldq, uint8_t* S, int64_t lds, float (*tile)[65]) {
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  load_tile_t(X, ld, R, C, r0, c0, tile);
  const int cc = threadIdx.x >> 2, part = threadIdx.x & 3;
  float v[16];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    v[k] = tile[part * 16 + k][cc];
    m = fmaxf(m, fabsf(v[k]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));      // every lane is still active here
  const int e = mx6_exponent<EB, MB>(m);
  const int c = c0 + cc, rbase = r0 + part * 16;
  if (c >= C || rbase >= R) return;        // R % 32 == 0: rows rbase .. rbase + 15 all exist
  uint8_t* blk = QT + (int64_t)c * ldq + (rbase - 16 * (part & 1));
  store96(blk + 12 * (part & 1), pack8_fp6<EB, MB>(v, e), pack8_fp6<EB, MB>(v + 8, e));
  if (part & 1) *reinterpret_cast<uint2*>(blk + 24) = uint2{0u, 0u};
  const int b = rbase / 32;
  if ((part & 1) == 0) S[(int64_t)(b >> 2) * lds + 4 * c + (b & 3)] = (uint8_t)(e + 127);
}

__global__ void quant_mx6_rows_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* Q, int64_t ldq,
                                      uint8_t* S, int64_t lds, int f6) {
  if (f6 == 2) quant_mx6_rows<2, 3>(X, ld, R, C, Q, ldq, S, lds);
  else quant_mx6_rows<3, 2>(X, ld, R, C, Q, ldq, S, lds);
}

__global__ void quant_mx6_cols_t_kernel(const uint16_t* X, int64_t ld, int R, int C, uint8_t* QT, int64_t ldq,
                                        uint8_t* S, int64_t lds, int f6) {
  __shared__ float tile[64][65];
  if (f6 == 2) quant_mx6_cols_t<2, 3>(X, ld, R, C, QT, ldq, S, lds, tile);
  else quant_mx6_cols_t<3, 2>(X, ld, R, C, QT, ldq, S, lds, tile);
}

}  // namespace coda
