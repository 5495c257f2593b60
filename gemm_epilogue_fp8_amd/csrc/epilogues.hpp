// Epilogue primitives and the composed epilogue programs.
//
// The CODA paper (arXiv 2605.19269), §3.1, names five primitive classes that
// an epilogue may apply to the output tile while it is still on chip:
//   P1 elementwise / pairwise maps (residual update, activation, RoPE, SwiGLU),
//   P2 rank-1 vector loads / stores broadcast over the tile,
//   P3 rank-2 tile loads / stores (residual stream, saved activations),
//   P4 tile row reductions written as partials and merged later,
//   P5 running state (online max / sum-exp for log-sum-exp).
// §2.2 adds the locality rule: an epilogue sees its tile, its accumulator and
// consistently indexed auxiliaries only, so a reduction wider than the tile
// becomes per-tile partials finished elsewhere.
//
// Here each primitive is a small device function over the accumulator
// fragment that the mainloop leaves in registers.  Lane l of the wave at
// (wm0, wn0) holds, for MFMA tile (i, j) and group q, row
//   m = m0 + wm0 + 32 i + (l & 31)
// and the 4 consecutive columns
//   n = n0 + wn0 + 32 j + 8 q + 4 (l >> 5) + {0,1,2,3}
// in acc.c[i][j][4 q + {0..3}].  A row of the workgroup tile is spread over
// lanes l and l ^ 32 of WAVES_N waves: row reductions add in-lane, then
// across the lane pair, then across waves through LDS in a fixed order (no
// atomics, bitwise deterministic).
//
// The programs (structs below) compose the primitives for the GEMMs of the
// reparameterised block (forward F1-F4, backward B1-B8), config-1 SwiGLU,
// and linear + cross-entropy (C1-C4).
#pragma once
#include "gemm_core.hpp"

namespace coda {

struct EpiArgs {
  void* out;  int64_t ld_out;          // main output tile store
  void* out2; int64_t ld_out2;         // second output (k of QKV)
  void* out3; int64_t ld_out3;         // third output (v of QKV)
  const void* aux0; int64_t ld_aux0;   // rank-2 tile operand 0
  const void* aux1; int64_t ld_aux1;   // rank-2 tile operand 1
  void* save; int64_t ld_save;         // rank-2 tile store of pre-activations
  const float* row_partials;           // [n_row_partials][M] partials finished in the prologue
  int n_row_partials;
  const float* rowvec;                 // [M] row vector
  const float* rowscale;               // [M] fp8 row (activation) scales
  const float* colscale;               // [N] fp8 column (weight) scales
  const float* colvec;                 // per-column / per-head-column gain
  const float* colvec2;                // second gain (k of QKV)
  const float* table;                  // RoPE [seq_len][64][2] (cos, sin)
  const int* labels;                   // [M] int32 labels
  float* partial_out;                  // [tiles_n][M] row partials
  float* partial_out2;                 // second partial (sum-exp)
  float* rowvec_out;                   // [M] row vector output
  const float* alpha_dev;              // device scalar multiplier or null
  float alpha, beta, eps;
  int norm_dim;                        // D of the norm being finished
  int region;                          // QKV: width D of each of q, k, v
  int seq_len;
  int vocab;                           // CE: valid column count
};

template <class Cfg>
struct Ctx {
  int m0, n0, wm0, wn0, lane, tid, wn, M, N, tn;
  char* smem;
  __device__ __forceinline__ int lrow(int i) const { return wm0 + 32 * i + (lane & 31); }
  __device__ __forceinline__ int row(int i) const { return m0 + lrow(i); }
  __device__ __forceinline__ int col(int j, int q) const { return n0 + wn0 + 32 * j + 8 * q + 4 * (lane >> 5); }
  // LDS after the mainloop: [0, 2 BM) row vectors, then [WAVES_N][BM] reduction scratch
  __device__ __forceinline__ float* rowv() const { return reinterpret_cast<float*>(smem); }
  __device__ __forceinline__ float* rowv2() const { return reinterpret_cast<float*>(smem) + Cfg::BM; }
  __device__ __forceinline__ float* red() const { return reinterpret_cast<float*>(smem) + 2 * Cfg::BM; }
  __device__ __forceinline__ float* red2() const { return reinterpret_cast<float*>(smem) + (2 + Cfg::WAVES_N) * Cfg::BM; }
};

// ---------------------------------------------------------------- P3 tile loads / stores
__device__ __forceinline__ f32x4_t load_bf16x4(const void* base, int64_t ld, int m, int n) {
  uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + (int64_t)m * ld + n);
  return f32x4_t{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
}
__device__ __forceinline__ void store_bf16x4(void* base, int64_t ld, int m, int n, f32x4_t v) {
  uint2 w = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + (int64_t)m * ld + n) = w;
}
__device__ __forceinline__ f32x4_t load_f32x4(const void* base, int64_t ld, int m, int n) {
  return *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + (int64_t)m * ld + n);
}
__device__ __forceinline__ void store_f32x4(void* base, int64_t ld, int m, int n, f32x4_t v) {
  *reinterpret_cast<f32x4_t*>(static_cast<float*>(base) + (int64_t)m * ld + n) = v;
}
__device__ __forceinline__ f32x4_t round_bf4(f32x4_t v) {
  return f32x4_t{round_bf(v[0]), round_bf(v[1]), round_bf(v[2]), round_bf(v[3])};
}

template <class Cfg>
__device__ __forceinline__ f32x4_t frag(const Acc<Cfg>& acc, int i, int j, int q) {
  return f32x4_t{acc.c[i][j][4 * q], acc.c[i][j][4 * q + 1], acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3]};
}
template <class Cfg>
__device__ __forceinline__ void set_frag(Acc<Cfg>& acc, int i, int j, int q, f32x4_t v) {
#pragma unroll
  for (int t = 0; t < 4; ++t) acc.c[i][j][4 * q + t] = v[t];
}

// ---------------------------------------------------------------- P2 vector loads: fp8 dequant scales
// acc <- acc * s_row[m] * s_col[n] (the per-token and per-channel E4M3 scales)
template <class Cfg>
__device__ __forceinline__ void apply_fp8_scales(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc) {
  if constexpr (Cfg::FP8) {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      int m = c.row(i);
      float sr = m < c.M ? e.rowscale[m] : 0.0f;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int n = c.col(j, q);
          f32x4_t sc = n < c.N ? *reinterpret_cast<const f32x4_t*>(e.colscale + n) : f32x4_t{0, 0, 0, 0};
#pragma unroll
          for (int t = 0; t < 4; ++t) acc.c[i][j][4 * q + t] = (acc.c[i][j][4 * q + t] * sr) * sc[t];
        }
    }
  }
}

// ---------------------------------------------------------------- P4 row reduction over the tile
// part[i] is this lane's share of local row lrow(i); writes the tile total of
// every local row to out[BM] (LDS) in a fixed order.
template <class Cfg>
__device__ __forceinline__ void row_sum_tile(const Ctx<Cfg>& c, float (&part)[Cfg::TM], float* out) {
  float* red = c.red();
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
    float s = part[i] + __shfl_xor(part[i], 32, 64);
    if ((c.lane >> 5) == 0) red[c.wn * Cfg::BM + c.lrow(i)] = s;
  }
  __syncthreads();
  for (int r = c.tid; r < Cfg::BM; r += Cfg::T) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < Cfg::WAVES_N; ++w) s += red[w * Cfg::BM + r];
    out[r] = s;
  }
  __syncthreads();
}

// Writes a per-(N tile, row) partial P[tn][m] for the tile's rows.
template <class Cfg>
__device__ __forceinline__ void write_row_partial(const Ctx<Cfg>& c, const float* tot, float* P) {
  for (int r = c.tid; r < Cfg::BM; r += Cfg::T) {
    int m = c.m0 + r;
    if (m < c.M) P[(int64_t)c.tn * c.M + m] = tot[r];
  }
}

// ---------------------------------------------------------------- prologue: finish row partials
// Loads P[t][m0 + r] for every t < nP before the mainloop (up to MAXP values a
// thread, all loads independent) and after it reduces them into LDS.
template <class Cfg>
struct RowPartials {
  static constexpr int TPR = Cfg::T / Cfg::BM;   // threads per row
  static constexpr int MAXP = 16;                // partials per thread
  static constexpr int MAX_PARTIALS = MAXP * TPR;
  float v[MAXP];
  __device__ __forceinline__ void issue(const float* P, int nP, const Ctx<Cfg>& c) {
    const int r = c.tid % Cfg::BM, t0 = c.tid / Cfg::BM, m = c.m0 + r;
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      int t = t0 + k * TPR;
      v[k] = (P != nullptr && t < nP && m < c.M) ? P[(int64_t)t * c.M + m] : 0.0f;
    }
  }
  // out[r] = sum over t of P[t][m0 + r]
  __device__ __forceinline__ void reduce(const Ctx<Cfg>& c, float* out) const {
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < MAXP; ++k) s += v[k];
    float* red = c.red();
    red[c.tid] = s;
    __syncthreads();
    if (c.tid < Cfg::BM) {
      float tsum = 0.0f;
#pragma unroll
      for (int t = 0; t < TPR; ++t) tsum += red[t * Cfg::BM + c.tid];
      out[c.tid] = tsum;
    }
    __syncthreads();
  }
};

// ================================================================ programs

// --- Linear chain: [row scale] [col scale] [alpha] [+ tile] -> store [+ sum-of-squares partial]
enum : int {
  EL_ROWVEC = 1,    // P2: multiply by rowvec[m]
  EL_COLVEC = 2,    // P2: multiply by colvec[n]
  EL_TILEADD = 4,   // P3: + aux0[m, n] (bf16)
  EL_SUMSQ = 8,     // P4: partial_out[tn][m] = sum over the tile of bf16(value)^2
  EL_F32OUT = 16,   // store fp32 as beta * out + value (else bf16)
  EL_ALPHADEV = 32, // multiply by *alpha_dev
};

template <class Cfg, int FLAGS>
struct EpiLinear {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    apply_fp8_scales<Cfg>(e, c, acc);
    float alpha = e.alpha;
    if constexpr (FLAGS & EL_ALPHADEV) alpha *= *e.alpha_dev;
    float part[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      part[i] = 0.0f;
      const int m = c.row(i);
      const bool mok = m < c.M;
      float rv = 1.0f;
      if constexpr (FLAGS & EL_ROWVEC) rv = mok ? e.rowvec[m] : 0.0f;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
          if (!mok || n >= c.N) continue;
          f32x4_t v = frag(acc, i, j, q);
          if constexpr (FLAGS & EL_ROWVEC) v = v * rv;
          if constexpr (FLAGS & EL_COLVEC) v = v * *reinterpret_cast<const f32x4_t*>(e.colvec + n);
          v = v * alpha;
          if constexpr (FLAGS & EL_TILEADD) v = v + load_bf16x4(e.aux0, e.ld_aux0, m, n);
          if constexpr (FLAGS & EL_F32OUT) {
            if (e.beta != 0.0f) v = v + e.beta * load_f32x4(e.out, e.ld_out, m, n);
            store_f32x4(e.out, e.ld_out, m, n, v);
          } else {
            store_bf16x4(e.out, e.ld_out, m, n, v);
            if constexpr (FLAGS & EL_SUMSQ) {
              f32x4_t s = round_bf4(v);
              part[i] += s[0] * s[0] + s[1] * s[1] + s[2] * s[2] + s[3] * s[3];
            }
          }
        }
    }
    if constexpr (FLAGS & EL_SUMSQ) {
      float* tot = c.rowv();
      row_sum_tile<Cfg>(c, part, tot);
      write_row_partial<Cfg>(c, tot, e.partial_out);
    }
  }
};

// --- row scale r from partials (or a given vector), then SwiGLU over the
// gate/up column pairs.  The packed weight holds, in every 64-column block, 32
// gate columns followed by the 32 matching up columns, so MFMA tiles j = 2p
// (gate) and 2p + 1 (up) put gate_f and up_f in the same lane and register.
template <class Cfg>
struct EpiSwiGLU {
  static_assert(Cfg::TN % 2 == 0, "SwiGLU needs gate/up tile pairs");
  struct Pro { RowPartials<Cfg> rp; };
  __device__ static void issue(const EpiArgs& e, const Ctx<Cfg>& c, Pro& p) {
    p.rp.issue(e.row_partials, e.n_row_partials, c);
  }
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro& p) {
    float* rv = c.rowv();
    if (e.row_partials) {
      p.rp.reduce(c, rv);
      if (c.tid < Cfg::BM) rv[c.tid] = rsqrtf(rv[c.tid] / (float)e.norm_dim + e.eps);
    } else if (c.tid < Cfg::BM) {
      int m = c.m0 + c.tid;
      rv[c.tid] = m < c.M ? e.rowvec[m] : 0.0f;
    }
    __syncthreads();
    if (e.rowvec_out && c.tn == 0 && c.tid < Cfg::BM && c.m0 + c.tid < c.M)
      e.rowvec_out[c.m0 + c.tid] = rv[c.tid];
    apply_fp8_scales<Cfg>(e, c, acc);
    const int F = c.N / 2;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = c.row(i);
      if (m >= c.M) continue;
      const float r = rv[c.lrow(i)];
#pragma unroll
      for (int p2 = 0; p2 < Cfg::TN / 2; ++p2)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ng = c.col(2 * p2, q);              // packed gate column
          const int f = (ng >> 6) * 32 + (ng & 31);     // output column
          if (f >= F) continue;
          f32x4_t hg = frag(acc, i, 2 * p2, q) * r;
          f32x4_t hu = frag(acc, i, 2 * p2 + 1, q) * r;
          f32x4_t a;
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = hg[t] * sigmoidf_(hg[t]) * hu[t];
          store_bf16x4(e.out, e.ld_out, m, f, a);
          if (e.save) {
            store_bf16x4(e.save, e.ld_save, m, ng, hg);
            store_bf16x4(e.save, e.ld_save, m, ng + 32, hu);
          }
        }
    }
  }
};

// --- QKV: row scale r1, per-head RMSNorm of q and k (128 columns, one gain
// vector per q / k shared by the heads), RoPE on adjacent column pairs, split
// store of q, k, v, and optional save of the pre-norm q, k.
template <class Cfg>
struct EpiQKNormRope {
  static_assert(Cfg::WN <= 128 && 128 % Cfg::WN == 0, "a wave must lie inside one head");
  struct Pro { RowPartials<Cfg> rp; };
  __device__ static void issue(const EpiArgs& e, const Ctx<Cfg>& c, Pro& p) {
    p.rp.issue(e.row_partials, e.n_row_partials, c);
  }
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro& p) {
    float* rv = c.rowv();
    if (e.row_partials) {
      p.rp.reduce(c, rv);
      if (c.tid < Cfg::BM) rv[c.tid] = rsqrtf(rv[c.tid] / (float)e.norm_dim + e.eps);
    } else if (c.tid < Cfg::BM) {
      int m = c.m0 + c.tid;
      rv[c.tid] = m < c.M ? e.rowvec[m] : 0.0f;
    }
    __syncthreads();
    if (e.rowvec_out && c.tn == 0 && c.tid < Cfg::BM && c.m0 + c.tid < c.M)
      e.rowvec_out[c.m0 + c.tid] = rv[c.tid];
    apply_fp8_scales<Cfg>(e, c, acc);
    const int D = e.region;
    const int head_base = c.n0 + c.wn0;                 // wave's first column
    const int reg = head_base / D;                       // 0 q, 1 k, 2 v (whole wave)
    // pre-norm values h = r1 * acc, and per-head partial sums of squares
    float part[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const float r = rv[c.lrow(i)];
      part[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          float h = acc.c[i][j][t] * r;
          acc.c[i][j][t] = h;
          part[i] += h * h;
        }
    }
    // combine the lane pair, then the waves covering the same head
    constexpr int WPH = 128 / Cfg::WN;                   // waves per head
    float* red = c.red();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      float s = part[i] + __shfl_xor(part[i], 32, 64);
      if ((c.lane >> 5) == 0) red[c.wn * Cfg::BM + c.lrow(i)] = s;
    }
    __syncthreads();
    const int w0 = (c.wn / WPH) * WPH;
    const float* g = reg == 0 ? e.colvec : e.colvec2;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = c.row(i);
      if (m >= c.M) continue;
      float ss = 0.0f;
#pragma unroll
      for (int w = 0; w < WPH; ++w) ss += red[(w0 + w) * Cfg::BM + c.lrow(i)];
      const float rho = rsqrtf(ss / 128.0f + e.eps);
      const int pos = m % e.seq_len;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
          if (n >= c.N) continue;
          f32x4_t h = frag(acc, i, j, q);
          if (reg == 2) {
            store_bf16x4(e.out3, e.ld_out3, m, n - 2 * D, h);
            continue;
          }
          const int cc = n & 127;                          // column inside the head
          if (e.save) store_bf16x4(e.save, e.ld_save, m, n, h);
          f32x4_t gg = *reinterpret_cast<const f32x4_t*>(g + cc);
          f32x4_t y = h * rho * gg;
          // pairs (cc, cc+1) and (cc+2, cc+3) -> frequencies cc/2, cc/2 + 1
          f32x4_t cs = *reinterpret_cast<const f32x4_t*>(e.table + ((int64_t)pos * 64 + (cc >> 1)) * 2);
          f32x4_t o;
          o[0] = y[0] * cs[0] - y[1] * cs[1];
          o[1] = y[0] * cs[1] + y[1] * cs[0];
          o[2] = y[2] * cs[2] - y[3] * cs[3];
          o[3] = y[2] * cs[3] + y[3] * cs[2];
          if (reg == 0) store_bf16x4(e.out, e.ld_out, m, n, o);
          else store_bf16x4(e.out2, e.ld_out2, m, n - D, o);
        }
    }
  }
};

// --- dSwiGLU (backward of the SwiGLU map) in the epilogue of da = dY W_d^T:
// loads the saved gate/up pre-activations (packed layout), forms dhg, dhu,
// scales by r2 and stores dh~ (bf16, packed), plus the partials
// T[tn][m] = sum over the tile of dh~ . h (for the RMSNorm backward).
template <class Cfg>
struct EpiDSwiGLU {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    apply_fp8_scales<Cfg>(e, c, acc);
    float part[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      part[i] = 0.0f;
      const int m = c.row(i);
      if (m >= c.M) continue;
      const float r = e.rowvec[m];
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = c.col(j, q);
          if (f >= c.N) continue;
          const int pg = (f >> 5) * 64 + (f & 31);
          f32x4_t hg = load_bf16x4(e.aux0, e.ld_aux0, m, pg);
          f32x4_t hu = load_bf16x4(e.aux0, e.ld_aux0, m, pg + 32);
          f32x4_t da = frag(acc, i, j, q);
          f32x4_t dg, du;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float s = sigmoidf_(hg[t]);
            dg[t] = round_bf(r * (da[t] * hu[t] * s * (1.0f + hg[t] * (1.0f - s))));
            du[t] = round_bf(r * (da[t] * hg[t] * s));
            part[i] += dg[t] * hg[t] + du[t] * hu[t];
          }
          store_bf16x4(e.out, e.ld_out, m, pg, dg);
          store_bf16x4(e.out, e.ld_out, m, pg + 32, du);
        }
    }
    float* tot = c.rowv();
    row_sum_tile<Cfg>(c, part, tot);
    write_row_partial<Cfg>(c, tot, e.partial_out);
  }
};

// --- RMSNorm-backward correction: out = acc - c[m] u[m,n] + res[m,n] with
// c = r T / D, T finished from the row partials in the prologue.
template <class Cfg>
struct EpiNormCorrection {
  struct Pro { RowPartials<Cfg> rp; };
  __device__ static void issue(const EpiArgs& e, const Ctx<Cfg>& c, Pro& p) {
    p.rp.issue(e.row_partials, e.n_row_partials, c);
  }
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro& p) {
    float* cv = c.rowv();
    p.rp.reduce(c, cv);
    if (c.tid < Cfg::BM) {
      int m = c.m0 + c.tid;
      cv[c.tid] = m < c.M ? e.rowvec[m] * cv[c.tid] / (float)e.norm_dim : 0.0f;
    }
    __syncthreads();
    apply_fp8_scales<Cfg>(e, c, acc);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = c.row(i);
      if (m >= c.M) continue;
      const float cc = cv[c.lrow(i)];
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
          if (n >= c.N) continue;
          f32x4_t v = frag(acc, i, j, q) - cc * load_bf16x4(e.aux0, e.ld_aux0, m, n);
          v = v + load_bf16x4(e.aux1, e.ld_aux1, m, n);
          store_bf16x4(e.out, e.ld_out, m, n, v);
        }
    }
  }
};

// --- weight gradient through a folded gain: dW = beta dW + g[m] acc (fp32)
// and the gain-gradient partials P[tn][m] = sum over the tile of W[m,n] acc.
template <class Cfg>
struct EpiWgradGain {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    apply_fp8_scales<Cfg>(e, c, acc);
    float part[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      part[i] = 0.0f;
      const int m = c.row(i);
      if (m >= c.M) continue;
      const float g = e.rowvec[m];
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
          if (n >= c.N) continue;
          f32x4_t a = frag(acc, i, j, q);
          f32x4_t w = load_bf16x4(e.aux0, e.ld_aux0, m, n);
          part[i] += w[0] * a[0] + w[1] * a[1] + w[2] * a[2] + w[3] * a[3];
          f32x4_t v = g * a;
          if (e.beta != 0.0f) v = v + e.beta * load_f32x4(e.out, e.ld_out, m, n);
          store_f32x4(e.out, e.ld_out, m, n, v);
        }
    }
    float* tot = c.rowv();
    row_sum_tile<Cfg>(c, part, tot);
    write_row_partial<Cfg>(c, tot, e.partial_out);
  }
};

// --- cross-entropy forward: per (row, N tile) online log-sum-exp state
// (max m_t and s_t = sum exp(z - m_t) over the tile's valid columns) and the
// gather of the label logit by the one lane that holds it.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;   // both empty
  s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
  m = mm;
}

template <class Cfg>
struct EpiCrossEntropy {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    apply_fp8_scales<Cfg>(e, c, acc);
    float* redm = c.red();
    float* reds = c.red2();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = c.row(i);
      const int y = m < c.M ? e.labels[m] : -1;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float z = acc.c[i][j][4 * q + t];
            if (n + t < e.vocab) mx = fmaxf(mx, z);
            if (n + t == y) e.rowvec_out[m] = z;       // label logit (one writer)
          }
        }
      float s = 0.0f;
      if (mx != -INFINITY) {
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = c.col(j, q);
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (n + t < e.vocab) s += __expf(acc.c[i][j][4 * q + t] - mx);
          }
      }
      float m2 = __shfl_xor(mx, 32, 64), s2 = __shfl_xor(s, 32, 64);
      lse_merge(mx, s, m2, s2);
      if ((c.lane >> 5) == 0) {
        redm[c.wn * Cfg::BM + c.lrow(i)] = mx;
        reds[c.wn * Cfg::BM + c.lrow(i)] = s;
      }
    }
    __syncthreads();
    for (int r = c.tid; r < Cfg::BM; r += Cfg::T) {
      float mx = -INFINITY, s = 0.0f;
#pragma unroll
      for (int w = 0; w < Cfg::WAVES_N; ++w) lse_merge(mx, s, redm[w * Cfg::BM + r], reds[w * Cfg::BM + r]);
      const int m = c.m0 + r;
      if (m < c.M) {
        e.partial_out[(int64_t)c.tn * c.M + m] = mx;
        e.partial_out2[(int64_t)c.tn * c.M + m] = s;
      }
    }
  }
};

// --- cross-entropy backward recompute: G = bf16(exp(z - lse) - [n == y]) on
// rows whose label is not ignored, 0 on ignored rows.
template <class Cfg>
struct EpiCrossEntropyGrad {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    apply_fp8_scales<Cfg>(e, c, acc);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = c.row(i);
      if (m >= c.M) continue;
      const int y = e.labels[m];
      const bool valid = y != -100;
      const float lse = e.rowvec[m];
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
          if (n >= c.N) continue;
          f32x4_t gv;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float p = __expf(acc.c[i][j][4 * q + t] - lse) - (n + t == y ? 1.0f : 0.0f);
            gv[t] = valid ? p : 0.0f;
          }
          store_bf16x4(e.out, e.ld_out, m, n, gv);
        }
    }
  }
};

// ================================================================ the kernel
template <class Cfg, class Epi>
__global__ __launch_bounds__(Cfg::T) void gemm_epi_kernel(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const TileCoord tc = tile_coord(blockIdx.x, g.tiles_m, g.tiles_n, 8);
  Ctx<Cfg> c;
  c.m0 = tc.tm * Cfg::BM;
  c.n0 = tc.tn * Cfg::BN;
  c.tn = tc.tn;
  c.wn = wave % Cfg::WAVES_N;
  c.wm0 = (wave / Cfg::WAVES_N) * Cfg::WM;
  c.wn0 = c.wn * Cfg::WN;
  c.lane = lane;
  c.tid = tid;
  c.M = g.M;
  c.N = g.N;
  c.smem = smem;
  typename Epi::Pro pro;
  Epi::issue(e, c, pro);
  Acc<Cfg> acc;
  mainloop<Cfg>(g, smem, acc, c.m0, c.n0, c.wm0, c.wn0, tid, lane);
  Epi::apply(e, c, acc, pro);
}

}  // namespace coda
