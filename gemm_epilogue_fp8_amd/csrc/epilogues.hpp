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
// Register layout.  Lane l of the wave at (wm0, wn0) holds, for MFMA tile
// (i, j) and group q, row m = m0 + wm0 + 32 i + (l & 31) and the 4 consecutive
// columns n = n0 + wn0 + 32 j + 8 q + 4 (l >> 5) + {0..3} in
// acc.c[i][j][4 q + {0..3}].  A row of the workgroup tile is spread over lanes
// l and l ^ 32 of WAVES_N waves: row reductions add in-lane, then across the
// lane pair, then across waves through LDS in a fixed order (no atomics,
// bitwise deterministic).
//
// Tile I/O (P3) is staged through LDS.  Stored straight from the register
// layout, one wave instruction would touch 32 rows x 16 bytes; here the tile
// goes to an LDS staging tile (8-byte writes in the register layout, 16-byte
// chunks XOR-swizzled by row) and the whole workgroup then moves it with
// row-contiguous 16-byte accesses (64 lanes = two full 512-byte rows), which
// is what keeps epilogue traffic near HBM speed.  Auxiliary tiles that share
// the output tile's layout (residual, saved pre-activations) are copied
// global -> LDS into the staging tile by buffer_load ... lds, all copies in
// flight at once; each lane then replaces its values by its outputs in place.
// Auxiliary tiles beside a second operand (the norm correction's u and res,
// the unfolded weight of the gain gradient) stream straight into registers
// one 32-row block ahead.  After the mainloop the 128 KB of pipeline LDS is
// free for staging; row vectors and reduction scratch live in a separate
// 10 KB.
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
  const float* rowvec2;                // second row vector (CE backward through a norm: r)
  float* rowvec_out2;                  // second row vector output (CE forward through a norm: r)
  int64_t split_stride;                // split K: fp32 elements between the slices' outputs
  int64_t split_pstride;               // split K: floats between the slices' row partials
  int col_offset;                      // CE gradient: global index of the tile's column 0 minus n0
};

template <class Cfg>
constexpr int scratch_bytes() { return (2 + 2 * Cfg::WAVES_N) * Cfg::BM * 4; }

template <class Cfg>
struct Ctx {
  int m0, n0, wm0, wn0, lane, tid, wn, M, N, tn;
  char* smem;
  __device__ __forceinline__ int lrow(int i) const { return wm0 + 32 * i + (lane & 31); }
  __device__ __forceinline__ int row(int i) const { return m0 + lrow(i); }
  __device__ __forceinline__ int lcol(int j, int q) const { return wn0 + 32 * j + 8 * q + 4 * (lane >> 5); }
  __device__ __forceinline__ int col(int j, int q) const { return n0 + lcol(j, q); }
  // indices clamped into the matrix, for vector loads whose values only reach
  // positions that are never stored (keeps the loads unconditional)
  __device__ __forceinline__ int rowc(int i) const { return min(row(i), M - 1); }
  __device__ __forceinline__ int colc(int j, int q) const { return min(col(j, q), N - 4); }
  __device__ __forceinline__ char* stage() const { return smem; }
  // scratch after the pipeline buffers: two row vectors, two [WAVES_N][BM] arrays
  __device__ __forceinline__ float* scratch() const { return reinterpret_cast<float*>(smem + Cfg::LDS_BYTES); }
  __device__ __forceinline__ float* rowv() const { return scratch(); }
  __device__ __forceinline__ float* rowv2() const { return scratch() + Cfg::BM; }
  __device__ __forceinline__ float* red() const { return scratch() + 2 * Cfg::BM; }
  __device__ __forceinline__ float* red2() const { return scratch() + (2 + Cfg::WAVES_N) * Cfg::BM; }
};

// 4 floats -> 4 packed bf16 (two conversions), and back
__device__ __forceinline__ uint2 pack_bf4(f32x4_t v) { return uint2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])}; }
__device__ __forceinline__ f32x4_t unpack_bf4(uint2 w) { return f32x4_t{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)}; }
__device__ __forceinline__ f32x4_t round_bf4(f32x4_t v) { return unpack_bf4(pack_bf4(v)); }

template <class Cfg>
__device__ __forceinline__ f32x4_t frag(const Acc<Cfg>& acc, int i, int j, int q) {
  return f32x4_t{acc.c[i][j][4 * q], acc.c[i][j][4 * q + 1], acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3]};
}
template <class Cfg>
__device__ __forceinline__ void set_frag(Acc<Cfg>& acc, int i, int j, int q, f32x4_t v) {
#pragma unroll
  for (int t = 0; t < 4; ++t) acc.c[i][j][4 * q + t] = v[t];
}

// ---------------------------------------------------------------- P3 staging tiles in LDS
// bf16 tile [R][C]: C * 2 bytes a row, 16-byte chunks XOR-swizzled by row.
template <int R, int C>
struct StageBF {
  static constexpr int CPR = C / 8;
  static_assert((CPR & (CPR - 1)) == 0, "chunks a row must be a power of two");
  static constexpr int BYTES = R * C * 2;
  __device__ __forceinline__ static uint32_t off(int r, int chunk) {
    return (uint32_t)(r * C * 2 + ((chunk ^ (r & (CPR - 1))) << 4));
  }
  // 4 consecutive bf16 at (r, col), col % 4 == 0
  __device__ __forceinline__ static uint32_t off4(int r, int col) { return off(r, col >> 3) + ((col & 4) << 1); }
  __device__ __forceinline__ static void put4(char* s, int r, int col, f32x4_t v) { put4p(s, r, col, pack_bf4(v)); }
  __device__ __forceinline__ static void put4p(char* s, int r, int col, uint2 w) {
    *reinterpret_cast<uint2*>(s + off4(r, col)) = w;
  }
  __device__ __forceinline__ static f32x4_t get4(const char* s, int r, int col) {
    uint2 w = *reinterpret_cast<const uint2*>(s + off4(r, col));
    return f32x4_t{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
  }
};

// fp32 tile [R][C]: C * 4 bytes a row, 16-byte chunks XOR-swizzled by row.
template <int R, int C>
struct StageF32 {
  static constexpr int CPR = C / 4;
  static_assert((CPR & (CPR - 1)) == 0, "chunks a row must be a power of two");
  static constexpr int BYTES = R * C * 4;
  __device__ __forceinline__ static uint32_t off(int r, int chunk) {
    return (uint32_t)(r * C * 4 + ((chunk ^ (r & (CPR - 1))) << 4));
  }
};

// Workgroup-wide row-contiguous moves between a staging tile and global
// memory.  dst(m_local, n_local) returns the global address of the 16-byte
// chunk that starts at local (row, column), or nullptr to skip it.
// The store reads a batch of chunks from LDS before storing any of them, so
// one LDS round trip serves the whole batch instead of each store waiting
// for its own read.
template <class Cfg, int R, int C, class Dst>
__device__ __forceinline__ void stage_store_bf(const char* s, int tid, Dst dst) {
  using S = StageBF<R, C>;
  constexpr int ITER = R * S::CPR / Cfg::T;           // chunks a thread stores
  static_assert(R * S::CPR % Cfg::T == 0, "whole rounds of 16-byte chunks");
  constexpr int NB = ITER < 8 ? ITER : 8;             // LDS reads in flight
  static_assert(ITER % NB == 0, "whole batches");
#pragma unroll
  for (int k0 = 0; k0 < ITER; k0 += NB) {
    uint4 v[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int id = tid + (k0 + k) * Cfg::T;
      v[k] = *reinterpret_cast<const uint4*>(s + S::off(id / S::CPR, id % S::CPR));
    }
    // pins every read here: left alone, the compiler sinks each read into
    // its conditional store, which serialises them again
#pragma unroll
    for (int k = 0; k < NB; ++k) asm volatile("" : "+v"(v[k].x), "+v"(v[k].y), "+v"(v[k].z), "+v"(v[k].w));
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int id = tid + (k0 + k) * Cfg::T;
      uint16_t* p = dst(id / S::CPR, (id % S::CPR) * 8);
      if (p) *reinterpret_cast<uint4*>(p) = v[k];
    }
  }
}
template <class Cfg, int R, int C, class Src>
__device__ __forceinline__ void stage_load_bf(char* s, int tid, Src src) {
  using S = StageBF<R, C>;
#pragma unroll 4
  for (int id = tid; id < R * S::CPR; id += Cfg::T) {
    const int r = id / S::CPR, ch = id % S::CPR;
    const uint16_t* p = src(r, ch * 8);
    *reinterpret_cast<uint4*>(s + S::off(r, ch)) = p ? *reinterpret_cast<const uint4*>(p) : uint4{0, 0, 0, 0};
  }
}

// bf16 tile [R][C] of the matrix at (m0 + r, col0 + c), rows < M and
// columns < N (N % 8 == 0), copied global -> LDS into the StageBF<R, C>
// layout by buffer_load ... lds: no registers, every copy of the workgroup in
// flight at once, positions outside the matrix read as zero.  Lane l of a
// copy writes the 16-byte LDS slot l of its row(s); it fetches the chunk that
// the row swizzle puts there.  The caller waits (vmcnt) and syncs.
template <class Cfg, int R, int C>
__device__ __forceinline__ void stage_dma_bf(char* s, const void* base, int64_t ld, int m0, int col0, int M, int N,
                                             int tid) {
  using S = StageBF<R, C>;
  constexpr int RPI = 64 / S::CPR;                       // rows per wave copy
  static_assert(S::CPR <= 64 && 64 % S::CPR == 0, "a wave copy covers whole rows");
  constexpr int NI = R / RPI;                             // copies of the workgroup
  static_assert(NI % Cfg::NWAVES == 0, "copies split evenly over the waves");
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const uint16_t* p = static_cast<const uint16_t*>(base) + (int64_t)m0 * ld + col0;
  const int64_t rows = M - m0 < R ? M - m0 : R;
  const uint64_t bytes = rows <= 0 ? 0 : (uint64_t)((rows - 1) * ld + (N - col0)) * 2;
  const auto rs = make_rsrc(p, bytes);
#pragma unroll
  for (int k = 0; k < NI / Cfg::NWAVES; ++k) {
    const int q = wave + Cfg::NWAVES * k;                 // copy index
    const int r = RPI * q + lane / S::CPR;
    const int chunk = (lane % S::CPR) ^ (r & (S::CPR - 1));
    const bool ok = m0 + r < M && col0 + chunk * 8 < N;
    const uint32_t off = ok ? (uint32_t)(((int64_t)r * ld + chunk * 8) * 2) : kOobOffset;
    raw_ptr_buffer_load_lds(rs, (lds_void_t*)(s + q * 1024), 16, (int)off, 0, 0, 0);
  }
}

// bf16 matrix at (m0 + r, n0 + col), with bounds (rows < M, cols < N); N % 8 == 0
struct MatBF {
  uint16_t* base; int64_t ld; int m0, n0, M, N;
  __device__ __forceinline__ uint16_t* operator()(int r, int col) const {
    const int m = m0 + r, n = n0 + col;
    return (m < M && n < N) ? base + (int64_t)m * ld + n : nullptr;
  }
};
struct CMatBF {
  const uint16_t* base; int64_t ld; int m0, n0, M, N;
  __device__ __forceinline__ const uint16_t* operator()(int r, int col) const {
    const int m = m0 + r, n = n0 + col;
    return (m < M && n < N) ? base + (int64_t)m * ld + n : nullptr;
  }
};

// Register values -> bf16 staging tile (rows of this wave, all its columns).
template <class Cfg, int C>
__device__ __forceinline__ void put_tile(const Ctx<Cfg>& c, const Acc<Cfg>& acc) {
  char* s = c.stage();
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) StageBF<Cfg::BM, C>::put4(s, c.lrow(i), c.lcol(j, q), frag(acc, i, j, q));
}

// A rank-2 bf16 operand tile read straight into registers in the MFMA
// layout, one 32-row block (i) at a time: lane values at (row(i), col(j, q)
// .. + 3).  Indices are clamped into the matrix, so every load is in bounds;
// positions outside it carry values that are never stored.
template <class Cfg>
struct RowBlock {
  uint2 v[Cfg::TN][4];
  // Rows m0 + lrow(i) of the bf16 matrix at base (row stride ld elements),
  // this lane's columns, through a buffer resource that starts at the tile's
  // first row: one offset register for the block, the column steps in the
  // instructions' immediate offsets.  Rows past M read as zero; columns
  // past N read what lies there (other rows or padding, inside the
  // resource), which reaches only positions that are never stored or are
  // masked out of the reductions.
  __device__ __forceinline__ void load(const void* base, int64_t ld, const Ctx<Cfg>& c, int i) {
    const char* b = static_cast<const char*>(base) + (int64_t)c.m0 * ld * 2;
    const int64_t bytes = ((int64_t)(c.M - c.m0 - 1) * ld + c.N) * 2;
    const auto rs = make_rsrc(b, bytes > 0 ? (uint64_t)bytes : 0);
    const uint32_t off = (uint32_t)(((int64_t)c.lrow(i) * ld + c.col(0, 0)) * 2);
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const i32x2_t w = buf_load8(rs, off + (uint32_t)(64 * j + 16 * q));   // 32 j + 8 q columns on
        v[j][q] = uint2{(uint32_t)w[0], (uint32_t)w[1]};
      }
  }
  __device__ __forceinline__ f32x4_t get(int j, int q) const {
    return f32x4_t{bf_lo(v[j][q].x), bf_hi(v[j][q].x), bf_lo(v[j][q].y), bf_hi(v[j][q].y)};
  }
};

// fp32 output D = beta D + v for the tile, staged through LDS in row halves
// (128 KB each); v is in the register layout in acc.
template <class Cfg>
__device__ __forceinline__ void store_f32_tile(const EpiArgs& e, const Ctx<Cfg>& c, const Acc<Cfg>& acc) {
  constexpr int HR = Cfg::BM / 2;
  using S = StageF32<HR, Cfg::BN>;
  static_assert(S::BYTES <= Cfg::LDS_BYTES, "half tile must fit the staging area");
  char* s = c.stage();
  float* out = static_cast<float*>(e.out);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int r = c.lrow(i) - h * HR;
      if (r < 0 || r >= HR) continue;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4_t*>(s + S::off(r, c.lcol(j, q) >> 2)) = frag(acc, i, j, q);
    }
    __syncthreads();
    // Batches of NB chunks: every prior value of a batch is loaded before
    // any of its stores, so the batch waits for one round trip (a loop that
    // loads, adds and stores chunk by chunk compiles to one exposed round
    // trip per chunk, the compiler being unable to move a load above the
    // previous chunk's store).
    constexpr int ITER = HR * S::CPR / Cfg::T;
    static_assert(HR * S::CPR % Cfg::T == 0, "whole rounds of 16-byte chunks");
    constexpr int NB = ITER < 4 ? ITER : 4;
    static_assert(ITER % NB == 0, "whole batches");
#pragma unroll
    for (int k0 = 0; k0 < ITER; k0 += NB) {
      f32x4_t v[NB], prior[NB];
      f32x4_t* p[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int id = c.tid + (k0 + k) * Cfg::T;
        const int r = id / S::CPR, ch = id % S::CPR;
        const int m = c.m0 + h * HR + r, n = c.n0 + ch * 4;
        p[k] = (m < c.M && n < c.N) ? reinterpret_cast<f32x4_t*>(out + (int64_t)m * e.ld_out + n) : nullptr;
        v[k] = *reinterpret_cast<const f32x4_t*>(s + S::off(r, ch));
      }
      if (e.beta != 0.0f) {
#pragma unroll
        for (int k = 0; k < NB; ++k) prior[k] = p[k] ? *p[k] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < NB; ++k) v[k] = v[k] + e.beta * prior[k];
      }
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (p[k]) *p[k] = v[k];
    }
  }
}

// ---------------------------------------------------------------- P2 vector loads: fp8 dequant scales
// acc <- acc * s_row[m] * s_col[n] (the per-token and per-channel E4M3 scales)
template <class Cfg>
__device__ __forceinline__ void apply_fp8_scales(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc) {
  if constexpr (Cfg::FP8 && !Cfg::MX) {   // MXFP8 blocks are scaled inside the MFMA
    float sr[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) sr[i] = e.rowscale[c.rowc(i)];
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(e.colscale + c.colc(j, q));
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc.c[i][j][4 * q + t] = (acc.c[i][j][4 * q + t] * sr[i]) * sc[t];
      }
  }
}

// ---------------------------------------------------------------- P4 row reduction over the tile
// part[i] is this lane's share of local row lrow(i); writes the tile total of
// every local row to out[BM] (LDS scratch) in a fixed order.
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
// thread, all loads independent) and after it reduces them into LDS.  The
// values stay in registers through the mainloop, so their number is kept
// small; a wider set of partials is first summed to one row by an auxiliary
// kernel (the light merge step of the paper, §3.1).
template <class Cfg>
struct RowPartials {
  static constexpr int TPR = Cfg::T / Cfg::BM;   // threads per row
  static constexpr int MAXP = 4;                 // partials per thread
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

// Finishes the per-row factor of the tile's rows into c.rowv():
// r = (sum of partials / D + eps)^(-1/2), or a given row vector; the tiles of
// the first N tile also write it to r_out when given.
template <class Cfg>
__device__ __forceinline__ void finish_inv_rms(const EpiArgs& e, const Ctx<Cfg>& c, const RowPartials<Cfg>& rp,
                                               float* r_out) {
  float* rv = c.rowv();
  if (e.row_partials) {
    rp.reduce(c, rv);
    if (c.tid < Cfg::BM) rv[c.tid] = rsqrtf(rv[c.tid] / (float)e.norm_dim + e.eps);
  } else if (c.tid < Cfg::BM) {
    int m = c.m0 + c.tid;
    rv[c.tid] = m < c.M ? e.rowvec[m] : 0.0f;
  }
  __syncthreads();
  if (r_out && c.tn == 0 && c.tid < Cfg::BM && c.m0 + c.tid < c.M) r_out[c.m0 + c.tid] = rv[c.tid];
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes
// have completed; its global stores and global->LDS copies may still be in
// flight (__syncthreads would wait for those too).
__device__ __forceinline__ void lds_barrier() {
  wait_lgkmcnt0();
  phase_barrier();
}

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
    using S = StageBF<Cfg::BM, Cfg::BN>;
    apply_fp8_scales<Cfg>(e, c, acc);
    float alpha = e.alpha;
    if constexpr (FLAGS & EL_ALPHADEV) alpha *= *e.alpha_dev;
    constexpr bool ADD = (FLAGS & EL_TILEADD) != 0;
    static_assert(!ADD || !(FLAGS & EL_F32OUT), "the residual is added to bf16 outputs");
    if constexpr (ADD) {
      // the residual tile comes into the staging tile; each lane replaces its
      // values by the outputs (the stage is free after the mainloop)
      stage_dma_bf<Cfg, Cfg::BM, Cfg::BN>(c.stage(), e.aux0, e.ld_aux0, c.m0, c.n0, c.M, c.N, c.tid);
      wait_vmcnt<0>();
      __syncthreads();
    }
    float part[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      part[i] = 0.0f;
      const int m = c.row(i);
      float rv = 1.0f;
      if constexpr (FLAGS & EL_ROWVEC) rv = e.rowvec[c.rowc(i)];
      // the block's residual values are all read before any output replaces
      // them in place: one LDS round trip a block, not one per 4 columns
      uint2 z[Cfg::TN][4];
      if constexpr (ADD) {
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            z[j][q] = *reinterpret_cast<const uint2*>(c.stage() + S::off4(c.lrow(i), c.lcol(j, q)));
      }
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
          f32x4_t v = frag(acc, i, j, q);
          if constexpr (FLAGS & EL_ROWVEC) v = v * rv;
          if constexpr (FLAGS & EL_COLVEC)
            v = v * *reinterpret_cast<const f32x4_t*>(e.colvec + c.colc(j, q));
          v = v * alpha;
          if constexpr (ADD) v = v + unpack_bf4(z[j][q]);
          if constexpr (!(FLAGS & EL_F32OUT)) {
            const uint2 pk = pack_bf4(v);
            if constexpr (FLAGS & EL_SUMSQ) {
              const f32x4_t w = unpack_bf4(pk);   // the stored values
              if (m < c.M && n < c.N) part[i] += w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
            }
            S::put4p(c.stage(), c.lrow(i), c.lcol(j, q), pk);   // the stage is free after the mainloop
          } else {
            set_frag(acc, i, j, q, v);
          }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FLAGS & EL_F32OUT) {
      store_f32_tile<Cfg>(e, c, acc);
    } else {
      __syncthreads();
      stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(c.stage(), c.tid,
          MatBF{static_cast<uint16_t*>(e.out), e.ld_out, c.m0, c.n0, c.M, c.N});
      if constexpr (FLAGS & EL_SUMSQ) {
        float* tot = c.rowv();
        row_sum_tile<Cfg>(c, part, tot);
        write_row_partial<Cfg>(c, tot, e.partial_out);
      }
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
    finish_inv_rms<Cfg>(e, c, p.rp, e.rowvec_out);
    apply_fp8_scales<Cfg>(e, c, acc);
    const float* rv = c.rowv();
    // h = r * acc (kept in acc); a = SiLU(h_gate) * h_up staged as [BM][BN/2]
    constexpr int CA = Cfg::BN / 2;
    char* s = c.stage();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const float r = rv[c.lrow(i)];
#pragma unroll
      for (int p2 = 0; p2 < Cfg::TN / 2; ++p2)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t hg = frag(acc, i, 2 * p2, q) * r;
          f32x4_t hu = frag(acc, i, 2 * p2 + 1, q) * r;
          f32x4_t a;
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = hg[t] * sigmoidf_(hg[t]) * hu[t];
          set_frag(acc, i, 2 * p2, q, hg);
          set_frag(acc, i, 2 * p2 + 1, q, hu);
          // local output column of gate column lcol: 32 per 64-column block
          const int lc = c.lcol(2 * p2, q);
          StageBF<Cfg::BM, CA>::put4(s, c.lrow(i), (lc >> 6) * 32 + (lc & 31), a);
        }
    }
    __syncthreads();
    const int F = c.N / 2;
    stage_store_bf<Cfg, Cfg::BM, CA>(s, c.tid, MatBF{static_cast<uint16_t*>(e.out), e.ld_out, c.m0, c.n0 / 2, c.M, F});
    if (e.save) {
      __syncthreads();
      put_tile<Cfg, Cfg::BN>(c, acc);
      __syncthreads();
      stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(s, c.tid,
          MatBF{static_cast<uint16_t*>(e.save), e.ld_save, c.m0, c.n0, c.M, c.N});
    }
  }
};

// Elementwise maps of the pre-norm activation layer: the value f(h) and the
// backward factor da f'(h).
struct MapSigmoid {
  __device__ static float f(float h) { return sigmoidf_(h); }
  __device__ static float back(float da, float h) {
    const float sg = sigmoidf_(h);
    return da * sg * (1.0f - sg);
  }
};
// GELU(h) = h Phi(h) with the normal CDF Phi(h) = (1 + erf(h / sqrt 2)) / 2
// (the exact form); GELU'(h) = Phi(h) + h phi(h), phi the normal density.
struct MapGelu {
  __device__ static float f(float h) { return 0.5f * h * (1.0f + erff(h * 0.70710678118654752f)); }
  __device__ static float back(float da, float h) {
    const float cdf = 0.5f * (1.0f + erff(h * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * __expf(-0.5f * h * h);
    return da * (cdf + h * pdf);
  }
};

// --- row scale r from partials (or a given vector), then an elementwise map:
// h = r acc, out = f(h), optional save of h (for the backward).
template <class Cfg, class Map>
struct EpiActMap {
  struct Pro { RowPartials<Cfg> rp; };
  __device__ static void issue(const EpiArgs& e, const Ctx<Cfg>& c, Pro& p) {
    p.rp.issue(e.row_partials, e.n_row_partials, c);
  }
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro& p) {
    using S = StageBF<Cfg::BM, Cfg::BN>;
    finish_inv_rms<Cfg>(e, c, p.rp, e.rowvec_out);
    apply_fp8_scales<Cfg>(e, c, acc);
    char* s = c.stage();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const float r = c.rowv()[c.lrow(i)];
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t h = frag(acc, i, j, q) * r;
          f32x4_t a;
#pragma unroll
          for (int t = 0; t < 4; ++t) a[t] = Map::f(h[t]);
          S::put4(s, c.lrow(i), c.lcol(j, q), a);
          set_frag(acc, i, j, q, h);
        }
    }
    __syncthreads();
    stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(s, c.tid, MatBF{static_cast<uint16_t*>(e.out), e.ld_out, c.m0, c.n0, c.M, c.N});
    if (e.save) {
      __syncthreads();
      put_tile<Cfg, Cfg::BN>(c, acc);
      __syncthreads();
      stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(s, c.tid,
          MatBF{static_cast<uint16_t*>(e.save), e.ld_save, c.m0, c.n0, c.M, c.N});
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
    finish_inv_rms<Cfg>(e, c, p.rp, e.rowvec_out);
    apply_fp8_scales<Cfg>(e, c, acc);
    const float* rv = c.rowv();
    const int D = e.region;
    const int reg = (c.n0 + c.wn0) / D;                  // 0 q, 1 k, 2 v (whole wave)
    char* s = c.stage();
    // pre-norm values h = r1 * acc and per-head partial sums of squares
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
    // save of the pre-norm q, k (columns < 2D)
    if (e.save) {
      put_tile<Cfg, Cfg::BN>(c, acc);
      __syncthreads();
      stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(s, c.tid,
          MatBF{static_cast<uint16_t*>(e.save), e.ld_save, c.m0, c.n0, c.M, 2 * D});
      __syncthreads();
    }
    // combine the lane pair, then the waves covering the same head
    constexpr int WPH = 128 / Cfg::WN;                   // waves per head
    float* red = c.red();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      float sp = part[i] + __shfl_xor(part[i], 32, 64);
      if ((c.lane >> 5) == 0) red[c.wn * Cfg::BM + c.lrow(i)] = sp;
    }
    __syncthreads();
    const int w0 = (c.wn / WPH) * WPH;
    const float* g = reg == 0 ? e.colvec : e.colvec2;
    if (reg < 2) {
      // The gains of this lane's columns, and the cos/sin of a row's column
      // pairs, are loaded as whole batches (one row ahead), so that each row
      // waits for one round of table loads rather than one per column group.
      f32x4_t gg[Cfg::TN][4], cs[2][Cfg::TN][4];
      auto load_cs = [&](int i, f32x4_t (&d)[Cfg::TN][4]) {
        const int m = c.row(i);
        const int pos = (m < c.M ? m : 0) % e.seq_len;
        const float* t = e.table + (int64_t)pos * 128;
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) d[j][q] = *reinterpret_cast<const f32x4_t*>(t + (c.col(j, q) & 127));
      };
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) gg[j][q] = *reinterpret_cast<const f32x4_t*>(g + (c.col(j, q) & 127));
      load_cs(0, cs[0]);
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i) {
        if (i + 1 < Cfg::TM) load_cs(i + 1, cs[(i + 1) & 1]);
        float ss = 0.0f;
#pragma unroll
        for (int w = 0; w < WPH; ++w) ss += red[(w0 + w) * Cfg::BM + c.lrow(i)];
        const float rho = rsqrtf(ss / 128.0f + e.eps);
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4_t h = frag(acc, i, j, q);
            f32x4_t y = h * rho * gg[j][q];
            // pairs (cc, cc+1) and (cc+2, cc+3) of column cc = col & 127 ->
            // frequencies cc/2 and cc/2 + 1, whose (cos, sin) pairs are the
            // 4 floats at 2 (cc/2) = cc of the position's table row
            const f32x4_t cs4 = cs[i & 1][j][q];
            f32x4_t o;
            o[0] = y[0] * cs4[0] - y[1] * cs4[1];
            o[1] = y[0] * cs4[1] + y[1] * cs4[0];
            o[2] = y[2] * cs4[2] - y[3] * cs4[3];
            o[3] = y[2] * cs4[3] + y[3] * cs4[2];
            set_frag(acc, i, j, q, o);
          }
      }
    }
    put_tile<Cfg, Cfg::BN>(c, acc);
    __syncthreads();
    // split store: each 16-byte chunk lies inside one of q, k, v (D % 8 == 0)
    uint16_t* outs[3] = {static_cast<uint16_t*>(e.out), static_cast<uint16_t*>(e.out2), static_cast<uint16_t*>(e.out3)};
    const int64_t lds_[3] = {e.ld_out, e.ld_out2, e.ld_out3};
    const int m0 = c.m0, n0 = c.n0, M = c.M, N = c.N;
    stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(s, c.tid, [&](int r, int col) -> uint16_t* {
      const int m = m0 + r, n = n0 + col;
      if (m >= M || n >= N) return nullptr;
      const int rg = n / D;
      return outs[rg] + (int64_t)m * lds_[rg] + (n - rg * D);
    });
  }
};

// --- dSwiGLU (backward of the SwiGLU map) in the epilogue of da = dY W_d^T:
// loads the saved gate/up pre-activations (packed layout), forms dhg, dhu,
// scales by r2 and stores dh~ (bf16, packed), plus the partials
// T[tn][m] = sum over the tile of dh~ . h (for the RMSNorm backward).
// The 256 da columns of a tile map to 512 packed columns of hg/hu and dh~, so
// the tile is done in two 128-row halves (one per wave group) of 128 KB: the
// half of the saved tile is copied into LDS (stage_dma_bf), the group that
// owns those rows replaces every hg/hu pair by dhg/dhu in place, and the
// workgroup stores the half with row-contiguous 16-byte writes.
template <class Cfg>
struct EpiDSwiGLU {
  struct Pro {};
  static constexpr int HR = Cfg::BM / 2, PC = 2 * Cfg::BN;   // half rows, packed columns
  using S = StageBF<HR, PC>;
  static_assert(S::BYTES <= Cfg::LDS_BYTES, "a half tile must fit the staging area");
  static_assert(HR == Cfg::WM, "each wave group owns one half");
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}

  __device__ __forceinline__ static int packed_gate(int f) { return (f >> 5) * 64 + (f & 31); }

  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    apply_fp8_scales<Cfg>(e, c, acc);
    float part[Cfg::TM], rr[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      part[i] = 0.0f;
      rr[i] = e.rowvec[c.rowc(i)];
    }
    char* s = c.stage();
    const int grp = c.wm0 / Cfg::WM;
    const int F2 = 2 * c.N;
    __syncthreads();   // the pipeline stages are free
    stage_dma_bf<Cfg, HR, PC>(s, e.aux0, e.ld_aux0, c.m0, 2 * c.n0, c.M, F2, c.tid);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // this half's saved tile has landed (with the previous half's stores,
      // which drained while it was in flight)
      wait_vmcnt<0>();
      lds_barrier();
      if (grp == h) {
#pragma unroll
        for (int i = 0; i < Cfg::TM; ++i) {
          __builtin_amdgcn_sched_barrier(0);
          const int lr = c.lrow(i) - h * HR;
          const int m = c.row(i);
          const float r = rr[i];
#pragma unroll
          for (int j = 0; j < Cfg::TN; ++j) {
            // every saved value of the 32 x 32 tile first, then its outputs in
            // place: one LDS round trip a tile, not one per 4 columns
            uint2 g[4], u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int pg = packed_gate(c.lcol(j, q));
              g[q] = *reinterpret_cast<const uint2*>(s + S::off4(lr, pg));
              u[q] = *reinterpret_cast<const uint2*>(s + S::off4(lr, pg + 32));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int pg = packed_gate(c.lcol(j, q));
              const f32x4_t hg = unpack_bf4(g[q]);
              const f32x4_t hu = unpack_bf4(u[q]);
              const f32x4_t da = frag(acc, i, j, q);
              f32x4_t dg, du;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const float sg = sigmoidf_(hg[t]);
                dg[t] = r * (da[t] * hu[t] * sg * (1.0f + hg[t] * (1.0f - sg)));
                du[t] = r * (da[t] * hg[t] * sg);
              }
              const uint2 pdg = pack_bf4(dg), pdu = pack_bf4(du);
              if (m < c.M && c.col(j, q) < c.N) {   // F % 32 == 0: the 4 columns are all in or all out
                const f32x4_t rg = unpack_bf4(pdg), ru = unpack_bf4(pdu);   // the stored values
#pragma unroll
                for (int t = 0; t < 4; ++t) part[i] += rg[t] * hg[t] + ru[t] * hu[t];
              }
              S::put4p(s, lr, pg, pdg);
              S::put4p(s, lr, pg + 32, pdu);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      lds_barrier();
      stage_store_bf<Cfg, HR, PC>(s, c.tid,
          MatBF{static_cast<uint16_t*>(e.out), e.ld_out, c.m0 + h * HR, 2 * c.n0, c.M, F2});
      if (h == 0) {
        // every wave has read the first half out of LDS: the second half's
        // copy may land there while those stores are still in flight
        lds_barrier();
        stage_dma_bf<Cfg, HR, PC>(s, e.aux0, e.ld_aux0, c.m0 + HR, 2 * c.n0, c.M, F2, c.tid);
      }
    }
    float* tot = c.rowv();
    row_sum_tile<Cfg>(c, part, tot);
    write_row_partial<Cfg>(c, tot, e.partial_out);
  }
};

// --- backward of the elementwise map in the epilogue of da = dY Wn^T: with
// the saved h (copied into the staging tile), dh~ = bf16(r da f'(h)) replaces
// h in place and is stored; T[tn][m] = sum over the tile of dh~ h is written
// as row partials.
template <class Cfg, class Map>
struct EpiActMapBack {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    using S = StageBF<Cfg::BM, Cfg::BN>;
    apply_fp8_scales<Cfg>(e, c, acc);
    char* s = c.stage();
    stage_dma_bf<Cfg, Cfg::BM, Cfg::BN>(s, e.aux0, e.ld_aux0, c.m0, c.n0, c.M, c.N, c.tid);
    wait_vmcnt<0>();
    __syncthreads();
    float part[Cfg::TM], rr[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) rr[i] = e.rowvec[c.rowc(i)];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      part[i] = 0.0f;
      const int m = c.row(i);
      const float r = rr[i];
      uint2 hs[Cfg::TN][4];   // the block's saved values first, then the outputs in place
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) hs[j][q] = *reinterpret_cast<const uint2*>(s + S::off4(c.lrow(i), c.lcol(j, q)));
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t h = unpack_bf4(hs[j][q]);
          const f32x4_t da = frag(acc, i, j, q);
          f32x4_t d;
#pragma unroll
          for (int t = 0; t < 4; ++t) d[t] = r * Map::back(da[t], h[t]);
          const uint2 pk = pack_bf4(d);
          const f32x4_t dr = unpack_bf4(pk);   // the stored values
          if (m < c.M && c.col(j, q) < c.N) part[i] += dr[0] * h[0] + dr[1] * h[1] + dr[2] * h[2] + dr[3] * h[3];
          S::put4p(s, c.lrow(i), c.lcol(j, q), pk);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float* tot = c.rowv();
    row_sum_tile<Cfg>(c, part, tot);   // its barriers also order the staging writes
    write_row_partial<Cfg>(c, tot, e.partial_out);
    stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(s, c.tid, MatBF{static_cast<uint16_t*>(e.out), e.ld_out, c.m0, c.n0, c.M, c.N});
  }
};

template <class Cfg> using EpiSigmoid = EpiActMap<Cfg, MapSigmoid>;
template <class Cfg> using EpiDSigmoid = EpiActMapBack<Cfg, MapSigmoid>;
template <class Cfg> using EpiGelu = EpiActMap<Cfg, MapGelu>;
template <class Cfg> using EpiDGelu = EpiActMapBack<Cfg, MapGelu>;

// --- RMSNorm-backward correction: out = acc - c[m] u[m,n] + res[m,n] with
// c = r T / D, T finished from the row partials in the prologue.
template <class Cfg>
struct EpiNormCorrection {
  struct Pro { RowPartials<Cfg> rp; };
  __device__ static void issue(const EpiArgs& e, const Ctx<Cfg>& c, Pro& p) {
    p.rp.issue(e.row_partials, e.n_row_partials, c);
  }
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro& p) {
    using S = StageBF<Cfg::BM, Cfg::BN>;
    // u and res come into registers one 32-row block at a time
    // out = sc (acc - c u) + res, with sc = alpha (* *alpha_dev) and res optional
    RowBlock<Cfg> u[2], z[2];
    const bool has_res = e.aux1 != nullptr;
    u[0].load(e.aux0, e.ld_aux0, c, 0);
    if (has_res) z[0].load(e.aux1, e.ld_aux1, c, 0);
    if (Cfg::TM > 1) {
      u[1].load(e.aux0, e.ld_aux0, c, 1);
      if (has_res) z[1].load(e.aux1, e.ld_aux1, c, 1);
    }
    const float sc = e.alpha_dev ? e.alpha * *e.alpha_dev : e.alpha;
    float* cv = c.rowv();
    p.rp.reduce(c, cv);
    if (c.tid < Cfg::BM) {
      int m = c.m0 + c.tid;
      cv[c.tid] = m < c.M ? e.rowvec[m] * cv[c.tid] / (float)e.norm_dim : 0.0f;
    }
    __syncthreads();
    apply_fp8_scales<Cfg>(e, c, acc);
    char* s = c.stage();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const float cc = cv[c.lrow(i)];
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          S::put4(s, c.lrow(i), c.lcol(j, q),
                  sc * (frag(acc, i, j, q) - cc * u[i & 1].get(j, q)) +
                      (has_res ? z[i & 1].get(j, q) : f32x4_t{0, 0, 0, 0}));
      if (i + 2 < Cfg::TM) {
        u[i & 1].load(e.aux0, e.ld_aux0, c, i + 2);
        if (has_res) z[i & 1].load(e.aux1, e.ld_aux1, c, i + 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(s, c.tid, MatBF{static_cast<uint16_t*>(e.out), e.ld_out, c.m0, c.n0, c.M, c.N});
  }
};

// --- weight gradient through a folded gain: dW = beta dW + g[m] acc (fp32)
// and the gain-gradient partials P[tn][m] = sum over the tile of W[m,n] acc.
template <class Cfg>
struct EpiWgradGain {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    RowBlock<Cfg> w[2];
    w[0].load(e.aux0, e.ld_aux0, c, 0);
    if (Cfg::TM > 1) w[1].load(e.aux0, e.ld_aux0, c, 1);
    apply_fp8_scales<Cfg>(e, c, acc);
    const float sc = e.alpha_dev ? e.alpha * *e.alpha_dev : e.alpha;   // scales dW and the gain partials
    float part[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      part[i] = 0.0f;
      const int m = c.row(i);
      const float g = e.rowvec[c.rowc(i)];
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t a = frag(acc, i, j, q);
          const f32x4_t wv = w[i & 1].get(j, q);
          if (m < c.M && c.col(j, q) < c.N) part[i] += wv[0] * a[0] + wv[1] * a[1] + wv[2] * a[2] + wv[3] * a[3];
          set_frag(acc, i, j, q, (g * a) * sc);
        }
      part[i] *= sc;
      if (i + 2 < Cfg::TM) w[i & 1].load(e.aux0, e.ld_aux0, c, i + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the reduction first: partials kept live across the staged store cost spills
    float* tot = c.rowv();
    row_sum_tile<Cfg>(c, part, tot);
    write_row_partial<Cfg>(c, tot, e.partial_out);
    store_f32_tile<Cfg>(e, c, acc);
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

// NORM: the logits pass through a final RMSNorm folded into the weight
// (the third GEMM-residual-RMSNorm-GEMM occurrence of the CODA paper,
// §3.2.1): z = r acc with r finished from sum-of-squares partials in the
// prologue (written to rowvec_out2 when given).
template <class Cfg, bool NORM = false>
struct EpiCrossEntropy {
  struct Pro { RowPartials<Cfg> rp; };
  __device__ static void issue(const EpiArgs& e, const Ctx<Cfg>& c, Pro& p) {
    if constexpr (NORM) p.rp.issue(e.row_partials, e.n_row_partials, c);
  }
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro& p) {
    apply_fp8_scales<Cfg>(e, c, acc);
    if constexpr (NORM) {
      finish_inv_rms<Cfg>(e, c, p.rp, e.rowvec_out2);
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i) {
        const float r = c.rowv()[c.lrow(i)];
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j) acc.c[i][j] = acc.c[i][j] * r;
      }
    }
    float* redm = c.red();
    float* reds = c.red2();
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = c.row(i);
      const int yl = e.labels[c.rowc(i)];
      const int y = m < c.M ? yl : -1;
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
// rows whose label lies in [0, vocab), 0 on every other row (the ignore index
// and labels out of range alike: the forward leaves both out of the mean).
// NORM: z = r acc with the given r (rowvec2); the stored tile is
// G~ = bf16(r (p - onehot)) and T[tn][m] = sum over the tile of G~ z is
// written as row partials (the RMSNorm-backward statistic).
template <class Cfg, bool NORM = false>
struct EpiCrossEntropyGrad {
  struct Pro {};
  __device__ static void issue(const EpiArgs&, const Ctx<Cfg>&, Pro&) {}
  __device__ static void apply(const EpiArgs& e, const Ctx<Cfg>& c, Acc<Cfg>& acc, Pro&) {
    apply_fp8_scales<Cfg>(e, c, acc);
    float part[Cfg::TM];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      part[i] = 0.0f;
      const int m = c.row(i);
      const int y = e.labels[c.rowc(i)];
      const bool valid = m < c.M && y >= 0 && y < e.vocab;
      const float lse = e.rowvec[c.rowc(i)];
      const float r = NORM ? e.rowvec2[c.rowc(i)] : 1.0f;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.col(j, q);
          f32x4_t gv, zv;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            zv[t] = NORM ? r * acc.c[i][j][4 * q + t] : acc.c[i][j][4 * q + t];
            const float p = __expf(zv[t] - lse) - (n + e.col_offset + t == y ? 1.0f : 0.0f);
            gv[t] = valid ? (NORM ? r * p : p) : 0.0f;
          }
          const uint2 pk = pack_bf4(gv);
          if constexpr (NORM) {
            const f32x4_t gr = unpack_bf4(pk);   // the stored values
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (n + t < c.N) part[i] += gr[t] * zv[t];
          }
          StageBF<Cfg::BM, Cfg::BN>::put4p(c.stage(), c.lrow(i), c.lcol(j, q), pk);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NORM) {   // the reduction first: partials kept live across the store cost spills
      float* tot = c.rowv();
      row_sum_tile<Cfg>(c, part, tot);   // its barriers also order the staging writes
      write_row_partial<Cfg>(c, tot, e.partial_out);
    } else {
      __syncthreads();
    }
    stage_store_bf<Cfg, Cfg::BM, Cfg::BN>(c.stage(), c.tid,
        MatBF{static_cast<uint16_t*>(e.out), e.ld_out, c.m0, c.n0, c.M, c.N});
  }
};

// ================================================================ the kernel
// One output tile per workgroup; the XCD-aware tile order lives in tile_coord.
// The single-group (4-wave) tile asks for two waves a SIMD, which keeps a
// wave within 256 registers so that two workgroups share a compute unit.
template <class Cfg, class Epi>
__global__ __launch_bounds__(Cfg::T, Cfg::WAVES_M == 1 ? 2 : 1) void gemm_epi_kernel(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES + scratch_bytes<Cfg>()];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (gridDim.y > 1) {
    // split K (fp32 outputs only): slice y covers K [y kchunk, min(K, (y + 1) kchunk)) and
    // writes its own output and partials, which a separate pass adds up in a fixed order
    const int kb = blockIdx.y * g.kchunk;
    g.K = min(g.kchunk, g.K - kb);
    g.A = static_cast<const char*>(g.A) + (Cfg::A_KC ? (int64_t)kb * Cfg::ESIZE : (int64_t)kb * g.lda * Cfg::ESIZE);
    g.B = static_cast<const char*>(g.B) + (Cfg::B_KC ? (int64_t)kb * Cfg::ESIZE : (int64_t)kb * g.ldb * Cfg::ESIZE);
    if constexpr (Cfg::MX) {   // kchunk covers whole word rows: 128 bytes (E4M3) or 64 (E2M1)
      constexpr int WB = Cfg::FP4 ? 64 : 128;
      g.sA = static_cast<const char*>(g.sA) + (kb / WB) * g.lds_a;
      g.sB = static_cast<const char*>(g.sB) + (kb / WB) * g.lds_b;
    }
    e.out = static_cast<float*>(e.out) + blockIdx.y * e.split_stride;
    if (e.partial_out) e.partial_out += blockIdx.y * e.split_pstride;
  }
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
  if constexpr (Cfg::WAVES_M == 1)
    mainloop_solo<Cfg>(g, smem, acc, c.m0, c.n0, c.wm0, c.wn0, tid, lane);
  else
    mainloop<Cfg>(g, smem, acc, c.m0, c.n0, c.wm0, c.wn0, tid, lane);
  Epi::apply(e, c, acc, pro);
}

}  // namespace coda
