// The fixed GEMM mainloop: C[M,N] (fp32) = sum_k A[m,k] B[k,n] on gfx950
// matrix cores, bf16 (v_mfma_f32_32x32x16_bf16) or OCP E4M3
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).
//
// The CODA paper (arXiv 2605.19269), §2.2 and §3.1, keeps an expert-tuned
// mainloop fixed and programs only the epilogue; this file is that fixed part.
//
// Design (CDNA4-first, not a port of the paper's Hopper kernels):
//  * Workgroup tile BM x BN, 128 bytes of K per stage (64 bf16 or 128 fp8),
//    two LDS stages (global loads of stage k+1 are in flight while the MFMAs
//    of stage k run; one barrier per stage).
//  * Both operands are staged in LDS as [rows][128 bytes] with the 16-byte
//    chunks XOR-swizzled by (row & 7) so that 32 lanes reading one K chunk of
//    32 rows hit distinct banks.
//  * An operand whose K axis is contiguous in memory is copied 16 bytes at a
//    time.  An operand whose M/N axis is contiguous (the weight in a forward
//    NN product, both operands of a weight-gradient TN product) is loaded as
//    8(k) x 4(m/n) blocks and transposed in registers before the LDS store,
//    so the MFMA loop never sees the storage layout.
//  * Global loads go through buffer resources: out-of-range rows/columns are
//    read as zero by the hardware, so ragged M, N and K need no branches.
//  * MFMA operands are swapped (the B tile feeds the instruction's A port),
//    which leaves each lane holding 4 consecutive output columns of one row:
//    8-byte bf16 stores and in-lane pairwise transforms (RoPE pairs).
//  * Workgroup ids are remapped so that the tiles one XCD (8 per chip, each
//    with its own L2) runs are neighbours, then grouped along M.
#pragma once
#include "coda_device.hpp"

namespace coda {

__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, bool A_KC_, bool B_KC_, bool FP8_ = false>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NWAVES = WAVES_M * WAVES_N, T = 64 * NWAVES;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr bool A_KC = A_KC_, B_KC = B_KC_, FP8 = FP8_;
  static constexpr int ESIZE = FP8 ? 1 : 2;
  static constexpr int BK = 128 / ESIZE;
  static constexpr int STAGE_BYTES = (BM + BN) * 128;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!FP8 || (A_KC && B_KC), "fp8 operands are K-contiguous");
};

struct GemmArgs {
  const void* A;   // A_KC: [M, K] (lda >= K); else [K, M] (lda >= M)
  const void* B;   // B_KC: [N, K] (ldb >= K); else [K, N] (ldb >= N)
  int64_t lda, ldb;
  int M, N, K;
  int tiles_m, tiles_n;
};

// ---------------------------------------------------------------- operand loaders
// K-contiguous operand: R tile rows, 128 bytes of K per row, 16-byte chunks.
template <class Cfg, int R>
struct LoadKC {
  static constexpr int CH = R * 8;
  static_assert(CH % Cfg::T == 0, "chunks must divide among threads");
  static constexpr int PER = CH / Cfg::T;
  i32x4_t v[PER];

  __device__ __forceinline__ void load(const char* base, int64_t ld_bytes, int row0, int nrows,
                                       int64_t kbyte0, int64_t kbytes, int tid) {
    const char* p = base + (int64_t)row0 * ld_bytes + kbyte0;
    // bytes from p to the end of the last stored row
    uint64_t rem = (uint64_t)(nrows - row0 - 1) * (uint64_t)ld_bytes + (uint64_t)kbytes - (uint64_t)kbyte0;
    auto rs = make_rsrc(p, rem);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int id = tid + i * Cfg::T;
      int r = id >> 3, c = id & 7;
      bool ok = (row0 + r < nrows) && (kbyte0 + c * 16 < kbytes);
      uint32_t off = ok ? (uint32_t)(r * ld_bytes + c * 16) : kOobOffset;
      v[i] = buf_load16(rs, off);
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int id = tid + i * Cfg::T;
      int r = id >> 3, c = id & 7;
      *reinterpret_cast<i32x4_t*>(lds + lds_off(r, c)) = v[i];
    }
  }
};

// M/N-contiguous bf16 operand stored [K, rows]: KB(k) x 4(rows) blocks,
// transposed in registers into K-contiguous LDS rows.
template <class Cfg, int R>
struct LoadMN {
  static constexpr int KB = (2 * R >= Cfg::T) ? 8 : 4;
  static constexpr int NSUB = (64 / KB) * (R / 4);
  static_assert(NSUB % Cfg::T == 0, "blocks must divide among threads");
  static constexpr int PER = NSUB / Cfg::T;
  i32x2_t v[PER][KB];

  __device__ __forceinline__ void load(const char* base, int64_t ld_bytes, int k0, int K,
                                       int col0, int ncols, int tid) {
    const char* p = base + (int64_t)k0 * ld_bytes + (int64_t)col0 * 2;
    uint64_t rem = (uint64_t)(K - k0 - 1) * (uint64_t)ld_bytes + (uint64_t)(ncols - col0) * 2;
    auto rs = make_rsrc(p, rem);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int id = tid + i * Cfg::T;
      int kb = id / (R / 4), rb = id % (R / 4);
      bool cok = col0 + rb * 4 < ncols;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        int k = kb * KB + j;
        bool ok = cok && (k0 + k < K);
        uint32_t off = ok ? (uint32_t)(k * ld_bytes + rb * 8) : kOobOffset;
        v[i][j] = buf_load8(rs, off);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int id = tid + i * Cfg::T;
      int kb = id / (R / 4), rb = id % (R / 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w[KB / 2];
#pragma unroll
        for (int j2 = 0; j2 < KB / 2; ++j2) {
          uint32_t a = (uint32_t)v[i][2 * j2][c >> 1], b = (uint32_t)v[i][2 * j2 + 1][c >> 1];
          w[j2] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
        }
        int r = rb * 4 + c;
        if constexpr (KB == 8) {
          i32x4_t q = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
          *reinterpret_cast<i32x4_t*>(lds + lds_off(r, kb)) = q;
        } else {
          i32x2_t q = {(int)w[0], (int)w[1]};
          *reinterpret_cast<i32x2_t*>(lds + lds_off(r, kb >> 1) + (kb & 1) * 8) = q;
        }
      }
    }
  }
};

template <class Cfg, int R, bool KC>
struct Loader;
template <class Cfg, int R>
struct Loader<Cfg, R, true> : LoadKC<Cfg, R> {};
template <class Cfg, int R>
struct Loader<Cfg, R, false> : LoadMN<Cfg, R> {};

// ---------------------------------------------------------------- tile scheduling
struct TileCoord { int tm, tn; };

__device__ __forceinline__ TileCoord tile_coord(int pid, int tiles_m, int tiles_n, int group_m) {
  int ntiles = tiles_m * tiles_n;
  // XCD-aware remap: the hardware deals workgroup ids round-robin over 8 XCDs;
  // give each XCD a contiguous range of tile indices so neighbours share its L2.
  int per = ntiles / 8, rem = ntiles % 8, x = pid % 8;
  pid = x * per + (x < rem ? x : rem) + pid / 8;
  int width = group_m * tiles_n;
  int group = pid / width;
  int first_m = group * group_m;
  int gsz = min(tiles_m - first_m, group_m);
  TileCoord t;
  t.tm = first_m + (pid % width) % gsz;
  t.tn = (pid % width) / gsz;
  return t;
}

// ---------------------------------------------------------------- mainloop
template <class Cfg>
struct Acc {
  f32x16_t c[Cfg::TM][Cfg::TN];
};

template <class Cfg>
__device__ __forceinline__ void mma_stage(const char* As, const char* Bs, Acc<Cfg>& acc,
                                          int wm0, int wn0, int lane) {
  const int lr = lane & 31, hi = lane >> 5;
  if constexpr (!Cfg::FP8) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int chunk = 2 * s + hi;
      bf16x8_t a[Cfg::TM], b[Cfg::TN];
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + lds_off(wm0 + 32 * i + lr, chunk));
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + lds_off(wn0 + 32 * j + lr, chunk));
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc.c[i][j], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int chunk = 4 * s + 2 * hi;
      i32x8_t a[Cfg::TM], b[Cfg::TN];
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i) {
        int r = wm0 + 32 * i + lr;
        i32x4_t lo = *reinterpret_cast<const i32x4_t*>(As + lds_off(r, chunk));
        i32x4_t up = *reinterpret_cast<const i32x4_t*>(As + lds_off(r, chunk + 1));
        a[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
      }
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        int r = wn0 + 32 * j + lr;
        i32x4_t lo = *reinterpret_cast<const i32x4_t*>(Bs + lds_off(r, chunk));
        i32x4_t up = *reinterpret_cast<const i32x4_t*>(Bs + lds_off(r, chunk + 1));
        b[j] = i32x8_t{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
      }
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::TN; ++j)
          // format 0 = E4M3 for both operands; block scales 127 = 2^0
          acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc.c[i][j],
                                                                         0, 0, 0, 127, 0, 127);
    }
  }
}

// Runs the whole K loop for the tile at (m0, n0); acc starts at zero.
template <class Cfg>
__device__ __forceinline__ void mainloop(const GemmArgs& g, char* smem, Acc<Cfg>& acc,
                                         int m0, int n0, int wm0, int wn0, int tid, int lane) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.0f;

  Loader<Cfg, Cfg::BM, Cfg::A_KC> la;
  Loader<Cfg, Cfg::BN, Cfg::B_KC> lb;
  const char* A = static_cast<const char*>(g.A);
  const char* B = static_cast<const char*>(g.B);
  const int64_t lda_b = g.lda * Cfg::ESIZE, ldb_b = g.ldb * Cfg::ESIZE;
  const int64_t kbytes = (int64_t)g.K * Cfg::ESIZE;
  const int nk = (g.K + Cfg::BK - 1) / Cfg::BK;

  auto load_stage = [&](int kt) {
    const int k0 = kt * Cfg::BK;
    if constexpr (Cfg::A_KC) la.load(A, lda_b, m0, g.M, (int64_t)k0 * Cfg::ESIZE, kbytes, tid);
    else la.load(A, lda_b, k0, g.K, m0, g.M, tid);
    if constexpr (Cfg::B_KC) lb.load(B, ldb_b, n0, g.N, (int64_t)k0 * Cfg::ESIZE, kbytes, tid);
    else lb.load(B, ldb_b, k0, g.K, n0, g.N, tid);
  };
  auto store_stage = [&](int buf) {
    char* s = smem + buf * Cfg::STAGE_BYTES;
    la.store(s, tid);
    lb.store(s + Cfg::BM * 128, tid);
  };

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_stage(kt + 1);
    const char* s = smem + (kt & 1) * Cfg::STAGE_BYTES;
    mma_stage<Cfg>(s, s + Cfg::BM * 128, acc, wm0, wn0, lane);
    if (more) store_stage((kt + 1) & 1);
    __syncthreads();
  }
}

}  // namespace coda
