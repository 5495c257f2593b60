// The fixed GEMM mainloop: C[M,N] (fp32) = sum_k A[m,k] B[k,n] on gfx950
// matrix cores, bf16 (v_mfma_f32_32x32x16_bf16) or OCP E4M3
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales).
//
// The CODA paper (arXiv 2605.19269), §2.2 and §3.1, keeps an expert-tuned
// mainloop fixed and programs only the epilogue; this file is that fixed part.
//
// Design (CDNA4-first, not a port of the paper's Hopper kernels):
//  * Workgroup tile BM x BN, 128 bytes of K per stage (64 bf16 or 128 fp8),
//    two LDS stages: while the MFMAs of stage k run, stage k+1 streams from
//    global memory straight into the other LDS buffer (buffer_load ... lds:
//    lane l of a wave instruction writes 16 bytes at lds + 16 l), so no
//    registers stage the operands.  One barrier per stage.
//  * A K-contiguous operand tile is [rows][128 bytes] with its 16-byte chunks
//    XOR-swizzled by (r ^ r>>2 ^ r>>3) & 7; each lane picks the global chunk
//    that belongs at its fixed LDS slot.  gfx950 LDS serves a 16-byte access
//    16 lanes at a time over 64 banks: the fragment reads (16 rows, one
//    chunk) and the stores (2 rows, 8 chunks) both hit 16 distinct slots.
//  * An M/N-contiguous operand (the weight of a forward NN product, both
//    operands of a TN weight gradient) keeps its storage order in LDS:
//    [64 k rows][R columns], chunks XOR-swizzled by 4 (k & 3).  Its MFMA
//    fragments come from ds_read_b64_tr_b16: in each 16-lane group, lane i
//    receives element i % 4 of the 4-element loads of lanes 4u + i/4, so
//    lanes pointing at (row kb + j/4, column c0 + 4 (j % 4)) deliver to lane
//    i the 4 K values kb..kb+3 of column c0 + i.  Two such reads make one
//    8-deep K fragment; 32 lanes read 4 rows x 64 bytes, bank-conflict free.
//  * Global loads go through buffer resources: out-of-range rows, columns and
//    K tails read as zero, so ragged M, N and K need no branches.
//  * MFMA operands are swapped (the B tile feeds the instruction's A port),
//    which leaves each lane holding 4 consecutive output columns of one row:
//    8-byte bf16 stores and in-lane pairwise transforms (RoPE pairs).
//  * Fragments of substep s+1 are read while substep s multiplies (pinned
//    with scheduling barriers).
//  * Workgroup ids are remapped so that the tiles one XCD (8 per chip, each
//    with its own L2) runs are neighbours, then grouped along M.
#pragma once
#include <type_traits>
#include "coda_device.hpp"

namespace coda {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// global -> LDS, 16 bytes a lane, lane l at lds + 16 l (lds is wave-uniform)
__device__ void raw_ptr_buffer_load_lds(__amdgpu_buffer_rsrc_t rsrc, lds_void_t* lds, int size, int voffset,
                                        int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.ptr.buffer.load.lds");

__device__ __forceinline__ int kc_swz(int row) { return (row ^ (row >> 2) ^ (row >> 3)) & 7; }

// byte offset of (row, 16-byte chunk) in a K-contiguous [rows][128 B] tile
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ kc_swz(row)) << 4));
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

// ---------------------------------------------------------------- operand tiles
// K-contiguous operand stored [rows, K]: tile = R rows x 128 bytes of K.
template <class Cfg, int R>
struct TileKC {
  static constexpr int NI = R * 128 / 1024 / Cfg::NWAVES;   // 1 KB wave instructions per wave
  static_assert(R * 128 % (1024 * Cfg::NWAVES) == 0, "tile must split into 1 KB wave loads");

  __device__ __forceinline__ static void issue(const char* base, int64_t ld_bytes, int row0, int nrows,
                                               int64_t kbyte0, int64_t kbytes, char* lds, int wave, int lane) {
    const char* p = base + (int64_t)row0 * ld_bytes + kbyte0;
    const uint64_t rem = (uint64_t)(nrows - row0 - 1) * (uint64_t)ld_bytes + (uint64_t)(kbytes - kbyte0);
    const auto rs = make_rsrc(p, rem);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = wave + Cfg::NWAVES * i;            // 8 rows per instruction
      const int row = 8 * q + (lane >> 3);
      const int chunk = (lane & 7) ^ kc_swz(row);      // the chunk that lives at this slot
      const bool ok = (row0 + row < nrows) && (kbyte0 + chunk * 16 < kbytes);
      const uint32_t off = ok ? (uint32_t)(row * ld_bytes + chunk * 16) : kOobOffset;
      raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + q * 1024), 16, (int)off, 0, 0, 0);
    }
  }
};

// M/N-contiguous bf16 operand stored [K, cols]: tile = 64 k rows x R columns.
template <class Cfg, int R>
struct TileMN {
  static constexpr int ROWB = 2 * R;                       // bytes per k row
  static constexpr int CPR = ROWB / 16;                    // chunks per k row
  static constexpr int RPI = 1024 / ROWB;                  // k rows per wave instruction
  static constexpr int NI = 64 * ROWB / 1024 / Cfg::NWAVES;
  static_assert(64 * ROWB % (1024 * Cfg::NWAVES) == 0, "tile must split into 1 KB wave loads");
  static_assert(CPR >= 16, "swizzle needs at least 16 chunks a row");

  __device__ __forceinline__ static int swz(int krow) { return 4 * (krow & 3); }

  __device__ __forceinline__ static void issue(const char* base, int64_t ld_bytes, int k0, int K, int col0,
                                               int ncols, char* lds, int wave, int lane) {
    const char* p = base + (int64_t)k0 * ld_bytes + (int64_t)col0 * 2;
    const uint64_t rem = (uint64_t)(K - k0 - 1) * (uint64_t)ld_bytes + (uint64_t)(ncols - col0) * 2;
    const auto rs = make_rsrc(p, rem);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = wave + Cfg::NWAVES * i;
      const int krow = RPI * q + lane / CPR;
      const int chunk = (lane % CPR) ^ swz(krow);
      const bool ok = (k0 + krow < K) && (col0 + chunk * 8 < ncols);
      const uint32_t off = ok ? (uint32_t)(krow * ld_bytes + chunk * 16) : kOobOffset;
      raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + q * 1024), 16, (int)off, 0, 0, 0);
    }
  }

  // bf16x8 fragment: column r0 + (lane & 31), K values 16 s + 8 (lane >> 5) + 0..7
  __device__ __forceinline__ static bf16x8_t frag(const char* lds, int r0, int s, int lane) {
    const int j = lane & 15, g = lane >> 4;
    const int col = r0 + 16 * (g & 1) + 4 * (j & 3);
    short4_t h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int krow = 16 * s + 8 * (g >> 1) + 4 * half + (j >> 2);
      const int chunk = (col >> 3) ^ swz(krow);
      const char* a = lds + krow * ROWB + chunk * 16 + (col & 7) * 2;
      h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)a);
    }
    short8_t v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

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

// Operand fragments of one K substep: bf16 substeps are 16 deep (8 K values a
// lane), fp8 substeps 64 deep (32 K values a lane).
template <class Cfg>
struct Frags {
  using T = typename std::conditional<Cfg::FP8, i32x8_t, bf16x8_t>::type;
  T a[Cfg::TM], b[Cfg::TN];
};

template <class Cfg>
constexpr int substeps() { return Cfg::FP8 ? 2 : 4; }

template <class Cfg, bool KC, int R>
__device__ __forceinline__ typename Frags<Cfg>::T read_frag(const char* tile, int r0, int s, int lane) {
  if constexpr (Cfg::FP8) {
    const int row = r0 + (lane & 31);
    const int chunk = 4 * s + 2 * (lane >> 5);
    i32x4_t lo = *reinterpret_cast<const i32x4_t*>(tile + lds_off(row, chunk));
    i32x4_t up = *reinterpret_cast<const i32x4_t*>(tile + lds_off(row, chunk + 1));
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
  } else if constexpr (KC) {
    return *reinterpret_cast<const bf16x8_t*>(tile + lds_off(r0 + (lane & 31), 2 * s + (lane >> 5)));
  } else {
    return TileMN<Cfg, R>::frag(tile, r0, s, lane);
  }
}

template <class Cfg>
__device__ __forceinline__ void load_frags(const char* As, const char* Bs, int s, Frags<Cfg>& f,
                                           int wm0, int wn0, int lane) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) f.a[i] = read_frag<Cfg, Cfg::A_KC, Cfg::BM>(As, wm0 + 32 * i, s, lane);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) f.b[j] = read_frag<Cfg, Cfg::B_KC, Cfg::BN>(Bs, wn0 + 32 * j, s, lane);
}

template <class Cfg>
__device__ __forceinline__ void mma_frags(const Frags<Cfg>& f, Acc<Cfg>& acc) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      if constexpr (!Cfg::FP8)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc.c[i][j], 0, 0, 0);
      else
        // format 0 = E4M3 for both operands; block scales 127 = 2^0
        acc.c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc.c[i][j],
                                                                       0, 0, 0, 127, 0, 127);
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

  const char* A = static_cast<const char*>(g.A);
  const char* B = static_cast<const char*>(g.B);
  const int64_t lda_b = g.lda * Cfg::ESIZE, ldb_b = g.ldb * Cfg::ESIZE;
  const int64_t kbytes = (int64_t)g.K * Cfg::ESIZE;
  const int nk = (g.K + Cfg::BK - 1) / Cfg::BK;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NS = substeps<Cfg>();

  auto issue_stage = [&](int kt, int buf) {
    char* As = smem + buf * Cfg::STAGE_BYTES;
    char* Bs = As + Cfg::BM * 128;
    const int k0 = kt * Cfg::BK;
    if constexpr (Cfg::A_KC)
      TileKC<Cfg, Cfg::BM>::issue(A, lda_b, m0, g.M, (int64_t)k0 * Cfg::ESIZE, kbytes, As, wave, lane);
    else
      TileMN<Cfg, Cfg::BM>::issue(A, lda_b, k0, g.K, m0, g.M, As, wave, lane);
    if constexpr (Cfg::B_KC)
      TileKC<Cfg, Cfg::BN>::issue(B, ldb_b, n0, g.N, (int64_t)k0 * Cfg::ESIZE, kbytes, Bs, wave, lane);
    else
      TileMN<Cfg, Cfg::BN>::issue(B, ldb_b, k0, g.K, n0, g.N, Bs, wave, lane);
  };

  issue_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wave's stage-0 copies are in LDS
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int p = kt & 1;
    if (kt + 1 < nk) issue_stage(kt + 1, 1 - p);   // that buffer was released by the last barrier
    const char* As = smem + p * Cfg::STAGE_BYTES;
    const char* Bs = As + Cfg::BM * 128;
    if constexpr (Cfg::FP8) {
      // fp8 fragments are 8 registers each: one set, read just before use
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Frags<Cfg> f;
        load_frags<Cfg>(As, Bs, s, f, wm0, wn0, lane);
        mma_frags<Cfg>(f, acc);
        __builtin_amdgcn_sched_barrier(0);   // do not hoist the next substep's reads
      }
    } else {
      Frags<Cfg> f[2];
      load_frags<Cfg>(As, Bs, 0, f[0], wm0, wn0, lane);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s + 1 < NS) load_frags<Cfg>(As, Bs, s + 1, f[(s + 1) & 1], wm0, wn0, lane);
        // keep the reads of substep s+1 ahead of the MFMAs of substep s
        __builtin_amdgcn_sched_barrier(0);
        mma_frags<Cfg>(f[s & 1], acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): stage kt+1 has landed in LDS
    __syncthreads();
  }
}

}  // namespace coda
