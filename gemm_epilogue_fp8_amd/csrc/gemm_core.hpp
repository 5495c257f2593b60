// The fixed GEMM mainloop: C[M,N] (fp32) = sum_k A[m,k] B[k,n] on gfx950
// matrix cores, bf16 (v_mfma_f32_32x32x16_bf16) or OCP E4M3
// (v_mfma_scale_f32_32x32x64_f8f6f4), the latter either with unit block
// scales (per-row / per-column scales are applied by the epilogue) or with
// one E8M0 power-of-two scale per 32 consecutive K values of every row of A
// and every column of B (MXFP8, the OCP Microscaling format), applied by the
// matrix core itself.
//
// The CODA paper (arXiv 2605.19269), §2.2 and §3.1, keeps an expert-tuned
// mainloop fixed and programs only the epilogue; this file is that fixed part.
//
// Design (CDNA4-first, not a port of the paper's Hopper kernels):
//  * Workgroup tile BM x BN = 256 x 256, 8 waves in two groups of four.  Group
//    g owns rows [128 g, 128 g + 128) of the tile; wave w of a group owns the
//    64 columns [64 w, 64 w + 64).  The hardware deals a workgroup's waves
//    round-robin over the CU's 4 SIMDs, so each SIMD holds one wave of each
//    group.
//  * Wave-group ping-pong.  The K loop runs in phases separated by
//    workgroup barriers.  In a "memory" phase a wave reads its MFMA fragments
//    of one stage pair (two 64-byte K stages) from LDS into registers and
//    issues its group's share of future global->LDS copies; in a "compute"
//    phase it only issues MFMAs (32 of them, 1024 matrix-core cycles a wave).
//    Group 1 starts one phase late, so on every SIMD one wave keeps the
//    matrix core busy while the other one moves data.  (The paper's Hopper
//    design gets the same overlap from two consumer warpgroups, §1; here it
//    is two waves per SIMD.)  A phase of two K stages rather than one halves
//    the barriers per MFMA; on MI355X that took plain-store GEMMs at 8192^3
//    from 1.09 to 1.20 PFLOP/s (row-major operands) and 1.16 to 1.24
//    (K-contiguous operands).
//  * 4 LDS stages of (256 + 256) x 64 B (64 B = 32 bf16 or 64 fp8 of K), i.e.
//    two stage pairs.  Stages stream from global memory straight into LDS
//    (buffer_load ... lds: lane l of a wave instruction writes 16 bytes at
//    lds + 16 l, no registers).  Group 0 copies the A tile of pair p + 1 in
//    its memory phase p, into the slots of pair p - 1.  Group 1, which reads
//    pair p last, copies the B tile of pair p + 2 into pair p's slots as soon
//    as its own fragment reads have landed; this is safe only because wave w
//    copies exactly the B columns that wave w of each group reads (its
//    partner in group 0 finished with them one phase earlier).  Each wave
//    waits (vmcnt) only for the pair that is read next.
//  * A K-contiguous operand tile is [rows][64 bytes] with its 16-byte chunks
//    XOR-swizzled by (r >> 2) & 3; each lane picks the global chunk that
//    belongs at its fixed LDS slot.  gfx950 LDS serves a 16-byte access 16
//    lanes at a time over 64 banks: a fragment read (16 rows, one chunk)
//    touches 16 distinct 16-byte bank groups.
//  * An M/N-contiguous operand (the weight of a forward NN product, both
//    operands of a TN weight gradient) is kept in LDS as four column blocks
//    of [32 k rows][64 columns] (128-byte rows), chunks XOR-swizzled by
//    4 ((k >> 1) & 1).  Its MFMA fragments come from ds_read_b64_tr_b16: in
//    each 16-lane group, lane i receives element i % 4 of the 4-element loads
//    of lanes 4u + i/4, so lanes pointing at (row kb + j/4, column
//    c0 + 4 (j % 4)) deliver to lane i the 4 K values kb..kb+3 of column
//    c0 + i.  Two such reads make one 8-deep K fragment; 32 lanes read 4 rows
//    x 64 bytes, which the swizzle spreads over all 64 banks.
//  * Global loads go through buffer resources: out-of-range rows, columns and
//    K tails read as zero, so ragged M, N and K need no branches.
//  * MFMA operands are swapped (the B tile feeds the instruction's A port),
//    which leaves each lane holding 4 consecutive output columns of one row:
//    8-byte bf16 stores and in-lane pairwise transforms (RoPE pairs).
//  * Workgroup ids are remapped so that the tiles one XCD (8 per chip, each
//    with its own L2) runs are neighbours, then grouped along M.
//  * MXFP8 block scales travel like the tiles: the E8M0 bytes of one stage
//    pair (128 K = 4 blocks) are one 4-byte word per operand row, stored
//    word row by word row so that the words of consecutive rows are
//    contiguous; they are copied global->LDS beside the pair
//    (buffer_load_dword ... lds, one wave instruction covers 64 rows = 256
//    contiguous bytes; with the exponents stored row by row the same copy
//    touched 64 cache lines and cost 10%) into two 2 KB slots, read in the memory
//    phase with the fragments and handed to the MFMA as its per-lane scale
//    operand.  A lane of the 32x32x64 MFMA supplies 16 K values of each of
//    the two 32-value blocks of its row, and the scale operand of lane
//    l holds the scale of block l >> 5 of row l % 32 (lane layout probed on
//    MI355X with one-hot operands and lane-distinct scales); the
//    instruction's byte select picks the block of stage 0 or 1 of the pair.
#pragma once
#include <type_traits>
#include <utility>
#include "coda_device.hpp"

namespace coda {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// global -> LDS, `size` (16 or 4) bytes a lane, lane l at lds + size l (lds is wave-uniform)
__device__ void raw_ptr_buffer_load_lds(__amdgpu_buffer_rsrc_t rsrc, lds_void_t* lds, int size, int voffset,
                                        int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.ptr.buffer.load.lds");

constexpr int kRowBytes = 64;   // bytes of K a stage holds per operand row

__device__ __forceinline__ int kc_swz(int row) { return (row >> 2) & 3; }

// byte offset of (row, 16-byte chunk) in a K-contiguous [rows][64 B] tile
__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * kRowBytes + ((chunk ^ kc_swz(row)) << 4));
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, bool A_KC_, bool B_KC_, bool FP8_ = false,
          bool MX_ = false, bool FP4_ = false, int F6_ = 0>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NWAVES = WAVES_M * WAVES_N, T = 64 * NWAVES;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr bool A_KC = A_KC_, B_KC = B_KC_, FP8 = FP8_, MX = MX_;
  // FP4: the byte operands hold two E2M1 values each; K, the tiles and the
  // copies count bytes, and only the MFMA sees values
  static constexpr bool FP4 = FP4_;
  // FP6 (F6 = the MFMA format code: 2 = E2M3, 3 = E3M2; 0 = none): a 32-value
  // block is 24 bytes of packed codes and 8 bytes of padding, so K, the tiles
  // and the copies count bytes exactly as for E4M3
  static constexpr int F6 = F6_;
  static constexpr bool FP6 = F6 != 0;
  static constexpr int WPP = FP4 ? 2 : 1;          // MX: exponent word rows a stage pair
  static constexpr int ESIZE = FP8 ? 1 : 2;
  static constexpr int BK = kRowBytes / ESIZE;     // K per stage: 32 bf16 or 64 fp8
  // LDS stages: four (two pairs) for the two-group tile; three for the
  // single-group tile, whose workgroup leaves room for a second one a CU
  static constexpr int NS = WAVES_M == 1 ? 3 : 4;
  static constexpr int STAGE_BYTES = (BM + BN) * kRowBytes;
  // MX: two slots of WPP x (BM + BN) 4-byte exponent words after the stages
  static constexpr int SCALE_OFF = NS * STAGE_BYTES;
  static constexpr int SCALE_SLOT = WPP * (BM + BN) * 4;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES + (MX ? 2 * SCALE_SLOT : 0);
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(WAVES_M == 2 || (WAVES_M == 1 && A_KC && !FP8),
                "two wave groups (the two row halves of the tile), or one bf16 group with K-contiguous A");
  static_assert(!FP8 || (A_KC && B_KC), "fp8 operands are K-contiguous");
  static_assert(!MX || FP8, "block scales come with E4M3 operands");
  static_assert(!FP4 || MX, "E2M1 operands are block-scaled");
  static_assert(!FP6 || (MX && !FP4 && (F6 == 2 || F6 == 3)), "FP6 operands are block-scaled E2M3 or E3M2");
};

struct GemmArgs {
  const void* A;   // A_KC: [M, K] (lda >= K); else [K, M] (lda >= M)
  const void* B;   // B_KC: [N, K] (ldb >= K); else [K, N] (ldb >= N)
  int64_t lda, ldb;
  int M, N, K;
  int tiles_m, tiles_n;
  int kchunk;      // split K: workgroup (x, y) runs K slice [y kchunk, (y + 1) kchunk); gridDim.y slices
  // MXFP8 only: E8M0 block exponents of A and B in word layout: word row
  // g (stride lds_a / lds_b bytes, a multiple of 4) holds one 4-byte word per
  // operand row r, bytes = the exponents of blocks 4 g .. 4 g + 3 (K values
  // 128 g .. 128 g + 127) of row r; K a multiple of 128
  const void* sA;
  const void* sB;
  int64_t lds_a, lds_b;
};

// ---------------------------------------------------------------- operand tiles
// K-contiguous operand stored [rows, K]: tile = R rows x 64 bytes of K,
// copied by the WAVES_N waves of one group; wave w copies the quarter of the
// rows that wave w of each group reads when the tile is the B operand.
template <class Cfg, int R>
struct TileKC {
  static constexpr int NI = R * kRowBytes / 1024 / Cfg::WAVES_N;   // 1 KB wave instructions per wave
  static_assert(R * kRowBytes % (1024 * Cfg::WAVES_N) == 0, "tile must split into 1 KB wave loads");

  __device__ __forceinline__ static void issue(const char* base, int64_t ld_bytes, int row0, int nrows,
                                               int64_t kbyte0, int64_t kbytes, char* lds, int w, int lane) {
    // the block-scaled mainloops (which also hold scale words) derive the
    // per-instruction offsets at each issue from the lane index instead of
    // holding them through the K loop: no spill, and faster than one lane
    // offset for all instructions with the group step in the buffer
    // resource (MXFP8 and MXFP4 GEMMs 1.6%, MXFP6 4.5%)
    if constexpr (Cfg::MX) lane = lane_here();
    const char* p = base + (int64_t)row0 * ld_bytes + kbyte0;
    const uint64_t rem = (uint64_t)(nrows - row0 - 1) * (uint64_t)ld_bytes + (uint64_t)(kbytes - kbyte0);
    const auto rs = make_rsrc(p, rem);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = NI * w + i;                        // 16 rows per instruction; wave w: rows [R/4 w, R/4 (w+1))
      const int row = 16 * q + (lane >> 2);
      const int chunk = (lane & 3) ^ kc_swz(row);      // the chunk that lives at this slot
      const bool ok = (row0 + row < nrows) && (kbyte0 + chunk * 16 < kbytes);
      const uint32_t off = ok ? (uint32_t)(row * ld_bytes + chunk * 16) : kOobOffset;
      raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + q * 1024), 16, (int)off, 0, 0, 0);
    }
  }
};

// M/N-contiguous bf16 operand stored [K, cols]: tile = BK k rows x R columns,
// copied by the WAVES_N waves of one group.  LDS holds it as R/64 column
// blocks of [BK k rows][64 columns] (128-byte rows, 4 KB a block), so that
// the 64 columns one wave reads as the B operand are one contiguous block,
// and wave w copies exactly block w.  16-byte chunks are XOR-swizzled by
// 4 ((k >> 1) & 1).
template <class Cfg, int R>
struct TileMN {
  static constexpr int ROWB = 128;                         // bytes per k row of a block
  static constexpr int BLOCK = Cfg::BK * ROWB;             // bytes per 64-column block
  static constexpr int NI = BLOCK / 1024;                  // wave instructions per block (8 k rows each)
  static_assert(Cfg::FP8 || 2 * Cfg::BK == kRowBytes, "an M/N tile has the bytes of a K-contiguous one");
  static_assert(R == 64 * Cfg::WAVES_N, "one 64-column block per wave");

  __device__ __forceinline__ static int swz(int krow) { return 4 * ((krow >> 1) & 1); }

  // lane l of instruction i of wave w: k row 8 i + l / 8, LDS chunk slot l % 8
  __device__ __forceinline__ static void issue(const char* base, int64_t ld_bytes, int k0, int K, int col0,
                                               int ncols, char* lds, int w, int lane) {
    const char* p = base + (int64_t)k0 * ld_bytes + (int64_t)col0 * 2;
    const uint64_t rem = (uint64_t)(K - k0 - 1) * (uint64_t)ld_bytes + (uint64_t)(ncols - col0) * 2;
    const auto rs = make_rsrc(p, rem);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int krow = 8 * i + (lane >> 3);
      const int chunk = (lane & 7) ^ swz(krow);            // the chunk that lives at this slot
      const int col = 64 * w + 8 * chunk;
      const bool ok = (k0 + krow < K) && (col0 + col < ncols);
      const uint32_t off = ok ? (uint32_t)(krow * ld_bytes + col * 2) : kOobOffset;
      raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + w * BLOCK + i * 1024), 16, (int)off, 0, 0, 0);
    }
  }

  // bf16x8 fragment: column r0 + (lane & 31), K values 16 s + 8 (lane >> 5) + 0..7
  __device__ __forceinline__ static bf16x8_t frag(const char* lds, int r0, int s, int lane) {
    const int j = lane & 15, g = lane >> 4;
    const int lc = (r0 & 63) + 16 * (g & 1) + 4 * (j & 3);
    const char* blk = lds + (r0 >> 6) * BLOCK;
    short4_t h[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int krow = 16 * s + 8 * (g >> 1) + 4 * half + (j >> 2);
      const int chunk = (lc >> 3) ^ swz(krow);
      const char* a = blk + krow * ROWB + chunk * 16 + (lc & 7) * 2;
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
constexpr int substeps() { return Cfg::FP8 && !Cfg::FP4 ? 1 : 2; }

template <class Cfg, bool KC, int R>
__device__ __forceinline__ typename Frags<Cfg>::T read_frag(const char* tile, int r0, int s, int lane) {
  if constexpr (Cfg::FP4) {
    // MFMA s of the stage: lanes 0-31 hold all 32 values (16 bytes) of K
    // block 2 s of their row, lanes 32-63 those of block 2 s + 1, one
    // 16-byte chunk; the matrix core reads E2M1 operands from the low 4
    // registers only
    const int row = r0 + (lane & 31);
    i32x4_t v = *reinterpret_cast<const i32x4_t*>(tile + lds_off(row, 2 * s + (lane >> 5)));
    return i32x8_t{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
  } else if constexpr (Cfg::FP6) {
    // lanes 0-31 hold K block 0 of their row, lanes 32-63 block 1: the 24
    // packed bytes (value v at bits [6 v, 6 v + 6)) at the start of the
    // block's 32, in the low 6 registers, which are all the matrix core reads.
    // Both chunks are read whole: 16-byte reads are served 16 lanes at a
    // time, so the swizzle keeps them conflict-free, whereas an 8-byte read
    // of the second chunk (32 lanes a pass) puts rows r and r + 16 on the
    // same banks.
    const int row = r0 + (lane & 31);
    const int h = lane >> 5;
    (void)s;
    i32x4_t lo = *reinterpret_cast<const i32x4_t*>(tile + lds_off(row, 2 * h));
    i32x4_t up = *reinterpret_cast<const i32x4_t*>(tile + lds_off(row, 2 * h + 1));
    return i32x8_t{lo[0], lo[1], lo[2], lo[3], up[0], up[1], 0, 0};
  } else if constexpr (Cfg::FP8) {
    // K bytes [16 h, 16 h + 16) and [32 + 16 h, 32 + 16 h + 16) of the row,
    // h = lane >> 5: the matrix core reads a lane's first 16 bytes as part of
    // K block 0 (of 32) and its last 16 as part of block 1, and scales block
    // b of row l % 32 with the scale operand of lane l % 32 + 32 b
    const int row = r0 + (lane & 31);
    const int h = lane >> 5;
    (void)s;
    i32x4_t lo = *reinterpret_cast<const i32x4_t*>(tile + lds_off(row, h));
    i32x4_t up = *reinterpret_cast<const i32x4_t*>(tile + lds_off(row, 2 + h));
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

// MXFP8: per-lane scale bytes of one stage pair, two operand tiles a
// register: word t of A holds (tile 2t, stage 0), (tile 2t + 1, stage 0),
// (tile 2t, stage 1), (tile 2t + 1, stage 1) in bytes 0..3, and likewise B.
// The MFMA's byte select then picks tile and stage with no further moves.
template <class Cfg>
struct Scales {
  static_assert(Cfg::TM % 2 == 0 && Cfg::TN == 2, "scale bytes are packed two tiles a word");
  int a[Cfg::TM / 2], b[Cfg::TN / 2];
};

// two rows' words (bytes = blocks 4p .. 4p + 3) -> the packed word of the
// lane's K half h: blocks h (stage 0) and 2 + h (stage 1) of each row
__device__ __forceinline__ int pack_scales(uint32_t w0, uint32_t w1, int sh) {
  return (int)(((w0 >> sh) & 0x00FF00FFu) | (((w1 >> sh) & 0x00FF00FFu) << 8));
}

template <class Cfg>
__device__ __forceinline__ void load_scales(const char* slot, Scales<Cfg>& sc, int wm0, int wn0, int lane) {
  // slot: BM words of A rows, then BN words of B rows
  const int sh = 8 * (lane >> 5);
  auto word = [&](int row) { return *reinterpret_cast<const uint32_t*>(slot + 4 * (row + (lane & 31))); };
#pragma unroll
  for (int t = 0; t < Cfg::TM / 2; ++t) sc.a[t] = pack_scales(word(wm0 + 64 * t), word(wm0 + 64 * t + 32), sh);
#pragma unroll
  for (int t = 0; t < Cfg::TN / 2; ++t)
    sc.b[t] = pack_scales(word(Cfg::BM + wn0 + 64 * t), word(Cfg::BM + wn0 + 64 * t + 32), sh);
}

// One MFMA of stage S with block scales; the byte selects are immediates, so
// tile indices are template arguments.  Operands swapped as in mma_frags:
// B's scale goes with the instruction's first operand.
template <class Cfg, int S, int I, int J>
__device__ __forceinline__ void mma_mx_one(const Frags<Cfg>& f, const Scales<Cfg>& sc, Acc<Cfg>& acc) {
  // operand formats: 0 = E4M3, 2 = E2M3, 3 = E3M2, 4 = E2M1
  constexpr int FMT = Cfg::FP4 ? 4 : Cfg::F6;
  acc.c[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[J], f.a[I], acc.c[I][J], FMT, FMT,
                                                                2 * S + (J & 1), sc.b[J >> 1],
                                                                2 * S + (I & 1), sc.a[I >> 1]);
}
template <class Cfg, int S, int I, int... J>
__device__ __forceinline__ void mma_mx_row(const Frags<Cfg>& f, const Scales<Cfg>& sc, Acc<Cfg>& acc,
                                           std::integer_sequence<int, J...>) {
  (mma_mx_one<Cfg, S, I, J>(f, sc, acc), ...);
}
template <class Cfg, int S, int... I>
__device__ __forceinline__ void mma_mx_all(const Frags<Cfg>& f, const Scales<Cfg>& sc, Acc<Cfg>& acc,
                                           std::integer_sequence<int, I...>) {
  (mma_mx_row<Cfg, S, I>(f, sc, acc, std::make_integer_sequence<int, Cfg::TN>{}), ...);
}
template <class Cfg, int S>
__device__ __forceinline__ void mma_frags_mx(const Frags<Cfg>& f, const Scales<Cfg>& sc, Acc<Cfg>& acc) {
  mma_mx_all<Cfg, S>(f, sc, acc, std::make_integer_sequence<int, Cfg::TM>{});
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4], lgkmcnt[11:8]; the other counters at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// s_waitcnt lgkmcnt(0), vmcnt and expcnt unconstrained
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that neither waits for outstanding memory operations nor
// lets the compiler move instructions across it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Runs the whole K loop for the tile at (m0, n0); acc starts at zero.  Every
// wave of the workgroup passes the same number of barriers (2 np + 1, np =
// stage pairs).  An odd stage count ends with a stage past K, which the buffer
// bounds read as zeros.
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
  const int np = (nk + 1) / 2;             // stage pairs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / Cfg::WAVES_N;     // 0 copies A and leads; 1 copies B and trails one phase
  const int w = wave % Cfg::WAVES_N;
  constexpr int NS = Cfg::NS;
  static_assert(NS == 4, "two stage pairs");
  constexpr int SUB = substeps<Cfg>();

  // copies one stage issues per wave (each group copies one operand tile)
  constexpr int LPS = Cfg::A_KC ? TileKC<Cfg, Cfg::BM>::NI : TileMN<Cfg, Cfg::BM>::NI;
  static_assert(LPS == (Cfg::B_KC ? TileKC<Cfg, Cfg::BN>::NI : TileMN<Cfg, Cfg::BN>::NI),
                "both groups issue the same number of copies");

  auto issue_stage = [&](int kt) {
    char* As = smem + (kt % NS) * Cfg::STAGE_BYTES;
    char* Bs = As + Cfg::BM * kRowBytes;
    const int k0 = kt * Cfg::BK;
    if (grp == 0) {
      if constexpr (Cfg::A_KC)
        TileKC<Cfg, Cfg::BM>::issue(A, lda_b, m0, g.M, (int64_t)k0 * Cfg::ESIZE, kbytes, As, w, lane);
      else
        TileMN<Cfg, Cfg::BM>::issue(A, lda_b, k0, g.K, m0, g.M, As, w, lane);
    } else {
      if constexpr (Cfg::B_KC)
        TileKC<Cfg, Cfg::BN>::issue(B, ldb_b, n0, g.N, (int64_t)k0 * Cfg::ESIZE, kbytes, Bs, w, lane);
      else
        TileMN<Cfg, Cfg::BN>::issue(B, ldb_b, k0, g.K, n0, g.N, Bs, w, lane);
    }
  };
  // MXFP8: the 4 block exponents (one word) of stage pair p for rows
  // [64 w, 64 w + 64) of this group's operand tile, from word row p; wave w
  // of group 1 copies the words of exactly the B rows that wave w of each
  // group reads
  // E2M1 (FP4): a stage of 64 bytes holds 128 values, so each stage has a
  // word row of its own and a pair copies two (WPP); a word row past the
  // last one (an odd stage count) gets an empty buffer range and reads as 0
  auto issue_scales = [&](int p) {
    if constexpr (Cfg::MX) {
      const bool a = grp == 0;
      const char* base = static_cast<const char*>(a ? g.sA : g.sB);
      const int64_t ld = a ? g.lds_a : g.lds_b;
      const int row0 = a ? m0 : n0, nrows = a ? g.M : g.N;
      const int r = 64 * w + lane;
      const int nwords = Cfg::FP4 ? nk : np;
      const uint32_t off = (row0 + r < nrows) ? (uint32_t)(4 * r) : kOobOffset;
#pragma unroll
      for (int t = 0; t < Cfg::WPP; ++t) {
        const int wr = Cfg::WPP * p + t;
        const auto rs = make_rsrc(base + (int64_t)wr * ld + 4 * (int64_t)row0,
                                  wr < nwords ? 4 * (uint64_t)(nrows - row0) : 0);
        char* dst = smem + Cfg::SCALE_OFF + (p & 1) * Cfg::SCALE_SLOT + t * (Cfg::BM + Cfg::BN) * 4 +
                    (a ? 0 : 4 * Cfg::BM) + 256 * w;
        raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 4, (int)off, 0, 0, 0);
      }
    }
  };
  auto issue_pair = [&](int p) { issue_stage(2 * p); issue_stage(2 * p + 1); issue_scales(p); };
  // copies a wave issues per stage pair
  constexpr int PAIR_LOADS = 2 * LPS + (Cfg::MX ? Cfg::WPP : 0);
  static_assert(!Cfg::MX || (Cfg::BM == 256 && Cfg::BN == 256 && Cfg::WAVES_N == 4),
                "one 64-row scale instruction per wave covers a 256-row tile");

  // prologue: group 0 copies the A tiles of pair 0, group 1 the B tiles of
  // pairs 0 and 1; pair 0 must land
  issue_pair(0);
  if (grp == 1 && np > 1) {
    issue_pair(1);
    wait_vmcnt<PAIR_LOADS>();
  } else {
    wait_vmcnt<0>();
  }
  phase_barrier();                         // pair 0 is complete
  if (grp == 1) phase_barrier();           // group 1 trails by one phase

  for (int p = 0; p < np; ++p) {
    // ---- memory phase: fragments of pair p
    const char* S0 = smem + ((2 * p) % NS) * Cfg::STAGE_BYTES;
    const char* S1 = smem + ((2 * p + 1) % NS) * Cfg::STAGE_BYTES;
    Frags<Cfg> f[2 * SUB];
#pragma unroll
    for (int s = 0; s < SUB; ++s) load_frags<Cfg>(S0, S0 + Cfg::BM * kRowBytes, s, f[s], wm0, wn0, lane);
#pragma unroll
    for (int s = 0; s < SUB; ++s) load_frags<Cfg>(S1, S1 + Cfg::BM * kRowBytes, s, f[SUB + s], wm0, wn0, lane);
    Scales<Cfg> sc[Cfg::WPP];              // one set a word row: the pair (E4M3) or each stage (E2M1)
    if constexpr (Cfg::MX) {
#pragma unroll
      for (int t = 0; t < Cfg::WPP; ++t)
        load_scales<Cfg>(smem + Cfg::SCALE_OFF + (p & 1) * Cfg::SCALE_SLOT + t * (Cfg::BM + Cfg::BN) * 4, sc[t],
                         wm0, wn0, lane);
    }
    // Pair p + 1 must land before the barrier that ends the phase in which
    // group 1 reads pair p (group 0 reads pair p + 1 in the next one).
    if (grp == 0) {
      // A of pair p + 1 into the slots of pair p - 1, which group 1 finished
      // reading in the previous phase
      if (p + 1 < np) issue_pair(p + 1);
      wait_lgkmcnt0();                     // fragments in registers
    } else {
      // B of pair p + 2 into the slots of pair p.  Wave w copies exactly the
      // B columns that wave w of either group reads: group 0 read them in the
      // previous phase and this wave's own reads have landed, so no other
      // wave still needs what is overwritten.
      wait_lgkmcnt0();
      if (p + 2 < np) {
        issue_pair(p + 2);
        wait_vmcnt<PAIR_LOADS>();          // pair p + 1 has landed
      } else {
        wait_vmcnt<0>();
      }
    }
    phase_barrier();
    // ---- compute phase
    if constexpr (Cfg::MX && Cfg::FP4) {
      // f[2 t + s]: stage t, MFMA s; blocks 2 s and 2 s + 1 of stage t's word
      mma_frags_mx<Cfg, 0>(f[0], sc[0], acc);
      mma_frags_mx<Cfg, 1>(f[1], sc[0], acc);
      mma_frags_mx<Cfg, 0>(f[2], sc[Cfg::WPP - 1], acc);
      mma_frags_mx<Cfg, 1>(f[3], sc[Cfg::WPP - 1], acc);
    } else if constexpr (Cfg::MX) {
      // f[t]: stage t, K blocks 2 t and 2 t + 1 of the pair's word
      mma_frags_mx<Cfg, 0>(f[0], sc[0], acc);
      mma_frags_mx<Cfg, 1>(f[1], sc[0], acc);
    } else {
#pragma unroll
      for (int s = 0; s < 2 * SUB; ++s) mma_frags<Cfg>(f[s], acc);
    }
    if (grp == 0) wait_vmcnt<0>();         // A of pair p + 1 has landed
    phase_barrier();
  }
  if (grp == 0) phase_barrier();           // realign: both groups have passed 2 np + 1 barriers
}

// Single wave group (WAVES_M == 1, the co-resident schedule): every wave
// copies its share of both operand tiles of a stage and computes its
// WM x WN block.  Three stages: while stage kt is multiplied, stage kt + 1
// has landed (its fragments are read into the second register set) and
// stage kt + 2 is in flight.  One barrier a stage.  The workgroup (4 waves,
// 3 stages, at most 256 registers a lane) is sized so that two share a
// compute unit: while one runs its epilogue or drains its stores, the
// other's matrix instructions keep the cores busy, which is the
// co-residency form of hiding one tile's epilogue under another tile's
// mainloop.
template <class Cfg>
__device__ __forceinline__ void mainloop_solo(const GemmArgs& g, char* smem, Acc<Cfg>& acc,
                                              int m0, int n0, int wm0, int wn0, int tid, int lane) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc.c[i][j][e] = 0.0f;

  static_assert(Cfg::WAVES_M == 1 && Cfg::NS == 3 && !Cfg::FP8, "one bf16 wave group, three stages");
  const char* A = static_cast<const char*>(g.A);
  const char* B = static_cast<const char*>(g.B);
  const int64_t lda_b = g.lda * Cfg::ESIZE, ldb_b = g.ldb * Cfg::ESIZE;
  const int64_t kbytes = (int64_t)g.K * Cfg::ESIZE;
  const int nk = (g.K + Cfg::BK - 1) / Cfg::BK;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int SUB = substeps<Cfg>();
  // copies a wave issues a stage: its share of the A tile and of the B tile
  constexpr int LPS = TileKC<Cfg, Cfg::BM>::NI + (Cfg::B_KC ? TileKC<Cfg, Cfg::BN>::NI : TileMN<Cfg, Cfg::BN>::NI);

  auto issue_stage = [&](int kt, int slot) {
    char* As = smem + slot * Cfg::STAGE_BYTES;
    char* Bs = As + Cfg::BM * kRowBytes;
    const int64_t kb0 = (int64_t)kt * Cfg::BK * Cfg::ESIZE;
    TileKC<Cfg, Cfg::BM>::issue(A, lda_b, m0, g.M, kb0, kbytes, As, w, lane);
    if constexpr (Cfg::B_KC)
      TileKC<Cfg, Cfg::BN>::issue(B, ldb_b, n0, g.N, kb0, kbytes, Bs, w, lane);
    else
      TileMN<Cfg, Cfg::BN>::issue(B, ldb_b, kt * Cfg::BK, g.K, n0, g.N, Bs, w, lane);
  };

  // No branches in the loop: stages past K are copied as zeros (every chunk
  // out of the buffer range) and the loop runs over an even number of
  // stages, so the reads, copies and MFMAs of a step form one block that
  // the scheduler can interleave.
  const int nk2 = (nk + 1) & ~1;
  issue_stage(0, 0);
  issue_stage(1, 1);
  Frags<Cfg> f[2][SUB];
  wait_vmcnt<LPS>();
  phase_barrier();                         // stage 0 has landed for every wave
#pragma unroll
  for (int s = 0; s < SUB; ++s) load_frags<Cfg>(smem, smem + Cfg::BM * kRowBytes, s, f[0][s], wm0, wn0, lane);
  int nx = 1;                              // slot of stage kt + 1
  auto step = [&](int kt, Frags<Cfg>(&cur)[SUB], Frags<Cfg>(&nxt)[SUB]) {
    wait_vmcnt<0>();                       // this wave's copies of stage kt + 1 have landed
    wait_lgkmcnt0();                       // cur (stage kt) is in registers
    // every wave's copies of stage kt + 1 have landed and every wave has
    // read stage kt, so the slot of stage kt - 1 is free for stage kt + 2
    phase_barrier();
    // the fragment reads go ahead of the copies: the compiler waits for
    // every copy in flight before a transposed LDS read, so a copy issued
    // ahead of them would be waited for at once
    const char* S1 = smem + nx * Cfg::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < SUB; ++s) load_frags<Cfg>(S1, S1 + Cfg::BM * kRowBytes, s, nxt[s], wm0, wn0, lane);
    issue_stage(kt + 2, nx == 2 ? 0 : nx + 1);
#pragma unroll
    for (int s = 0; s < SUB; ++s) mma_frags<Cfg>(cur[s], acc);
    // order: the DS reads (0x100) and the copies (0x020, which write LDS and
    // so stay behind the reads) go out within the first MFMAs (0x008), so
    // the copies have the rest of the step to land
    constexpr int NMMA = SUB * Cfg::TM * Cfg::TN;
    constexpr int NRD = SUB * (Cfg::TM + (Cfg::B_KC ? 1 : 2) * Cfg::TN);
    static_assert(NMMA > 3, "MFMAs to hide the reads and copies behind");
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NRD / 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NRD - NRD / 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, LPS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NMMA - 3, 0);
    __builtin_amdgcn_sched_barrier(0);
    nx = nx == 2 ? 0 : nx + 1;
  };
  for (int kt = 0; kt < nk2; kt += 2) {
    step(kt, f[0], f[1]);
    step(kt + 1, f[1], f[0]);
  }
  wait_vmcnt<0>();                         // the zero stages past the end have landed too
  wait_lgkmcnt0();
  phase_barrier();                         // every wave is done reading LDS before the epilogue reuses it
}

}  // namespace coda
