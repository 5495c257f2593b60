// Host-side launch interface of the compiled GEMM + epilogue programs.
#pragma once
#include <hip/hip_runtime.h>
#include "epilogues.hpp"

namespace coda {

// Operand storage of a GEMM C[M,N] = A B (K = contracted axis):
//   NN: A [M,K], B [K,N]   NT: A [M,K], B [N,K]   TN: A [K,M], B [K,N]   TT: A [K,M], B [N,K]
enum Layout : int { LAYOUT_NN = 0, LAYOUT_NT = 1, LAYOUT_TN = 2, LAYOUT_TT = 3 };

enum class Prog : int {
  Store,          // bf16 store
  StoreF32,       // fp32 beta-accumulate
  RowColStore,    // row vector, column vector, bf16 store
  ResidSumsq,     // + tile, bf16 store, sum-of-squares partials
  Resid,          // + tile, bf16 store
  SwiGLU,         // row scale (finished from partials or given), SwiGLU, store, saves
  QKRope,         // row scale, QK-norm, RoPE, split store, saves
  DSwiGLU,        // dSwiGLU with saved pre-activations, r scale, store dh~, T partials
  NormCorr,       // - c u + res, bf16 store (c finished from partials)
  WgradGain,      // fp32 beta-acc of g * acc, gain partials
  CrossEntropy,   // online (max, sum-exp) partials, label gather
  CrossEntropyG,  // G = exp(z - lse) - onehot
  StoreAlphaDev,  // bf16 store of (*alpha_dev) * acc
  F32AlphaDev,    // fp32 beta-accumulate of (*alpha_dev) * acc
  CrossEntropyNorm,   // z = r acc (r from sum-of-squares partials), then as CrossEntropy
  CrossEntropyGNorm,  // z = r acc (given r), G~ = r (exp(z - lse) - onehot), T partials
  Sigmoid,        // row scale (finished from partials or given), sigmoid, store, save h
  DSigmoid,       // sigmoid backward with the saved h, r scale, store dh~, T partials
  Gelu,           // as Sigmoid with the GELU map
  DGelu,          // as DSigmoid with the GELU derivative
};

constexpr int kBM = 256, kBN = 256;

// The process-wide launch schedule of the bf16 SwiGLU program (coda_schedule):
// true selects the co-resident 128 x 256 single-group tile.
bool coresident_schedule();

inline int tiles(int n, int b) { return (n + b - 1) / b; }

// Launches program `p` with the given layout and precision; returns
// hipErrorInvalidValue when that combination is not compiled.
hipError_t launch_gemm(Prog p, int layout, bool fp8, GemmArgs g, const EpiArgs& e, hipStream_t s);

hipError_t launch_gemm_nn(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s);
hipError_t launch_gemm_nt(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s);
hipError_t launch_gemm_tn(Prog p, int layout, GemmArgs g, const EpiArgs& e, hipStream_t s);
hipError_t launch_gemm_fp8(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s);
// MXFP8 operands (g.sA, g.sB set): the programs of the generic entry point
// and of the block's forward and backward
hipError_t launch_gemm_mx(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s);
// MXFP4 operands (E2M1 packed two a byte; g.K counts bytes): the programs of
// the generic entry point
hipError_t launch_gemm_mx4(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s);
// MXFP6 operands (f6 = 2: E2M3, 3: E3M2; 32-value blocks of 24 packed bytes
// and 8 bytes of padding, so g.K counts values and bytes alike): the forward
// programs of the generic entry point and of the block
hipError_t launch_gemm_mx6(Prog p, int f6, GemmArgs g, const EpiArgs& e, hipStream_t s);

template <class Cfg, class Epi>
hipError_t launch_one(GemmArgs g, const EpiArgs& e, hipStream_t s) {
  g.tiles_m = tiles(g.M, Cfg::BM);
  g.tiles_n = tiles(g.N, Cfg::BN);
  const int ntiles = g.tiles_m * g.tiles_n;
  if (ntiles == 0) return hipSuccess;
  const int slices = g.kchunk > 0 && g.kchunk < g.K ? (g.K + g.kchunk - 1) / g.kchunk : 1;
  hipLaunchKernelGGL((gemm_epi_kernel<Cfg, Epi>), dim3(ntiles, slices), dim3(Cfg::T), 0, s, g, e);
  return hipGetLastError();
}

}  // namespace coda
