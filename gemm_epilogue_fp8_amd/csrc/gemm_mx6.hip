// MXFP6 GEMM programs: E2M3 or E3M2 operands, both K-contiguous (A [M, K]
// bytes, B stored [N, K] bytes), a 32-value block packed into 24 bytes and 8
// bytes of padding, each block with one E8M0 scale applied by the scaled
// MFMA; the epilogue sees the dequantised fp32 product.  The programs are
// those of the generic entry point and of the block's forward and backward.
#include "launch.hpp"

namespace coda {
template <int F6>
using CfgMX6 = GemmCfg<kBM, kBN, 2, 4, true, true, true, true, false, F6>;

template <int F6>
static hipError_t launch_mx6(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  using C = CfgMX6<F6>;
  switch (p) {
    case Prog::Store: return launch_one<C, EpiLinear<C, 0>>(g, e, s);
    case Prog::StoreF32: return launch_one<C, EpiLinear<C, EL_F32OUT>>(g, e, s);
    case Prog::RowColStore: return launch_one<C, EpiLinear<C, EL_ROWVEC | EL_COLVEC>>(g, e, s);
    case Prog::ResidSumsq: return launch_one<C, EpiLinear<C, EL_TILEADD | EL_SUMSQ>>(g, e, s);
    case Prog::Resid: return launch_one<C, EpiLinear<C, EL_TILEADD>>(g, e, s);
    case Prog::SwiGLU: return launch_one<C, EpiSwiGLU<C>>(g, e, s);
    case Prog::Sigmoid: return launch_one<C, EpiSigmoid<C>>(g, e, s);
    case Prog::Gelu: return launch_one<C, EpiGelu<C>>(g, e, s);
    case Prog::QKRope: return launch_one<C, EpiQKNormRope<C>>(g, e, s);
    case Prog::DSwiGLU: return launch_one<C, EpiDSwiGLU<C>>(g, e, s);
    case Prog::DSigmoid: return launch_one<C, EpiDSigmoid<C>>(g, e, s);
    case Prog::DGelu: return launch_one<C, EpiDGelu<C>>(g, e, s);
    case Prog::NormCorr: return launch_one<C, EpiNormCorrection<C>>(g, e, s);
    case Prog::WgradGain: return launch_one<C, EpiWgradGain<C>>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_mx6(Prog p, int f6, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  if (f6 == 2) return launch_mx6<2>(p, g, e, s);
  if (f6 == 3) return launch_mx6<3>(p, g, e, s);
  return hipErrorInvalidValue;
}
}  // namespace coda
