// MXFP8 GEMM programs: E4M3 operands, both K-contiguous (A [M,K], B stored
// [N,K]), each with one E8M0 scale per 32 K values of a row, applied by the
// scaled MFMA; the epilogue sees the dequantised fp32 product.
#include "launch.hpp"

namespace coda {
using CfgMX = GemmCfg<kBM, kBN, 2, 4, true, true, true, true>;

hipError_t launch_gemm_mx(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  switch (p) {
    case Prog::Store: return launch_one<CfgMX, EpiLinear<CfgMX, 0>>(g, e, s);
    case Prog::StoreF32: return launch_one<CfgMX, EpiLinear<CfgMX, EL_F32OUT>>(g, e, s);
    case Prog::RowColStore: return launch_one<CfgMX, EpiLinear<CfgMX, EL_ROWVEC | EL_COLVEC>>(g, e, s);
    case Prog::ResidSumsq: return launch_one<CfgMX, EpiLinear<CfgMX, EL_TILEADD | EL_SUMSQ>>(g, e, s);
    case Prog::Resid: return launch_one<CfgMX, EpiLinear<CfgMX, EL_TILEADD>>(g, e, s);
    case Prog::SwiGLU: return launch_one<CfgMX, EpiSwiGLU<CfgMX>>(g, e, s);
    case Prog::Sigmoid: return launch_one<CfgMX, EpiSigmoid<CfgMX>>(g, e, s);
    case Prog::Gelu: return launch_one<CfgMX, EpiGelu<CfgMX>>(g, e, s);
    case Prog::QKRope: return launch_one<CfgMX, EpiQKNormRope<CfgMX>>(g, e, s);
    case Prog::DSwiGLU: return launch_one<CfgMX, EpiDSwiGLU<CfgMX>>(g, e, s);
    case Prog::DSigmoid: return launch_one<CfgMX, EpiDSigmoid<CfgMX>>(g, e, s);
    case Prog::DGelu: return launch_one<CfgMX, EpiDGelu<CfgMX>>(g, e, s);
    case Prog::NormCorr: return launch_one<CfgMX, EpiNormCorrection<CfgMX>>(g, e, s);
    case Prog::WgradGain: return launch_one<CfgMX, EpiWgradGain<CfgMX>>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace coda
