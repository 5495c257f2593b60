// MXFP4 GEMM programs: E2M1 operands packed two a byte, both K-contiguous
// (A [M, K/2 bytes], B stored [N, K/2 bytes]), each with one E8M0 scale per
// 32 K values of a row, applied by the scaled MFMA; the epilogue sees the
// dequantised fp32 product.  The programs are those of the generic entry
// point and of the forward functional entry points.
#include "launch.hpp"

namespace coda {
using CfgMX4 = GemmCfg<kBM, kBN, 2, 4, true, true, true, true, true>;

hipError_t launch_gemm_mx4(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  switch (p) {
    case Prog::Store: return launch_one<CfgMX4, EpiLinear<CfgMX4, 0>>(g, e, s);
    case Prog::StoreF32: return launch_one<CfgMX4, EpiLinear<CfgMX4, EL_F32OUT>>(g, e, s);
    case Prog::RowColStore: return launch_one<CfgMX4, EpiLinear<CfgMX4, EL_ROWVEC | EL_COLVEC>>(g, e, s);
    case Prog::ResidSumsq: return launch_one<CfgMX4, EpiLinear<CfgMX4, EL_TILEADD | EL_SUMSQ>>(g, e, s);
    case Prog::Resid: return launch_one<CfgMX4, EpiLinear<CfgMX4, EL_TILEADD>>(g, e, s);
    case Prog::SwiGLU: return launch_one<CfgMX4, EpiSwiGLU<CfgMX4>>(g, e, s);
    case Prog::Sigmoid: return launch_one<CfgMX4, EpiSigmoid<CfgMX4>>(g, e, s);
    case Prog::Gelu: return launch_one<CfgMX4, EpiGelu<CfgMX4>>(g, e, s);
    case Prog::QKRope: return launch_one<CfgMX4, EpiQKNormRope<CfgMX4>>(g, e, s);
    case Prog::DSwiGLU: return launch_one<CfgMX4, EpiDSwiGLU<CfgMX4>>(g, e, s);
    case Prog::DSigmoid: return launch_one<CfgMX4, EpiDSigmoid<CfgMX4>>(g, e, s);
    case Prog::DGelu: return launch_one<CfgMX4, EpiDGelu<CfgMX4>>(g, e, s);
    case Prog::NormCorr: return launch_one<CfgMX4, EpiNormCorrection<CfgMX4>>(g, e, s);
    case Prog::WgradGain: return launch_one<CfgMX4, EpiWgradGain<CfgMX4>>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace coda
