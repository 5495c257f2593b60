// bf16 GEMM programs with A [M,K] and B stored [N,K] (input-gradient products).
#include "launch.hpp"

namespace coda {
using CfgNT = GemmCfg<kBM, kBN, 2, 4, true, true>;

hipError_t launch_gemm_nt(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  switch (p) {
    case Prog::Store: return launch_one<CfgNT, EpiLinear<CfgNT, 0>>(g, e, s);
    case Prog::StoreF32: return launch_one<CfgNT, EpiLinear<CfgNT, EL_F32OUT>>(g, e, s);
    case Prog::DSwiGLU: return launch_one<CfgNT, EpiDSwiGLU<CfgNT>>(g, e, s);
    case Prog::DSigmoid: return launch_one<CfgNT, EpiDSigmoid<CfgNT>>(g, e, s);
    case Prog::DGelu: return launch_one<CfgNT, EpiDGelu<CfgNT>>(g, e, s);
    case Prog::NormCorr: return launch_one<CfgNT, EpiNormCorrection<CfgNT>>(g, e, s);
    case Prog::StoreAlphaDev: return launch_one<CfgNT, EpiLinear<CfgNT, EL_ALPHADEV>>(g, e, s);
    case Prog::F32AlphaDev: return launch_one<CfgNT, EpiLinear<CfgNT, EL_F32OUT | EL_ALPHADEV>>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace coda
