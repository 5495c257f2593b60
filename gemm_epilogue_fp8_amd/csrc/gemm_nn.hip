// bf16 GEMM programs with A [M,K] and B [K,N] (forward products).
#include "launch.hpp"

namespace coda {
using CfgNN = GemmCfg<kBM, kBN, 2, 4, true, false>;
// the co-resident schedule: 128 x 256 tile, one group of 4 waves, two
// workgroups a compute unit
using CfgNN1 = GemmCfg<128, kBN, 1, 4, true, false>;

hipError_t launch_gemm_nn(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  switch (p) {
    case Prog::Store: return launch_one<CfgNN, EpiLinear<CfgNN, 0>>(g, e, s);
    case Prog::StoreF32: return launch_one<CfgNN, EpiLinear<CfgNN, EL_F32OUT>>(g, e, s);
    case Prog::RowColStore: return launch_one<CfgNN, EpiLinear<CfgNN, EL_ROWVEC | EL_COLVEC>>(g, e, s);
    case Prog::ResidSumsq: return launch_one<CfgNN, EpiLinear<CfgNN, EL_TILEADD | EL_SUMSQ>>(g, e, s);
    case Prog::Resid: return launch_one<CfgNN, EpiLinear<CfgNN, EL_TILEADD>>(g, e, s);
    case Prog::SwiGLU:
      if (coresident_schedule()) return launch_one<CfgNN1, EpiSwiGLU<CfgNN1>>(g, e, s);
      return launch_one<CfgNN, EpiSwiGLU<CfgNN>>(g, e, s);
    case Prog::QKRope: return launch_one<CfgNN, EpiQKNormRope<CfgNN>>(g, e, s);
    case Prog::CrossEntropy: return launch_one<CfgNN, EpiCrossEntropy<CfgNN>>(g, e, s);
    case Prog::CrossEntropyG: return launch_one<CfgNN, EpiCrossEntropyGrad<CfgNN>>(g, e, s);
    case Prog::Sigmoid: return launch_one<CfgNN, EpiSigmoid<CfgNN>>(g, e, s);
    case Prog::Gelu: return launch_one<CfgNN, EpiGelu<CfgNN>>(g, e, s);
    case Prog::CrossEntropyNorm: return launch_one<CfgNN, EpiCrossEntropy<CfgNN, true>>(g, e, s);
    case Prog::CrossEntropyGNorm: return launch_one<CfgNN, EpiCrossEntropyGrad<CfgNN, true>>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace coda
