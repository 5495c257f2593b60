// bf16 GEMM programs with A stored [K,M] (weight-gradient products).
#include "launch.hpp"

namespace coda {
using CfgTN = GemmCfg<kBM, kBN, 2, 4, false, false>;
using CfgTT = GemmCfg<kBM, kBN, 2, 4, false, true>;

hipError_t launch_gemm_tn(Prog p, int layout, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  if (layout == LAYOUT_TT) {
    switch (p) {
      case Prog::Store: return launch_one<CfgTT, EpiLinear<CfgTT, 0>>(g, e, s);
      case Prog::StoreF32: return launch_one<CfgTT, EpiLinear<CfgTT, EL_F32OUT>>(g, e, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p) {
    case Prog::Store: return launch_one<CfgTN, EpiLinear<CfgTN, 0>>(g, e, s);
    case Prog::StoreF32: return launch_one<CfgTN, EpiLinear<CfgTN, EL_F32OUT>>(g, e, s);
    case Prog::WgradGain: return launch_one<CfgTN, EpiWgradGain<CfgTN>>(g, e, s);
    case Prog::F32AlphaDev: return launch_one<CfgTN, EpiLinear<CfgTN, EL_F32OUT | EL_ALPHADEV>>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace coda
