// E4M3 GEMM programs: both operands K-contiguous (A [M,K], B stored [N,K]);
// the quantisers write the transposed copies the weight-gradient products need.
#include "launch.hpp"

namespace coda {
using Cfg8 = GemmCfg<kBM, kBN, 2, 4, true, true, true>;

hipError_t launch_gemm_fp8(Prog p, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  switch (p) {
    case Prog::Store: return launch_one<Cfg8, EpiLinear<Cfg8, 0>>(g, e, s);
    case Prog::StoreF32: return launch_one<Cfg8, EpiLinear<Cfg8, EL_F32OUT>>(g, e, s);
    case Prog::ResidSumsq: return launch_one<Cfg8, EpiLinear<Cfg8, EL_TILEADD | EL_SUMSQ>>(g, e, s);
    case Prog::Resid: return launch_one<Cfg8, EpiLinear<Cfg8, EL_TILEADD>>(g, e, s);
    case Prog::SwiGLU: return launch_one<Cfg8, EpiSwiGLU<Cfg8>>(g, e, s);
    case Prog::Sigmoid: return launch_one<Cfg8, EpiSigmoid<Cfg8>>(g, e, s);
    case Prog::Gelu: return launch_one<Cfg8, EpiGelu<Cfg8>>(g, e, s);
    case Prog::QKRope: return launch_one<Cfg8, EpiQKNormRope<Cfg8>>(g, e, s);
    case Prog::DSwiGLU: return launch_one<Cfg8, EpiDSwiGLU<Cfg8>>(g, e, s);
    case Prog::DSigmoid: return launch_one<Cfg8, EpiDSigmoid<Cfg8>>(g, e, s);
    case Prog::DGelu: return launch_one<Cfg8, EpiDGelu<Cfg8>>(g, e, s);
    case Prog::NormCorr: return launch_one<Cfg8, EpiNormCorrection<Cfg8>>(g, e, s);
    case Prog::WgradGain: return launch_one<Cfg8, EpiWgradGain<Cfg8>>(g, e, s);
    case Prog::CrossEntropy: return launch_one<Cfg8, EpiCrossEntropy<Cfg8>>(g, e, s);
    case Prog::CrossEntropyG: return launch_one<Cfg8, EpiCrossEntropyGrad<Cfg8>>(g, e, s);
    case Prog::StoreAlphaDev: return launch_one<Cfg8, EpiLinear<Cfg8, EL_ALPHADEV>>(g, e, s);
    case Prog::F32AlphaDev: return launch_one<Cfg8, EpiLinear<Cfg8, EL_F32OUT | EL_ALPHADEV>>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(Prog p, int layout, bool fp8, GemmArgs g, const EpiArgs& e, hipStream_t s) {
  // E4M3 operands: block-scaled when the exponents come with the operands
  if (fp8) return layout != LAYOUT_NT ? hipErrorInvalidValue : g.sA ? launch_gemm_mx(p, g, e, s) : launch_gemm_fp8(p, g, e, s);
  switch (layout) {
    case LAYOUT_NN: return launch_gemm_nn(p, g, e, s);
    case LAYOUT_NT: return launch_gemm_nt(p, g, e, s);
    default: return launch_gemm_tn(p, layout, g, e, s);
  }
}
}  // namespace coda
