// MFMA-only loop: the matrix-core rate the chip sustains with nothing else in
// flight (contract in coda_probe.h).
#include "../../include/coda_probe.h"
#include "capi_util.hpp"

namespace {

// FMT: -1 = bf16, 0 = E4M3, 4 = E2M1 (the scaled MFMA's operand format)
template <int FMT>
__global__ __launch_bounds__(512) void mfma_loop_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  // operands that depend on the lane, so nothing folds; small values keep
  // the sums finite
  bf16x8_t a, b;
  i32x8_t qa, qb;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(1e-3f * (float)((lane + k) & 7));
    b[k] = (__bf16)(1e-3f * (float)((lane * 3 + k) & 7));
    qa[k] = 0x38383838 + ((lane + k) & 1);   // E4M3 bytes near 1.0 (E2M1 nibbles: small values)
    qb[k] = 0x30303030 + ((lane + 2 * k) & 1);
  }
  const uint64_t t0 = clock64(), r0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
    if constexpr (FMT >= 0) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qb, c0, FMT, FMT, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qb, qa, c1, FMT, FMT, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qa, c2, FMT, FMT, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qb, qb, c3, FMT, FMT, 0, 127, 0, 127);
    } else {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
  }
  const uint64_t t1 = clock64(), r1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (threadIdx.x == 0) {
    float* o = out + 3 * (int64_t)blockIdx.x;
    o[0] = s;
    o[1] = (float)(t1 - t0);
    o[2] = (float)(r1 - r0);
  }
}

}  // namespace

extern "C" coda_status coda_probe_mfma_loop(int32_t dtype, int32_t blocks, int32_t iters, const coda_mat* out,
                                            double* flops, void* stream) {
  if (dtype != CODA_BF16 && dtype != CODA_E4M3 && dtype != CODA_E2M1X2)
    return fail(CODA_ERR_DTYPE, "probe: dtype must be BF16, E4M3 or E2M1X2");
  if (blocks < 1 || blocks > 65536) return fail(CODA_ERR_SHAPE, "probe: blocks must be in [1, 65536]");
  if (iters < 1 || iters > (1 << 20)) return fail(CODA_ERR_SHAPE, "probe: iters must be in [1, 2^20]");
  if (!flops) return fail(CODA_ERR_NULL, "probe: flops: NULL");
  TRY(check_vec(out, "out", CODA_F32, 3 * (int64_t)blocks));
  const double per = dtype == CODA_BF16 ? 32768.0 : 131072.0;   // 32 x 32 x 16 or 32 x 32 x 64, 2 flops each
  *flops = per * 4.0 * (double)iters * 8.0 * (double)blocks;
  float* o = static_cast<float*>(out->ptr);
  if (dtype == CODA_BF16)
    hipLaunchKernelGGL(mfma_loop_kernel<-1>, dim3(blocks), dim3(512), 0, S(stream), (int)iters, o);
  else if (dtype == CODA_E4M3)
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(512), 0, S(stream), (int)iters, o);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<4>, dim3(blocks), dim3(512), 0, S(stream), (int)iters, o);
  return check_launch("probe: mfma loop");
}
