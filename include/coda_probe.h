/*
 * coda_probe.h - a measurement helper of the GEMM+epilogue library.
 *
 * The published matrix-core peak assumes the 2.4 GHz peak engine clock; under
 * a full matrix-core load the chip runs slower.  This entry point measures
 * the rate the chip sustains when the matrix cores do nothing else, the
 * achievable reference beside the published peak for the GEMM kernels'
 * roofline fractions.  It is not part of any GEMM path.
 *
 * Same conventions as coda.h: device pointers in coda_mat descriptors,
 * caller-owned memory, asynchronous on `stream`, host-side validation before
 * any HIP call, status codes.
 */
#ifndef CODA_PROBE_H_
#define CODA_PROBE_H_

#include "coda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA-only loop: `blocks` workgroups of 8 waves (two a SIMD, as in the
 * GEMM kernels), each wave issuing `iters` rounds of 4 independent
 * 32 x 32 accumulator chains with operands held in registers:
 *   dtype CODA_BF16: v_mfma_f32_32x32x16_bf16, 32768 flops an instruction;
 *   dtype CODA_E4M3: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands
 *                    and unit block scales, 131072 flops an instruction;
 *   dtype CODA_E2M1X2: the same instruction with E2M1 (FP4) operands.
 * out: fp32 1 x (3 blocks), caller-owned device memory.  Workgroup b writes
 * out[3b] = a sum of its first lane's accumulators (keeps the loop live),
 * out[3b + 1] = engine-clock cycles and out[3b + 2] = 100 MHz constant-clock
 * ticks that its first wave spent in the loop (their ratio x 100 MHz is the
 * engine clock under this load).  *flops (host) receives the loop's total
 * floating-point operations.  blocks in [1, 65536], iters in [1, 2^20]. */
coda_status coda_probe_mfma_loop(int32_t dtype, int32_t blocks, int32_t iters, const coda_mat* out, double* flops,
                                 void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CODA_PROBE_H_ */
