// Device-side helpers for the CDNA4 (gfx950) GEMM+epilogue kernels: vector
// types, bf16 conversion, bounds-checked buffer loads and cross-lane moves.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

namespace coda {

// Offsets at or beyond this value read as zero through a buffer resource whose
// record count is below it; used to mask loads outside the matrix.
constexpr uint32_t kOobOffset = 0xFFFFFFF0u;
constexpr uint32_t kMaxRecords = 0xFFFFFFE0u;

// The lane index, computed at the point of use by an instruction pair the
// compiler may not move or merge (volatile asm, no memory access).  Values
// derived from it inside a loop are then recomputed there instead of being
// held in a register across the loop (or spilled, when registers run out).
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  uint32_t n = bytes > kMaxRecords ? kMaxRecords : (uint32_t)bytes;
  // dword3 0x00020000: raw (untyped) buffer access on the gfx9 family
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ i32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ i32x2_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ float bf2f(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> a packed bf16 pair (lo in bits 0-15), round to nearest even;
// NaN stays NaN.  One v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f2bf(float f) { return pack_bf2(f, 0.0f) & 0xFFFFu; }
// value of f after rounding to bf16
__device__ __forceinline__ float round_bf(float f) { return bf_lo(pack_bf2(f, 0.0f)); }

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
// sigmoid through the hardware reciprocal (v_rcp_f32, 1 ulp) instead of a
// correctly rounded fp32 division, which costs about ten instructions
__device__ __forceinline__ float sigmoidf_(float t) { return __builtin_amdgcn_rcpf(1.0f + __expf(-t)); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Sum over the 64 lanes of a wave (result in every lane).
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

}  // namespace coda
