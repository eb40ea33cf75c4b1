// Helpers shared by the matrix-core stage-1 kernels (gfx950, wave64).
#pragma once

#include "common.h"

namespace da_mfma {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define DA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ half2_t as_h2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ uint32_t as_u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float h_lo(uint32_t w) { return (float)as_h2(w)[0]; }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)as_h2(w)[1]; }

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  half2_t h = {(_Float16)a, (_Float16)b};
  return as_u(h);
}

// value held by lane ^ 16, ^ 32 (gfx950 permlane swaps, no LDS round trip)
__device__ __forceinline__ float xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ int32_t lds_read_i32(uint32_t addr) {
  int32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}

// Power of two that brings a row of Q into fp16 range: with m = max |q|
// over the row, m * 2^sh lies in [2^14, 2^15), so every bf16 element maps
// to fp16 exactly unless it sits more than 2^28 below m (then it rounds in
// fp16's subnormal range).  0 for an all-zero row.
__device__ __forceinline__ int q_row_shift(float row_absmax) {
  int ex = 0;
  if (row_absmax > 0.f) (void)frexpf(row_absmax, &ex);  // row_absmax < 2^ex
  return 15 - ex;
}

}  // namespace da_mfma
