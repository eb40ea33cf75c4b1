// Shared device / host helpers of libdecode_attn (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_attn.h"

namespace da {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------- conversions
// bf16 is the upper half of an fp32 word, so widening is a shift / mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  _Float16 h;
  uint16_t b = (uint16_t)bits16;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t float_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// signed byte k (0..3) of a word, exactly as float
__device__ __forceinline__ float sbyte_to_float(uint32_t w, int k) {
  return (float)(int32_t)((int32_t)(w << (24 - 8 * k)) >> 24);
}

// ---------------------------------------------------------------- wave helpers
template <int MASK>
__device__ __forceinline__ float xor_shfl(float x) {
  return __shfl_xor(x, MASK, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace da

// ---------------------------------------------------------------- host side
namespace da_host {

inline int32_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace da_host
