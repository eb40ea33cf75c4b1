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

// Eight consecutive query elements, starting at element e0, as floats; the
// query is bf16 (F32 false) or fp32 in memory, 16-byte aligned at e0.
template <bool F32>
__device__ __forceinline__ void load_q8(const void* q, long long e0, float (&f)[8]) {
  if constexpr (F32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + e0);
    const float4 x = p[0], y = p[1];
    f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
    f[4] = y.x; f[5] = y.y; f[6] = y.z; f[7] = y.w;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + e0);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = da::bf16_lo(w[e]);
      f[2 * e + 1] = da::bf16_hi(w[e]);
    }
  }
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

// End of a matrix-core stage-1 workgroup (256 threads): combine the per-wave
// states of its query rows, sm_acc [waves][ROWS][D] (unscaled output sums),
// sm_m / sm_l [waves][ROWS] (running reference and weight sum, log2 units),
// and write the split's partial rows r0 .. r0 + nr - 1 of kv-head g.  A row
// is taken by D / 8 threads of 8 columns each (thread t: row t / (D / 8) +
// (2048 / D) k, columns 8 * (t % (D / 8)) .. + 7), so the per-row terms are
// formed once per thread and the stores are two 16-byte writes.  lse_shift
// (log2 units) is a constant factor carried in l; the output sums carry
// 2^-acc_shift times l's factor (an exact power of two, taken out of the sum
// of weights before the division).
template <int WAVES, int ROWS = 16, int D = 128>
__device__ __forceinline__ void write_partials(const float* sm_acc, const float* sm_m,
                                               const float* sm_l, int r0, int nr, int G, int g,
                                               int b, int qn, int Hq, int S, int s,
                                               float lse_shift, float* o, float* lse,
                                               int acc_shift = 0) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int kTpr = D / 8;           // threads per row
  constexpr int kRpp = 256 / kTpr;      // rows per pass
  const int d0 = 8 * (threadIdx.x & (kTpr - 1));
#pragma unroll
  for (int k = 0; k < (ROWS + kRpp - 1) / kRpp; ++k) {
    const int r = threadIdx.x / kTpr + kRpp * k;
    if (r >= nr) return;
    float mw[WAVES], M = da::kNegInf;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      mw[w] = sm_m[w * ROWS + r];
      M = fmaxf(M, mw[w]);
    }
    float lsum = 0.f, y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != da::kNegInf) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = da::fast_exp2(mw[w] - M);
        lsum = fmaf(sm_l[w * ROWS + r], f, lsum);
        const float4* x = reinterpret_cast<const float4*>(sm_acc + (w * ROWS + r) * D + d0);
        const float4 x0 = x[0], x1 = x[1];
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fmaf(xs[e], f, y[e]);
      }
    }
    const float den = ldexpf(lsum, -acc_shift);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = lsum > 0.f ? y[e] / den : 0.f;
    const int rr = r0 + r, i = rr / G, h = g * G + rr % G;
    const long long orow = (((long long)b * qn + i) * Hq + h) * S + s;
    float4* dst = reinterpret_cast<float4*>(o + orow * D + d0);
    dst[0] = make_float4(y[0], y[1], y[2], y[3]);
    dst[1] = make_float4(y[4], y[5], y[6], y[7]);
    if (d0 == 0)
      lse[orow] = lsum > 0.f ? (M + __log2f(lsum) - lse_shift) * da::kLn2 : da::kNegInf;
  }
}

// s_waitcnt that leaves min(ahead, MAXA) tiles of LOADS loads each in flight
// (ahead is wave-uniform)
template <int LOADS, int MAXA>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  static_assert(MAXA >= 0 && MAXA * LOADS <= 63, "vmcnt range");
  if constexpr (MAXA == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= MAXA) {
      wait_vmcnt<MAXA * LOADS>();
      return;
    }
    wait_tiles_ahead<LOADS, MAXA - 1>(ahead);
  }
}

}  // namespace da_mfma
