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

// ---------------------------------------------------------------- stage-1 work units
// Stage 1 runs one workgroup per (kv-head g, split s, dispatch slot z) on a
// 1-D grid.  Workgroups reach the chip's 8 XCDs round-robin by linear id,
// and each XCD has its own L2.  Two orders:
//  * spread: id = g + Hkv * (s + S * z).  With Hkv a multiple of 8 every
//    XCD gets one kv-head of every unit, the best balance; used where a
//    kv-head's rows fill whole cache lines (dense caches).
//  * grouped: units u = z * S + s are dealt to the XCDs in rounds of 8, in
//    snake order (round r sends unit 8r + j to XCD j for even r and to XCD
//    7 - j for odd r, keeping a longest-first order balanced), and a unit's
//    Hkv heads are that XCD's next Hkv workgroups.  Short rows of
//    neighbouring kv-heads (4-bit and 8-bit codes, their scales) share cache
//    lines; this way each such line is brought into one L2, once, by
//    workgroups that run side by side.
// Dispatch slots keep their order (longest requests first with a batch order).
constexpr int kXcds = 8;

struct WorkUnit {
  int g, s, z;
};

// false for the padding workgroups of the last round of units
template <bool GROUPED>
__device__ __forceinline__ bool stage1_unit(int Hkv, int S, int B, WorkUnit& w) {
  const int i = (int)blockIdx.x;
  if (!GROUPED) {
    const int u = i / Hkv;
    w.g = i - u * Hkv;
    w.z = u / S;
    w.s = u - w.z * S;
    return true;
  }
  const int x = i % kXcds, k = i / kXcds;
  const int r = k / Hkv;
  const int u = r * kXcds + ((r & 1) ? kXcds - 1 - x : x);
  w.g = k - r * Hkv;
  w.z = u / S;
  w.s = u - w.z * S;
  return u < S * B;
}

// request of dispatch slot z: order[z] when given and in range, else z
__device__ __forceinline__ int stage1_request(const int32_t* order, int z, int B) {
  const int b = order ? order[z] : z;
  return (unsigned)b < (unsigned)B ? b : z;
}

}  // namespace da

// ---------------------------------------------------------------- host side
namespace da_host {

inline int32_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Rows between consecutive slots and between consecutive kv-heads of a
// page, for the two pool layouts; a page is page_size * Hkv rows.  Row of
// (page p, slot t, head g) = p * page_size * Hkv + t * slot + g * head.
struct KvStrides {
  int slot, head;
};
inline bool kv_strides(int32_t kv_layout, int Hkv, int page_size, KvStrides& st) {
  if (kv_layout == DA_KV_NHD) {
    st.slot = Hkv;
    st.head = 1;
    return true;
  }
  if (kv_layout == DA_KV_HND) {
    st.slot = 1;
    st.head = page_size;
    return true;
  }
  return false;
}

// Everything a stage-1 launch needs, checked by the entry point; the
// specialised kernels take it whole and return -1 for shapes they do not
// cover (the entry point then launches the generic kernel).
struct SplitCall {
  const void* q;
  int q_bf16;
  const void* k;
  const void* v;
  const uint16_t* ks;  // scales (int8) or (scale, zero) pairs (int4); null for dense
  const uint16_t* vs;
  const int32_t* pt;
  int pt_stride, max_pages;
  const int32_t* seqlens;
  const int32_t* order;
  int batch, qn, Hq, Hkv, D, ps, num_pages, S;
  KvStrides kv;
  float scale;
  int causal;
  float* o;
  float* lse;
  hipStream_t stream;
};

// 1-D grid of stage 1 (see da::stage1_unit); the grouped order pads to
// whole rounds of 8 units
inline unsigned stage1_grid(int Hkv, int S, int B, bool grouped) {
  const long long units = (long long)S * B;
  if (!grouped) return (unsigned)(units * Hkv);
  return (unsigned)(da::kXcds * (long long)Hkv * ((units + da::kXcds - 1) / da::kXcds));
}

}  // namespace da_host
