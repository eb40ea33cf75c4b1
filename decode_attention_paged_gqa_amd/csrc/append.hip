// KV append with quantise-on-write: the new tokens' K/V rows go to their
// token slots (SGLang PR #29843 digest, test listing: out_cache_loc holds one
// slot per new token, written before attention runs), encoded on the way for
// the INT8 / INT4 caches of LightLLM PR #1549 ("Covered decode kernels").
//
// One wave per (token, kv-head) row, K then V; lane l holds elements 2l and
// 2l+1 (D/2 lanes active).
//   INT8:  s = fp16(max|x| / 127), 1 if that is 0; code = clamp(rne(x/s), ±127);
//          the max is a wave reduction.
//   INT4:  per 32-group (16 lanes): s = fp16((max - min) / 15), 1 if 0;
//          z = fp16(clamp(rne(-min / s), 0, 15)) (+0 for zero); nib = clamp(rne(x/s) + z, 0, 15);
//          lane l writes byte l = nib(2l) | nib(2l+1) << 4.
//   dense: the bits are copied.
// Every decision is taken in IEEE fp32 (correctly rounded division, rintf,
// round-to-nearest-even to fp16), so the codes are reproducible bit for bit.
#include "common.h"

namespace {

constexpr int kWaves = 4;

struct AppendArgs {
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int64_t* loc;
  uint8_t* k_pool;
  uint8_t* v_pool;
  uint16_t* k_scale;
  uint16_t* v_scale;
  long long rows;  // num_tokens * Hkv
  int Hkv, D, page_size;
  long long slots;  // num_pages * page_size
  int slot_stride, head_stride;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
// over the 16 lanes of a group (xor within a 16-lane row)
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float group_min(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ uint16_t half_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// fp16(v), with 0 replaced by 1 (an all-equal row or group)
__device__ __forceinline__ _Float16 scale_fp16(float v) {
  const _Float16 s = (_Float16)v;
  return s == (_Float16)0.f ? (_Float16)1.f : s;
}

template <bool IN_BF16>
__device__ __forceinline__ void load_pair(const uint8_t* row, int lane, bool on, float& x0,
                                          float& x1) {
  x0 = x1 = 0.f;
  if (!on) return;
  if (IN_BF16) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
    x0 = da::bf16_lo(w);
    x1 = da::bf16_hi(w);
  } else {
    const float2 v = reinterpret_cast<const float2*>(row)[lane];
    x0 = v.x;
    x1 = v.y;
  }
}

template <int FMT, bool IN_BF16>
__global__ __launch_bounds__(64 * kWaves) void append_kernel(const AppendArgs a) {
  const long long r = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (r >= a.rows) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const long long n = r / a.Hkv;
  const int g = (int)(r - n * a.Hkv);
  const long long slot = a.loc[n];
  if (slot < 0 || slot >= a.slots) return;  // sentinel or outside the pool
  const long long page = slot / a.page_size, off = slot - page * a.page_size;
  const long long dst = page * a.page_size * a.Hkv + off * a.slot_stride + (long long)g * a.head_stride;
  const bool on = lane < a.D / 2;
  const int in_row_bytes = a.D * (IN_BF16 ? 2 : 4);

#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint8_t* src = (kv ? a.v_new : a.k_new) + r * in_row_bytes;
    uint8_t* pool = kv ? a.v_pool : a.k_pool;
    if (FMT == DA_CACHE_DENSE) {
      if (!on) continue;
      if (IN_BF16)
        reinterpret_cast<uint32_t*>(pool + dst * in_row_bytes)[lane] =
            reinterpret_cast<const uint32_t*>(src)[lane];
      else
        reinterpret_cast<float2*>(pool + dst * in_row_bytes)[lane] =
            reinterpret_cast<const float2*>(src)[lane];
      continue;
    }
    float x0, x1;
    load_pair<IN_BF16>(src, lane, on, x0, x1);
    uint16_t* scale = kv ? a.v_scale : a.k_scale;
    if (FMT == DA_CACHE_INT8) {
      const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      const _Float16 s = scale_fp16(amax / 127.f);
      const float sf = (float)s;
      const int q0 = (int)fminf(fmaxf(rintf(x0 / sf), -127.f), 127.f);
      const int q1 = (int)fminf(fmaxf(rintf(x1 / sf), -127.f), 127.f);
      if (on)
        reinterpret_cast<uint16_t*>(pool + dst * a.D)[lane] =
            (uint16_t)((q0 & 0xff) | ((q1 & 0xff) << 8));
      if (lane == 0) scale[dst] = half_bits(s);
    } else {  // INT4
      const float mn = group_min(on ? fminf(x0, x1) : 0.f);
      const float mx = group_max(on ? fmaxf(x0, x1) : 0.f);
      const _Float16 s = scale_fp16((mx - mn) / 15.f);
      const float sf = (float)s;
      const float z = fminf(fmaxf(rintf(-mn / sf), 0.f), 15.f) + 0.f;  // a -0 code -> +0
      const int n0 = (int)fminf(fmaxf(rintf(x0 / sf) + z, 0.f), 15.f);
      const int n1 = (int)fminf(fmaxf(rintf(x1 / sf) + z, 0.f), 15.f);
      if (on) (pool + dst * (a.D / 2))[lane] = (uint8_t)(n0 | (n1 << 4));
      if (on && (lane & 15) == 0) {
        const int grp = lane >> 4;
        const uint32_t sz = (uint32_t)half_bits(s) | ((uint32_t)half_bits((_Float16)z) << 16);
        reinterpret_cast<uint32_t*>(scale)[dst * (a.D / 32) + grp] = sz;
      }
    }
  }
}

template <int FMT>
int32_t launch_fmt(const AppendArgs& a, bool bf16, hipStream_t st) {
  const unsigned blocks = (unsigned)((a.rows + kWaves - 1) / kWaves);
  if (bf16)
    hipLaunchKernelGGL((append_kernel<FMT, true>), dim3(blocks), dim3(64 * kWaves), 0, st, a);
  else
    hipLaunchKernelGGL((append_kernel<FMT, false>), dim3(blocks), dim3(64 * kWaves), 0, st, a);
  return da_host::launch_status();
}

}  // namespace

extern "C" int32_t decode_attn_append_kv(const void* k_new, const void* v_new, int32_t new_dtype,
                                         const int64_t* out_cache_loc, int32_t num_tokens,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t cache_format, void* k_pool, void* v_pool,
                                         uint16_t* k_scale, uint16_t* v_scale, int32_t page_size,
                                         int32_t num_pages, int32_t kv_layout, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || page_size <= 0 || num_pages <= 0)
    return DA_ERR_INVALID_ARG;
  if (new_dtype != DA_BF16 && new_dtype != DA_FP32) return DA_ERR_UNSUPPORTED;
  if (cache_format != DA_CACHE_DENSE && cache_format != DA_CACHE_INT8 &&
      cache_format != DA_CACHE_INT4)
    return DA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return DA_ERR_UNSUPPORTED;
  da_host::KvStrides kv;
  if (!da_host::kv_strides(kv_layout, num_kv_heads, page_size, kv)) return DA_ERR_INVALID_ARG;
  if (num_tokens == 0) return DA_OK;
  if (!k_new || !v_new || !out_cache_loc || !k_pool || !v_pool) return DA_ERR_INVALID_ARG;
  if (cache_format != DA_CACHE_DENSE && (!k_scale || !v_scale)) return DA_ERR_INVALID_ARG;
  AppendArgs a;
  a.k_new = (const uint8_t*)k_new; a.v_new = (const uint8_t*)v_new; a.loc = out_cache_loc;
  a.k_pool = (uint8_t*)k_pool; a.v_pool = (uint8_t*)v_pool;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.rows = (long long)num_tokens * num_kv_heads;
  a.Hkv = num_kv_heads; a.D = head_dim; a.page_size = page_size;
  a.slots = (long long)num_pages * page_size;
  a.slot_stride = kv.slot; a.head_stride = kv.head;
  const bool bf16 = new_dtype == DA_BF16;
  hipStream_t st = (hipStream_t)stream;
  if (cache_format == DA_CACHE_DENSE) return launch_fmt<DA_CACHE_DENSE>(a, bf16, st);
  if (cache_format == DA_CACHE_INT8) return launch_fmt<DA_CACHE_INT8>(a, bf16, st);
  return launch_fmt<DA_CACHE_INT4>(a, bf16, st);
}
