// decode_attn_decode_static: stage 1 and the merge in one call, with the
// split partials in a scratch array the library holds per device, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that must not call hipMalloc, harnesses that forbid it).
// The kernels are those of decode_attn_split / _int8 / _int4 and
// decode_attn_merge; only where the partials live differs.
#include <atomic>
#include <mutex>

#include "common.h"


namespace {

// One copy per GPU, allocated when the library's code object is loaded on
// that GPU and held until the process ends.  Host code never uses its name
// as an address: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[DA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<unsigned char*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up once per device (with
// that device current) and kept; null when HIP cannot report it.
unsigned char* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  unsigned char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = static_cast<unsigned char*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" int32_t decode_attn_decode_static(
    const void* q, int32_t q_dtype, int32_t cache_format, const void* k_pool, const void* v_pool,
    const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* page_table,
    int32_t page_table_stride, int32_t max_pages, const int32_t* cache_seqlens,
    const int32_t* batch_order, int32_t batch, int32_t q_per_req, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
    int32_t kv_layout, int32_t num_splits, const int32_t* split_counts, const int32_t* work_list,
    int32_t work_capacity, float softmax_scale, int32_t causal, void* out, int32_t out_dtype,
    float* lse_out, void* stream) {
  // the merge's own conditions first, so that a call the merge would refuse
  // enqueues nothing (stage 1 validates everything else)
  if (!out || !da_host::aligned(out, 4) || !da_host::aligned(lse_out, 4))
    return DA_ERR_INVALID_ARG;
  if (out_dtype != DA_BF16 && out_dtype != DA_FP32) return DA_ERR_UNSUPPORTED;
  if (cache_format != DA_CACHE_DENSE && cache_format != DA_CACHE_INT8 &&
      cache_format != DA_CACHE_INT4)
    return DA_ERR_INVALID_ARG;
  if (batch <= 0 || q_per_req <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0)
    return DA_ERR_INVALID_ARG;
  const long long rows = (long long)batch * q_per_req * num_q_heads;
  if (rows > (1ll << 30)) return DA_ERR_INVALID_ARG;
  // rows * S * (D + 1) floats must fit; tested by division, so that no
  // product of the (not yet validated) sizes can wrap
  const unsigned long long per_row = (unsigned long long)num_splits * ((unsigned long long)head_dim + 1);
  if (per_row > (unsigned long long)DA_STATIC_SCRATCH_BYTES / sizeof(float) / (unsigned long long)rows)
    return DA_ERR_TOO_LARGE;
  // partials: o [rows, S, D] fp32 from the start, lse [rows, S] fp32 after it
  const size_t o_bytes = align256((size_t)rows * num_splits * head_dim * sizeof(float));
  const size_t lse_bytes = (size_t)rows * num_splits * sizeof(float);
  if (o_bytes + lse_bytes > (size_t)DA_STATIC_SCRATCH_BYTES) return DA_ERR_TOO_LARGE;
  unsigned char* base = scratch_ptr();
  if (!base) return DA_ERR_LAUNCH;
  float* o_partial = reinterpret_cast<float*>(base);
  float* lse_partial = reinterpret_cast<float*>(base + o_bytes);
  int32_t st;
  if (cache_format == DA_CACHE_DENSE)
    st = decode_attn_split(q, q_dtype, k_pool, v_pool, page_table, page_table_stride, max_pages,
                           cache_seqlens, batch_order, batch, q_per_req, num_q_heads,
                           num_kv_heads, head_dim, page_size, num_pages, kv_layout, num_splits,
                           split_counts, work_list, work_capacity, softmax_scale, causal,
                           o_partial, lse_partial, stream);
  else if (cache_format == DA_CACHE_INT8)
    st = decode_attn_split_int8(q, q_dtype, (const int8_t*)k_pool, (const int8_t*)v_pool,
                                k_scale, v_scale, page_table, page_table_stride, max_pages,
                                cache_seqlens, batch_order, batch, q_per_req, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, kv_layout,
                                num_splits, split_counts, work_list, work_capacity, softmax_scale,
                                causal, o_partial, lse_partial, stream);
  else
    st = decode_attn_split_int4(q, q_dtype, (const uint8_t*)k_pool, (const uint8_t*)v_pool,
                                k_scale, v_scale, page_table, page_table_stride, max_pages,
                                cache_seqlens, batch_order, batch, q_per_req, num_q_heads,
                                num_kv_heads, head_dim, page_size, num_pages, kv_layout,
                                num_splits, split_counts, work_list, work_capacity, softmax_scale,
                                causal, o_partial, lse_partial, stream);
  if (st != DA_OK) return st;
  return decode_attn_merge(o_partial, lse_partial, batch, q_per_req, num_q_heads, head_dim,
                           num_splits, work_list ? split_counts : nullptr, out, out_dtype,
                           lse_out, stream);
}
