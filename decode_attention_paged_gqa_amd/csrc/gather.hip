// Test hook: dense copy of every request's tokens out of a paged pool, used
// to check page-table addressing bit-exactly.  Logical token t of request b
// is pool[page_table[b][t / page_size]][t % page_size] (the slot pool viewed
// by page, as the page table of SGLang PR #29843 digest addresses it).
//
// grid = (token blocks, batch); threads copy 2-byte units of the (slot, head) rows.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 16;

// one block per (16 tokens, request); 2-byte units, rows of any even size
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint16_t* __restrict__ pool, long long row_units, int Hkv, int slot_stride,
    int head_stride, int page_size, int num_pages, const int32_t* __restrict__ page_table,
    int pt_stride, int max_pages, const int32_t* __restrict__ seqlens,
    const int32_t* __restrict__ cu_k, uint16_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int L = min(max(seqlens[b], 0), max_pages * page_size);
  const long long base = cu_k[b];
  const int t0 = blockIdx.x * kTokensPerBlock;
  const long long token_units = row_units * Hkv;
  for (int tt = 0; tt < kTokensPerBlock; ++tt) {
    const int t = t0 + tt;
    if (t >= L) break;
    int pid = page_table[(long long)b * pt_stride + t / page_size];
    if (pid < 0 || pid >= num_pages) pid = 0;
    const long long row0 = (long long)pid * page_size * Hkv + (long long)(t % page_size) * slot_stride;
    uint16_t* dst = out + (base + t) * token_units;
    for (long long w = threadIdx.x; w < token_units; w += kThreads) {
      const long long g = w / row_units, e = w - g * row_units;
      dst[w] = pool[(row0 + g * head_stride) * row_units + e];
    }
  }
}

}  // namespace

extern "C" int32_t decode_attn_gather_kv(const void* pool, int64_t row_bytes, int32_t num_kv_heads,
                                         int32_t kv_layout, int32_t page_size, int32_t num_pages,
                                         const int32_t* page_table, int32_t page_table_stride,
                                         int32_t max_pages, const int32_t* cache_seqlens,
                                         const int32_t* cu_seqlens_k, int32_t batch, void* out,
                                         void* stream) {
  if (!pool || !page_table || !cache_seqlens || !cu_seqlens_k || !out) return DA_ERR_INVALID_ARG;
  if (row_bytes <= 0 || (row_bytes % 2) != 0 || num_kv_heads <= 0 || page_size <= 0 ||
      num_pages <= 0 || max_pages <= 0 || page_table_stride < max_pages || batch <= 0)
    return DA_ERR_INVALID_ARG;
  da_host::KvStrides kv;
  if (!da_host::kv_strides(kv_layout, num_kv_heads, page_size, kv)) return DA_ERR_INVALID_ARG;
  const long long max_tokens = (long long)max_pages * page_size;
  const int blocks = (int)((max_tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(gather_kernel, dim3(blocks, batch), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint16_t*)pool, (long long)(row_bytes / 2), num_kv_heads, kv.slot,
                     kv.head, page_size, num_pages, page_table, page_table_stride, max_pages,
                     cache_seqlens, cu_seqlens_k, (uint16_t*)out);
  return da_host::launch_status();
}
