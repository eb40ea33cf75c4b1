// Test hook: dense copy of every request's tokens out of a paged pool, used
// to check page-table addressing bit-exactly.  Logical token t of request b
// is pool[page_table[b][t / page_size]][t % page_size] (the slot pool viewed
// by page, as the page table of SGLang PR #29843 digest addresses it).
//
// grid = (token blocks, batch); each thread copies 4-byte words.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 16;

__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint32_t* __restrict__ pool, long long words_per_token, int page_size, int num_pages,
    const int32_t* __restrict__ page_table, int pt_stride, int max_pages,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ cu_k,
    uint32_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int L = min(max(seqlens[b], 0), max_pages * page_size);
  const long long base = cu_k[b];
  const int t0 = blockIdx.x * kTokensPerBlock;
  for (int tt = 0; tt < kTokensPerBlock; ++tt) {
    const int t = t0 + tt;
    if (t >= L) break;
    int pid = page_table[(long long)b * pt_stride + t / page_size];
    if (pid < 0 || pid >= num_pages) pid = 0;
    const uint32_t* src = pool + ((long long)pid * page_size + t % page_size) * words_per_token;
    uint32_t* dst = out + (base + t) * words_per_token;
    for (long long w = threadIdx.x; w < words_per_token; w += kThreads) dst[w] = src[w];
  }
}

}  // namespace

extern "C" int32_t decode_attn_gather_kv(const void* pool, int64_t token_bytes, int32_t page_size,
                                         int32_t num_pages, const int32_t* page_table,
                                         int32_t page_table_stride, int32_t max_pages,
                                         const int32_t* cache_seqlens,
                                         const int32_t* cu_seqlens_k, int32_t batch, void* out,
                                         void* stream) {
  if (!pool || !page_table || !cache_seqlens || !cu_seqlens_k || !out) return DA_ERR_INVALID_ARG;
  if (token_bytes <= 0 || (token_bytes % 4) != 0 || page_size <= 0 || num_pages <= 0 ||
      max_pages <= 0 || page_table_stride < max_pages || batch <= 0)
    return DA_ERR_INVALID_ARG;
  const long long max_tokens = (long long)max_pages * page_size;
  const int blocks = (int)((max_tokens + kTokensPerBlock - 1) / kTokensPerBlock);
  hipLaunchKernelGGL(gather_kernel, dim3(blocks, batch), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint32_t*)pool, (long long)(token_bytes / 4), page_size, num_pages,
                     page_table, page_table_stride, max_pages, cache_seqlens, cu_seqlens_k,
                     (uint32_t*)out);
  return da_host::launch_status();
}
