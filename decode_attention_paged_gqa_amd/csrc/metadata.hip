// Decode metadata prelude: cache_seqlens, cu_seqlens_k/q and page_table in
// one launch (SGLang PR #29843 digest, "Implementation breakdown": one
// program per batch row, three q modes, -1 sentinel guard; its tests cover
// a zero-padded page-table tail).
//
// One 256-thread workgroup per batch row b.  Row b computes its own
// exclusive prefix over rows [0, b) with a workgroup reduction, so no
// cross-workgroup scan (and no second launch) is needed; the last row also
// writes the closing entries cu_*[B].  Prefix sums are formed in 64-bit and
// stored as int32.  The optional batch order (requests by descending length,
// ties by index) is built the same way: row b counts the rows that sort
// before it and stores b at that rank.
//
// Two options ride in the same launch:
//  * SWA translation (same section: the fused kernel translates through a
//    full-to-SWA slot mapping the backend prepares): a second page table for
//    the sliding-window pool, from the mapped first slot of every page.
//  * Per-request split counts (LightLLM PR #1549, "Covered decode kernels":
//    configurations picked from the real request length over bucketed
//    keys): S_b from a per-bucket table, and the flattened work list of
//    (request, split) items that stage 1 walks, longest requests first.
//    Row b sums the counts of the rows that sort before it to find where
//    its items go; the last row in that order pads the list with -1.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBuckets = 16;

// per-request split-count table, passed by value in the kernel arguments
struct SplitTable {
  int32_t v[kMaxBuckets];
  int n, bucket_tokens, max_splits;
};

__device__ __forceinline__ int request_splits(const SplitTable& t, int L, int page_size) {
  int k = (int)(((long long)L + t.bucket_tokens - 1) / t.bucket_tokens);
  k = min(max(k, 1), t.n) - 1;
  const int n = (int)(((long long)L + page_size - 1) / page_size);
  return max(1, min(min(t.v[k], n), t.max_splits));
}

__device__ __forceinline__ long long block_sum(long long v, long long* sh) {
  // wave reduction, then across the 4 waves through LDS
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

__global__ __launch_bounds__(kThreads) void metadata_kernel(
    const int32_t* __restrict__ seq_lens, const int64_t* __restrict__ rpi,
    const int32_t* __restrict__ r2t, long long r2t_rows, long long r2t_cols,
    long long r2t_stride, int batch, int page_size, int max_pages, int q_mode,
    const int32_t* __restrict__ q_in, int q_stride, int32_t* __restrict__ cache_seqlens,
    int32_t* __restrict__ cu_k, int32_t* __restrict__ cu_q, int32_t* __restrict__ page_table,
    int32_t* __restrict__ order, const int64_t* __restrict__ f2s, long long f2s_len,
    int32_t* __restrict__ swa_pt, const SplitTable table, int32_t* __restrict__ counts,
    int32_t* __restrict__ work, int capacity, unsigned long long* checks) {
  __shared__ long long sh[4];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;

  // ---- one pass over the batch: exclusive prefixes (lengths, and q lengths
  // for cumsum), this row's rank in the batch order, and the split counts of
  // the rows ranked before it.  Every load here is independent of the others,
  // so the pass costs one memory round trip.
  const int L = max(seq_lens[b], 0);
  const long long r = rpi[b];
  const bool ranked = order || work;
  long long pk = 0, pq = 0, rank = 0, off = 0;
  for (int j = tid; j < batch; j += kThreads) {
    const int Lj = max(seq_lens[j], 0);
    if (j < b) {
      pk += Lj;
      if (q_mode == DA_Q_CUMSUM) pq += max(q_in[j], 0);
    }
    if (ranked) {
      const bool before = Lj > L || (Lj == L && j < b);
      rank += before ? 1 : 0;
      if (work && before) off += request_splits(table, Lj, page_size);
    }
  }

  // ---- page-table row: first slot of every page / page_size, zero tail.
  // Its loads need only L and r, so they go out before the reductions below.
  {
    const long long n = ((long long)L + page_size - 1) / page_size;
    const bool row_ok = r >= 0 && r < r2t_rows;
    // a negative row is the sentinel (a request with no slots), a row past
    // the table is a contract violation; so is a length the table cannot hold
    da::note(checks, tid != 0 || r < r2t_rows, DA_CHECK_REQ_ROW);
    da::note(checks, tid != 0 || (n <= max_pages && L <= r2t_cols), DA_CHECK_TOO_LONG);
    const int32_t* row = r2t + (row_ok ? r : 0) * r2t_stride;
    int32_t* out = page_table + (long long)b * max_pages;
    int32_t* swa_out = swa_pt ? swa_pt + (long long)b * max_pages : nullptr;
    for (int j = tid; j < max_pages; j += kThreads) {
      int32_t v = 0, w = 0;
      const long long col = (long long)j * page_size;
      if (row_ok && j < n && col < r2t_cols) {
        const int32_t slot = row[col];
        if (slot >= 0) {
          v = slot / page_size;
          if (swa_out && slot < f2s_len) {
            const long long m = f2s[slot];
            w = m >= 0 ? (int32_t)(m / page_size) : 0;
          }
        }
      }
      out[j] = v;
      if (swa_out) swa_out[j] = w;
    }
  }

  pk = block_sum(pk, sh);
  if (q_mode == DA_Q_CUMSUM) pq = block_sum(pq, sh);
  if (ranked) {
    rank = block_sum(rank, sh);
    if (order && tid == 0) order[rank] = b;
    if (work) {
      off = block_sum(off, sh);
      const int Sb = request_splits(table, L, page_size);
      if (tid == 0) counts[b] = Sb;
      for (int s2 = tid; s2 < Sb; s2 += kThreads)
        if (off + s2 < capacity) work[off + s2] = (b << da::kItemShift) | s2;
      if (rank == batch - 1)  // the last request in dispatch order closes the list
        for (long long u = off + Sb + tid; u < capacity; u += kThreads) work[u] = -1;
    }
  }
  if (tid == 0) {
    cache_seqlens[b] = L;
    cu_k[b] = (int32_t)pk;
    int32_t cq;
    if (q_mode == DA_Q_STRIDED) cq = (int32_t)((long long)b * q_stride);
    else if (q_mode == DA_Q_CUMSUM) cq = (int32_t)pq;
    else cq = q_in[b];
    cu_q[b] = cq;
    if (b == batch - 1) {
      cu_k[batch] = (int32_t)(pk + L);
      if (q_mode == DA_Q_STRIDED) cu_q[batch] = (int32_t)((long long)batch * q_stride);
      else if (q_mode == DA_Q_CUMSUM) cu_q[batch] = (int32_t)(pq + max(q_in[b], 0));
      else cu_q[batch] = q_in[batch];
    }
  }
}

}  // namespace

extern "C" int32_t decode_attn_metadata_ex(
    const int32_t* seq_lens, const int64_t* req_pool_indices, const int32_t* req_to_token,
    int64_t req_to_token_rows, int64_t req_to_token_cols, int64_t req_to_token_stride,
    int32_t batch, int32_t page_size, int32_t max_pages, int32_t q_mode, const int32_t* q_in,
    int32_t q_stride, int32_t* cache_seqlens, int32_t* cu_seqlens_k, int32_t* cu_seqlens_q,
    int32_t* page_table, int32_t* batch_order, const int64_t* full_to_swa,
    int64_t full_to_swa_len, int32_t* swa_page_table, const int32_t* split_table,
    int32_t n_buckets, int32_t bucket_tokens, int32_t max_splits, int32_t* split_counts,
    int32_t* work_list, int32_t work_capacity, void* stream) {
  if (!seq_lens || !req_pool_indices || !req_to_token || !cache_seqlens || !cu_seqlens_k ||
      !cu_seqlens_q || !page_table)
    return DA_ERR_INVALID_ARG;
  if (batch <= 0 || page_size <= 0 || max_pages <= 0 || req_to_token_rows <= 0 ||
      req_to_token_cols <= 0 || req_to_token_stride < req_to_token_cols)
    return DA_ERR_INVALID_ARG;
  if (q_mode != DA_Q_STRIDED && q_mode != DA_Q_CUMSUM && q_mode != DA_Q_PRESET)
    return DA_ERR_INVALID_ARG;
  if (q_mode != DA_Q_STRIDED && !q_in) return DA_ERR_INVALID_ARG;
  if (q_mode == DA_Q_STRIDED && q_stride < 0) return DA_ERR_INVALID_ARG;
  // SWA translation: mapping and output together
  if ((full_to_swa == nullptr) != (swa_page_table == nullptr)) return DA_ERR_INVALID_ARG;
  if (full_to_swa && full_to_swa_len <= 0) return DA_ERR_INVALID_ARG;
  // per-request split counts: host table, counts and work list together
  SplitTable table = {};
  const bool sched = split_table != nullptr;
  if (sched != (split_counts != nullptr) || sched != (work_list != nullptr))
    return DA_ERR_INVALID_ARG;
  if (sched) {
    if (n_buckets < 1 || n_buckets > kMaxBuckets || bucket_tokens <= 0 || max_splits < 1 ||
        max_splits > DA_MAX_SPLITS || batch >= (1 << (31 - da::kItemShift)))
      return DA_ERR_INVALID_ARG;
    int smax = 0;
    for (int k = 0; k < n_buckets; ++k) {
      if (split_table[k] < 1 || split_table[k] > DA_MAX_SPLITS) return DA_ERR_INVALID_ARG;
      table.v[k] = split_table[k];
      smax = split_table[k] > smax ? split_table[k] : smax;
    }
    if (smax > max_splits) smax = max_splits;
    // room for every request's largest possible count
    if ((long long)work_capacity < (long long)batch * smax) return DA_ERR_INVALID_ARG;
    table.n = n_buckets;
    table.bucket_tokens = bucket_tokens;
    table.max_splits = max_splits;
  }
  hipLaunchKernelGGL(metadata_kernel, dim3(batch), dim3(kThreads), 0, (hipStream_t)stream,
                     seq_lens, req_pool_indices, req_to_token, (long long)req_to_token_rows,
                     (long long)req_to_token_cols, (long long)req_to_token_stride, batch,
                     page_size, max_pages, q_mode, q_in, q_stride, cache_seqlens, cu_seqlens_k,
                     cu_seqlens_q, page_table, batch_order, full_to_swa,
                     (long long)full_to_swa_len, swa_page_table, table, split_counts, work_list,
                     sched ? work_capacity : 0, da_host::check_words());
  return da_host::launch_status();
}

extern "C" int32_t decode_attn_metadata(const int32_t* seq_lens, const int64_t* req_pool_indices,
                                        const int32_t* req_to_token, int64_t req_to_token_rows,
                                        int64_t req_to_token_cols, int64_t req_to_token_stride,
                                        int32_t batch, int32_t page_size, int32_t max_pages,
                                        int32_t q_mode, const int32_t* q_in, int32_t q_stride,
                                        int32_t* cache_seqlens, int32_t* cu_seqlens_k,
                                        int32_t* cu_seqlens_q, int32_t* page_table,
                                        int32_t* batch_order, void* stream) {
  return decode_attn_metadata_ex(seq_lens, req_pool_indices, req_to_token, req_to_token_rows,
                                 req_to_token_cols, req_to_token_stride, batch, page_size,
                                 max_pages, q_mode, q_in, q_stride, cache_seqlens, cu_seqlens_k,
                                 cu_seqlens_q, page_table, batch_order, nullptr, 0, nullptr,
                                 nullptr, 0, 0, 0, nullptr, nullptr, 0, stream);
}
