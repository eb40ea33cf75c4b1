// C-ABI entry points of stage 1 (decode_attn_split, decode_attn_split_int8,
// decode_attn_split_int4; LightLLM PR #1549, "Covered decode kernels": the
// GQA flash-decode stage 1 with its num_splits tunable and the INT8 / INT4
// KV stage-1 kernels).  Each entry point validates the whole call on the
// host, then hands it to the kernels built for its cache format; every
// kernel returns -1 for a shape it does not take, and the entry point then
// tries the next one or reports DA_ERR_UNSUPPORTED.  Nothing here touches
// device memory.
#include <float.h>

#include "common.h"

namespace {

int32_t check_common(const da_host::SplitCall& c, int32_t kv_layout) {
  if (!c.q || !c.k || !c.v || !c.pt || !c.seqlens || !c.o || !c.lse) return DA_ERR_INVALID_ARG;
  // 16-byte vector loads and stores (see "Alignment" in the header)
  if (!da_host::aligned(c.q, 16) || !da_host::aligned(c.k, 16) || !da_host::aligned(c.v, 16) ||
      !da_host::aligned(c.o, 16) || !da_host::aligned(c.ks, 4) || !da_host::aligned(c.vs, 4))
    return DA_ERR_INVALID_ARG;
  if (c.batch <= 0 || c.batch > 65535 || c.qn <= 0 || c.qn > DA_MAX_Q_PER_REQ || c.Hq <= 0 ||
      c.Hkv <= 0 || c.Hq % c.Hkv != 0 || c.num_pages <= 0 || c.max_pages <= 0 ||
      c.pt_stride < c.max_pages || c.S <= 0 || c.S > DA_MAX_SPLITS || c.ps <= 0)
    return DA_ERR_INVALID_ARG;
  if ((long long)c.max_pages * c.ps > (1ll << 30)) return DA_ERR_INVALID_ARG;
  // a work list needs the per-request counts and at most one entry per split slot
  if (c.work && (!c.counts || c.units <= 0 || (long long)c.units > (long long)c.batch * c.S))
    return DA_ERR_INVALID_ARG;
  if (kv_layout != DA_KV_NHD && kv_layout != DA_KV_HND) return DA_ERR_INVALID_ARG;
  // a softmax temperature: finite and positive (NaN fails both comparisons)
  if (!(c.scale > 0.f && c.scale <= FLT_MAX)) return DA_ERR_INVALID_ARG;
  if (c.D != 64 && c.D != 128) return DA_ERR_UNSUPPORTED;
  if (!da_host::is_pow2(c.ps) || c.ps < 16 || c.ps > 256) return DA_ERR_UNSUPPORTED;
  // offsets inside a page are 32-bit in the kernels: a page (page_size slots
  // of Hkv rows, at most 4 D bytes each) must stay below 2^31 bytes
  if ((long long)c.ps * c.Hkv * c.D * 4 >= (1ll << 31)) return DA_ERR_UNSUPPORTED;
  if (c.Hq / c.Hkv > (1 << 20)) return DA_ERR_INVALID_ARG;
  // the grouped order (the larger grid) must fit a 1-D launch
  if (da_host::stage1_grid((long long)c.Hkv * c.nrb, c.units, true) > 0x7fffffffll)
    return DA_ERR_INVALID_ARG;
  return DA_OK;
}

da_host::SplitCall make_call(const void* q, int q_bf16, const void* k, const void* v,
                             const uint16_t* ks, const uint16_t* vs, const int32_t* pt,
                             int32_t pt_stride, int32_t max_pages, const int32_t* seqlens,
                             const int32_t* order, int32_t batch, int32_t qn, int32_t Hq,
                             int32_t Hkv, int32_t D, int32_t ps, int32_t num_pages,
                             int32_t kv_layout, int32_t S, const int32_t* counts,
                             const int32_t* work, int32_t work_capacity, float scale,
                             int32_t causal, float* o, float* lse, void* stream) {
  da_host::SplitCall c;
  c.q = q; c.q_bf16 = q_bf16; c.k = k; c.v = v; c.ks = ks; c.vs = vs;
  c.pt = pt; c.pt_stride = pt_stride; c.max_pages = max_pages;
  c.seqlens = seqlens; c.order = order;
  c.work = work; c.counts = counts;
  c.checks = da_host::check_words();
  c.units = work ? work_capacity : (int)((long long)S * batch);
  c.batch = batch; c.qn = qn; c.Hq = Hq; c.Hkv = Hkv; c.D = D; c.ps = ps;
  c.num_pages = num_pages; c.S = S;
  c.rows = c.nrb = c.rb_rows = 1;
  if (Hkv > 0 && Hq > 0 && Hq % Hkv == 0 && qn > 0 && qn <= DA_MAX_Q_PER_REQ && Hq / Hkv <= (1 << 20)) {
    c.rows = (Hq / Hkv) * qn;
    da_host::row_blocks(c.rows, DA_MAX_ROWS, c.nrb, c.rb_rows);
  }
  if (!da_host::kv_strides(kv_layout, Hkv, ps, c.kv)) c.kv = {0, 0};  // rejected by the check
  c.scale = scale; c.causal = causal ? 1 : 0;
  c.o = o; c.lse = lse; c.stream = (hipStream_t)stream;
  return c;
}

}  // namespace

// The stage-1 kernels, by file; each returns -1 when the shape is not covered.
// Between them they cover every call that passes check_common (D = 64 or 128,
// any number of query rows), so the entry points report a -1 as unsupported.
// (rows per block: every kernel takes the rows of one row block, see DA_MAX_ROWS)
int32_t da_split_bf16_fast(const da_host::SplitCall& c);  // split_bf16.hip: <= 5 rows
int32_t da_split_bf16_mfma(const da_host::SplitCall& c);  // split_bf16_mfma.hip: >= 6 rows
int32_t da_split_f32_mfma(const da_host::SplitCall& c);   // split_f32_mfma.hip: fp32, >= 5 rows
int32_t da_split_f32_fma(const da_host::SplitCall& c);    // split_fma.hip: fp32, <= 4 rows
int32_t da_split_int8_mfma(const da_host::SplitCall& c);  // split_int8.hip: bf16 or fp32 Q
int32_t da_split_int4_mfma(const da_host::SplitCall& c);  // split_int4.hip: bf16 or fp32 Q

extern "C" int32_t decode_attn_split(const void* q, int32_t dtype, const void* k_pool,
                                     const void* v_pool, const int32_t* page_table,
                                     int32_t page_table_stride, int32_t max_pages,
                                     const int32_t* cache_seqlens, const int32_t* batch_order,
                                     int32_t batch, int32_t q_per_req, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                                     int32_t num_pages, int32_t kv_layout, int32_t num_splits,
                                     const int32_t* split_counts, const int32_t* work_list,
                                     int32_t work_capacity, float softmax_scale, int32_t causal,
                                     float* o_partial, float* lse_partial, void* stream) {
  const da_host::SplitCall c =
      make_call(q, dtype == DA_BF16, k_pool, v_pool, nullptr, nullptr, page_table,
                page_table_stride, max_pages, cache_seqlens, batch_order, batch, q_per_req,
                num_q_heads, num_kv_heads, head_dim, page_size, num_pages, kv_layout, num_splits,
                split_counts, work_list, work_capacity, softmax_scale, causal, o_partial,
                lse_partial, stream);
  if (const int32_t st = check_common(c, kv_layout)) return st;
  if (dtype != DA_BF16 && dtype != DA_FP32) return DA_ERR_UNSUPPORTED;
  if (dtype == DA_BF16) {
    const int32_t fast = da_split_bf16_fast(c);
    if (fast >= 0) return fast;
    const int32_t mf = da_split_bf16_mfma(c);
    return mf >= 0 ? mf : DA_ERR_UNSUPPORTED;
  }
  const int32_t mf = da_split_f32_mfma(c);
  if (mf >= 0) return mf;
  const int32_t v = da_split_f32_fma(c);
  return v >= 0 ? v : DA_ERR_UNSUPPORTED;
}

extern "C" int32_t decode_attn_split_int8(
    const void* q, int32_t q_dtype, const int8_t* k_pool, const int8_t* v_pool,
    const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* page_table,
    int32_t page_table_stride, int32_t max_pages, const int32_t* cache_seqlens,
    const int32_t* batch_order, int32_t batch, int32_t q_per_req, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
    int32_t kv_layout, int32_t num_splits, const int32_t* split_counts,
    const int32_t* work_list, int32_t work_capacity, float softmax_scale, int32_t causal,
    float* o_partial, float* lse_partial, void* stream) {
  const da_host::SplitCall c =
      make_call(q, q_dtype == DA_BF16, k_pool, v_pool, k_scale, v_scale, page_table,
                page_table_stride, max_pages, cache_seqlens, batch_order, batch, q_per_req,
                num_q_heads, num_kv_heads, head_dim, page_size, num_pages, kv_layout, num_splits,
                split_counts, work_list, work_capacity, softmax_scale, causal, o_partial,
                lse_partial, stream);
  if (const int32_t st = check_common(c, kv_layout)) return st;
  if (!k_scale || !v_scale) return DA_ERR_INVALID_ARG;
  if (q_dtype != DA_BF16 && q_dtype != DA_FP32) return DA_ERR_UNSUPPORTED;
  const int32_t mf = da_split_int8_mfma(c);
  return mf >= 0 ? mf : DA_ERR_UNSUPPORTED;
}

extern "C" int32_t decode_attn_split_int4(
    const void* q, int32_t q_dtype, const uint8_t* k_pool, const uint8_t* v_pool,
    const uint16_t* k_scale_zero, const uint16_t* v_scale_zero, const int32_t* page_table,
    int32_t page_table_stride, int32_t max_pages, const int32_t* cache_seqlens,
    const int32_t* batch_order, int32_t batch, int32_t q_per_req, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t num_pages,
    int32_t kv_layout, int32_t num_splits, const int32_t* split_counts,
    const int32_t* work_list, int32_t work_capacity, float softmax_scale, int32_t causal,
    float* o_partial, float* lse_partial, void* stream) {
  const da_host::SplitCall c =
      make_call(q, q_dtype == DA_BF16, k_pool, v_pool, k_scale_zero, v_scale_zero, page_table,
                page_table_stride, max_pages, cache_seqlens, batch_order, batch, q_per_req,
                num_q_heads, num_kv_heads, head_dim, page_size, num_pages, kv_layout, num_splits,
                split_counts, work_list, work_capacity, softmax_scale, causal, o_partial,
                lse_partial, stream);
  if (const int32_t st = check_common(c, kv_layout)) return st;
  if (!k_scale_zero || !v_scale_zero) return DA_ERR_INVALID_ARG;
  if (q_dtype != DA_BF16 && q_dtype != DA_FP32) return DA_ERR_UNSUPPORTED;
  const int32_t mf = da_split_int4_mfma(c);
  return mf >= 0 ? mf : DA_ERR_UNSUPPORTED;
}
