/*
 * decode_attn.h -- C ABI of libdecode_attn.so: single-step decode attention
 * over a paged KV cache on AMD MI355X (gfx950).
 *
 * The operation.  The decode kernels tuned in LightLLM PR #1549
 * "feat(autotune): separate general and decode attention warmup" (section
 * "Covered decode kernels") are a KV-cache decode attention with a
 * num_splits tunable, a GQA flash-decode stage 1, INT4 / INT8 KV stage-1
 * kernels and a two-stage MTP attention.  Here that is:
 *
 *   metadata : one launch builds cache_seqlens, cu_seqlens_k/q and page_table
 *              (SGLang PR #29843 digest, "Implementation breakdown").
 *   split    : stage 1.  For every (request b, kv-head g, split s) the
 *              softmax-normalised partial output of the G*q query rows that
 *              share kv-head g over the split's tokens, and its log-sum-exp.
 *   merge    : stage 2.  Combines the splits of every query row by their LSE.
 *   append   : writes the step's new K/V rows into the pool at their slots,
 *              encoding them for the INT8 / INT4 caches (the step before).
 *
 * Attention is out = softmax(scale * q K^T) V per query head h, with h reading
 * kv-head h / G (G = Hq / Hkv).  With q_per_req > 1 (MTP verify) and causal
 * != 0, query i of the request sees cache tokens t < L - (q_per_req - 1 - i).
 * The LSE values crossing the ABI are natural logarithms.
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless stated "host".  All memory is
 *     owned and allocated by the caller (the one exception is the scratch
 *     array of decode_attn_decode_static, which the library holds per GPU);
 *     the library never allocates, frees or synchronises, and never reads
 *     device data on the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Work is enqueued asynchronously on it; every call can be recorded in
 *     a HIP graph.
 *   - Arguments are checked on the host first.  On a non-zero return
 *     nothing has been enqueued, except DA_ERR_LAUNCH (launch failed).
 *   - Device data is the caller's contract and is not validated (that would
 *     need a sync).  Kernels still never read outside the buffers whose
 *     sizes the arguments give: out-of-range page ids read page 0, lengths
 *     are clamped to [0, max_pages * page_size], negative ids act as 0.
 *     Results for such rows are unspecified.
 *   - Alignment (checked, DA_ERR_INVALID_ARG): the stage-1 calls need q,
 *     the K/V pools and o_partial 16-byte aligned, the scale arrays 4-byte
 *     aligned (16-byte vector accesses); the merge needs its arrays 4-byte
 *     aligned (bf16 outputs are written in pairs).  Allocations from hipMalloc or a
 *     framework allocator are 256-byte aligned; a view into one keeps the
 *     alignment when its offset is a multiple of 16 bytes.
 *
 * Layouts (row-major, contiguous):
 *   q            [B, q_per_req, Hq, D]
 *   k/v pools    pages of page_size token slots.  A "row" is the entry of one
 *                (slot, kv-head): D elements (bf16 / fp32 / int8), or D/2
 *                bytes of 4-bit codes (element 2j in the low nibble of byte
 *                j); scale arrays have the same layout with their own rows.
 *                kv_layout DA_KV_NHD: [num_pages, page_size, Hkv, row]
 *                kv_layout DA_KV_HND: [num_pages, Hkv, page_size, row]
 *                (HND keeps a kv-head's rows of a page contiguous, which
 *                makes the stage-1 reads of short rows -- quantised codes,
 *                their scales -- long contiguous runs.  With NHD and Hkv a
 *                multiple of 4, the INT8 / INT4 stage-1 kernels, and the dense
 *                (bf16, fp32) ones at D = 64, give each of a
 *                workgroup's four waves its own kv-head, so the lines that
 *                neighbouring kv-heads share are read together; such calls
 *                want about four times the num_splits of one kv-head per
 *                workgroup.)
 *   page_table   [B, page_table_stride], first max_pages entries of a row used
 *   o_partial    [B, q_per_req, Hq, num_splits, D] fp32
 *   lse_partial  [B, q_per_req, Hq, num_splits]    fp32
 *   out          [B, q_per_req, Hq, D]  bf16 (RNE) or fp32
 *   lse_out      [B, q_per_req, Hq]     fp32
 *
 * Split partition: n = ceil(L / page_size) pages, c = ceil(n / num_splits)
 * pages per split; split s covers pages [s*c, min((s+1)*c, n)), clipped to
 * L tokens.  Splits with no visible token write (0, -inf); every slot of
 * o_partial / lse_partial is written, so they need no clearing.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DA_OK 0
#define DA_ERR_INVALID_ARG 1  /* null pointer, non-positive size, Hq % Hkv, range */
#define DA_ERR_UNSUPPORTED 2  /* a shape / dtype no kernel is built for          */
#define DA_ERR_LAUNCH 3       /* hipGetLastError() after the launch               */
#define DA_ERR_TOO_LARGE 4    /* partials beyond DA_STATIC_SCRATCH_BYTES (decode_attn_decode_static) */

/* element types */
#define DA_FP32 0
#define DA_BF16 1

/* cache formats of decode_attn_append_kv */
#define DA_CACHE_DENSE 0 /* rows stored as given (pool dtype = the new K/V's dtype) */
#define DA_CACHE_INT8 1  /* int8 codes + one fp16 scale per row                     */
#define DA_CACHE_INT4 2  /* 4-bit codes + fp16 (scale, zero) per 32-group           */

/* KV pool layouts within a page (see "Layouts" above) */
#define DA_KV_NHD 0 /* [num_pages, page_size, Hkv, row] */
#define DA_KV_HND 1 /* [num_pages, Hkv, page_size, row] */

/* cu_seqlens_q modes (SGLang PR #29843 digest, "Implementation breakdown":
   preset / cumsum / strided) */
#define DA_Q_STRIDED 0 /* cu_q[b] = b * q_stride, b = 0..B                        */
#define DA_Q_CUMSUM 1  /* cu_q = exclusive prefix of max(q_in[b], 0), q_in [B]     */
#define DA_Q_PRESET 2  /* cu_q = copy of q_in [B+1]                                */

/* contract checks of the checked build (bits of decode_attn_checks' flags) */
#define DA_CHECK_PAGE_ID 0x01u  /* a page id read by stage 1 outside [0, num_pages)        */
#define DA_CHECK_SEQLEN 0x02u   /* cache_seqlens outside [0, max_pages * page_size] (stage 1) */
#define DA_CHECK_ORDER 0x04u    /* a batch_order entry outside [0, batch)                    */
#define DA_CHECK_WORK 0x08u     /* a work-list entry neither -1 nor a valid (request, split)  */
#define DA_CHECK_COUNTS 0x10u   /* a split_counts entry outside [1, num_splits]               */
#define DA_CHECK_REQ_ROW 0x20u  /* metadata: req_pool_indices[b] >= req_to_token_rows        */
#define DA_CHECK_TOO_LONG 0x40u /* metadata: seq_lens[b] needs more than max_pages pages or
                                   exceeds req_to_token_cols                                 */

/* limits of the built kernels */
#define DA_MAX_SPLITS 256
#define DA_MAX_Q_PER_REQ 16
/* bytes of the per-device scratch array of decode_attn_decode_static */
#define DA_STATIC_SCRATCH_BYTES (64u << 20)
/* Query rows one stage-1 workgroup holds.  A kv-head serves R = G * q_per_req
 * rows; with R > DA_MAX_ROWS they are processed in ceil(R / DA_MAX_ROWS)
 * row blocks of ceil(R / blocks) rows, one workgroup each, and every block
 * reads the kv-head's pages (the blocks of a kv-head run side by side on one
 * XCD, so the later reads are mostly served by its L2). */
#define DA_MAX_ROWS 16

/*
 * Metadata prelude, one launch (SGLang PR #29843 digest, sections
 * "Features and motivation" and "Implementation breakdown"; the page-table
 * tail is zero-padded as its tests describe).
 *
 *   seq_lens          [batch] int32      KV length of each request (new tokens included)
 *   req_pool_indices  [batch] int64      row of req_to_token for each request
 *   req_to_token      [rows, stride] int32 token slot of every logical token;
 *                      slot = page * page_size + offset
 *   outputs: cache_seqlens [batch], cu_seqlens_k [batch+1], cu_seqlens_q [batch+1],
 *            page_table [batch, max_pages] (row stride max_pages), all int32.
 *
 *   cache_seqlens[b]  = max(seq_lens[b], 0)
 *   cu_seqlens_k      = exclusive prefix sum of cache_seqlens (sum must fit int32)
 *   page_table[b][j]  = req_to_token[rpi[b]][j * page_size] / page_size for
 *                       j < ceil(cache_seqlens[b] / page_size), else 0.  A negative
 *                       or >= req_to_token_rows rpi, a column >= req_to_token_cols,
 *                       or a negative slot gives 0 (-1 sentinel guard).
 *   q_in: device array, required for CUMSUM ([batch]) and PRESET ([batch+1]);
 *   ignored (may be NULL) for STRIDED.
 *   batch_order (nullable) [batch] int32: request indices by descending
 *   cache_seqlens, ties by ascending index.  Passed to the split calls, it
 *   makes the longest requests' splits start first (scheduling only: results
 *   do not depend on it).
 */
int32_t decode_attn_metadata(const int32_t* seq_lens, const int64_t* req_pool_indices,
                             const int32_t* req_to_token, int64_t req_to_token_rows,
                             int64_t req_to_token_cols, int64_t req_to_token_stride,
                             int32_t batch, int32_t page_size, int32_t max_pages,
                             int32_t q_mode, const int32_t* q_in, int32_t q_stride,
                             int32_t* cache_seqlens, int32_t* cu_seqlens_k,
                             int32_t* cu_seqlens_q, int32_t* page_table, int32_t* batch_order,
                             void* stream);

/*
 * decode_attn_metadata plus two options computed in the same launch.
 *
 * SWA translation (SGLang PR #29843 digest, "Implementation breakdown": the
 * fused kernel translates slots through the full-to-SWA mapping the backend
 * prepares for sliding-window layers, whose K/V live in a second pool):
 *   full_to_swa      [full_to_swa_len] int64: SWA-pool slot of every
 *                    full-pool slot, negative for a token not resident there
 *   swa_page_table   [batch, max_pages] int32 out:
 *                    full_to_swa[slot] / page_size, slot being the first
 *                    full-pool slot of logical page j (as for page_table).
 *                    0 where page_table's guards give 0, where slot >=
 *                    full_to_swa_len, where the mapped slot is negative, and
 *                    in the tail.
 *   Both NULL: no SWA table.
 *
 * Per-request split counts (LightLLM PR #1549, "Covered decode kernels":
 * configurations are tuned over bucketed KV-length keys while each run
 * picks one from the real request length):
 *   split_table      HOST [n_buckets] int32 (1..DA_MAX_SPLITS), n_buckets <= 16;
 *                    copied into the launch, so a captured graph keeps it
 *   split_counts     [batch] int32 out: S_b = max(1, min(split_table[k],
 *                    ceil(L_b / page_size), max_splits)) with bucket
 *                    k = clamp(ceil(L_b / bucket_tokens), 1, n_buckets) - 1
 *   work_list        [work_capacity] int32 out: one entry b * 256 + s per
 *                    (request, split s < S_b), requests by descending
 *                    cache_seqlens (ties by index), splits ascending; -1 after
 *                    the last entry.  work_capacity >= batch * min(max(split_table),
 *                    max_splits) (checked), batch < 2^23.
 *   split_table, split_counts and work_list are all NULL (no schedule) or
 *   all given.  Pass work_list, split_counts and num_splits = max_splits to
 *   the split calls and split_counts to decode_attn_merge.
 */
int32_t decode_attn_metadata_ex(const int32_t* seq_lens, const int64_t* req_pool_indices,
                                const int32_t* req_to_token, int64_t req_to_token_rows,
                                int64_t req_to_token_cols, int64_t req_to_token_stride,
                                int32_t batch, int32_t page_size, int32_t max_pages,
                                int32_t q_mode, const int32_t* q_in, int32_t q_stride,
                                int32_t* cache_seqlens, int32_t* cu_seqlens_k,
                                int32_t* cu_seqlens_q, int32_t* page_table,
                                int32_t* batch_order, const int64_t* full_to_swa,
                                int64_t full_to_swa_len, int32_t* swa_page_table,
                                const int32_t* split_table, int32_t n_buckets,
                                int32_t bucket_tokens, int32_t max_splits, int32_t* split_counts,
                                int32_t* work_list, int32_t work_capacity, void* stream);

/*
 * Stage-1 numerics (all paths accumulate in fp32 and keep one running max and
 * sum per query row; scores are formed in log2 units and exponentials are
 * exp2):
 *   - fp32 cache and Q: fp32 throughout.
 *   - bf16 cache, up to 5 query rows per kv-head: fp32 products of the bf16
 *     values, weights p in fp32.
 *   - bf16 cache, 6 or more rows: matrix-core products of the bf16 values
 *     (exact in fp32); p enters the P.V product as two bf16 terms, hi + lo,
 *     within 2^-16 |p|.
 *   - INT8 / INT4 caches: scores exact up to fp32 rounding (codes and Q enter
 *     the matrix cores exactly; a bf16 Q after a per-row power-of-two scaling,
 *     an fp32 Q as two fp16 terms of 22 significant bits together); the P.V
 *     product takes p and the dequantised V in fp16, one rounding each (unit
 *     roundoff u = 2^-11).
 * Partial outputs are the normalised fp32 rows O_s and their natural-log LSE.
 *
 * Range of the quantised caches: every finite fp16 scale and zero point.
 *   - INT8: V enters as fp16(b s); per partial row |dO| <= u * 2 max|v| +
 *     2^-25 (max over the split's tokens; the 2^-25 in fp16's subnormal
 *     range).  When a split's |b s| passes 65504, the kernel detects the
 *     overflow and computes that split again with fp16((b / 2^7) * s), below
 *     65504 for any scale, where the floor is 2^-18; other splits pay nothing.
 *   - INT4: V enters as two products, fp16(n s) less fp16(z s) (one rounding
 *     each, summed apart in fp32), |dO| <= u * (max|v| + max|n s| + max|z s|)
 *     + 2^-24.  When a split's fp16 operands overflow (|s| of 64 or more, or
 *     |z s| near 65504 or beyond), the kernel detects it and computes that
 *     split again with s * 2^-e (e the smallest power that brings every
 *     |s| max(1024, 15 + |z|) of the split below 2^15), adding at most
 *     2^-22 max |s| (15 + |z|); other splits pay nothing.
 *   - Scores: the fp32 terms of a score add up to M = scale * sum_d |q_d| u_d
 *     (u_d = |k_d| for dense caches, |s| (|b| + 128) for INT8, |s| (n_d + |z|)
 *     for INT4) and carry a few units of 2^-24 M; a score error E moves the
 *     LSE by at most E and a normalised output by at most 2 E max|v|.  With
 *     unit-scale data (|q|, |v| around 1) this is far inside the outputs' own
 *     rounding; with peaked inputs (M in the thousands) it reaches ~1e-4 in
 *     the LSE.  Inputs whose scores overflow fp32 (|scale q.k| > 3e38) are
 *     out of range.
 */

/*
 * Stage 1 over a dense bf16 or fp32 cache (GQA flash decode "stage 1" and
 * the num_splits KV-cache decode of LightLLM PR #1549, "Covered decode
 * kernels").  q and the pools share `dtype` (DA_BF16 or DA_FP32).
 *
 *   head_dim in {64, 128}; page_size in {16, 32, 64, 128, 256};
 *   page_size * num_kv_heads * head_dim * 4 < 2^31 (one page of any cache
 *   format below 2 GiB: the kernels address inside a page with 32-bit
 *   offsets; else DA_ERR_UNSUPPORTED; the same for the INT8 / INT4 calls);
 *   kv_layout DA_KV_NHD or DA_KV_HND (pool layout, see "Layouts");
 *   num_q_heads % num_kv_heads == 0 (any group G = Hq / Hkv; G * q_per_req
 *   rows beyond DA_MAX_ROWS run in row blocks, see DA_MAX_ROWS);
 *   1 <= num_splits <= DA_MAX_SPLITS; 1 <= q_per_req <= DA_MAX_Q_PER_REQ;
 *   units * num_kv_heads * row blocks < 2^31 workgroups, units being
 *   batch * num_splits, or work_capacity with a work list (else
 *   DA_ERR_INVALID_ARG).
 *   page_table_stride >= max_pages >= 1.  cache_seqlens is the [batch] int32
 *   array from decode_attn_metadata (or any caller array of KV lengths).
 *   batch_order (nullable): a permutation of [0, batch) giving the order in
 *   which requests are scheduled (decode_attn_metadata's batch_order); NULL
 *   means 0..batch-1.  An entry outside [0, batch) is replaced by the grid
 *   index; a non-permutation leaves some requests unprocessed (unspecified
 *   results, never an out-of-bounds access).
 *   Per-request split counts (work_list != NULL; batch_order is then unused):
 *   work_list [work_capacity] and split_counts [batch] as written by
 *   decode_attn_metadata_ex.  Request b is cut into split_counts[b] splits
 *   (clamped to [1, num_splits]) by the partition rule above, and num_splits
 *   is only the number of split slots per query row in o_partial /
 *   lse_partial: slots from split_counts[b] on are not written (pass the
 *   same split_counts to decode_attn_merge).  Each list entry b * 256 + s
 *   is one (request, split); entries that are -1, or name no valid request
 *   or split, are skipped.  1 <= work_capacity <= batch * num_splits.
 *   With work_list == NULL, split_counts and work_capacity are ignored and
 *   every request has num_splits splits.
 */
int32_t decode_attn_split(const void* q, int32_t dtype, const void* k_pool, const void* v_pool,
                          const int32_t* page_table, int32_t page_table_stride, int32_t max_pages,
                          const int32_t* cache_seqlens, const int32_t* batch_order,
                          int32_t batch, int32_t q_per_req,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t page_size, int32_t num_pages, int32_t kv_layout,
                          int32_t num_splits, const int32_t* split_counts,
                          const int32_t* work_list, int32_t work_capacity, float softmax_scale,
                          int32_t causal, float* o_partial, float* lse_partial, void* stream);

/*
 * Stage 1 over an INT8 cache (LightLLM PR #1549, "Covered decode kernels":
 * INT8 KV flash decode stage 1).  K = k_pool * k_scale, V = v_pool * v_scale
 * with one fp16 scale per (page, slot, kv-head):
 *   k_pool, v_pool    [num_pages, page_size, Hkv, D] int8
 *   k_scale, v_scale  [num_pages, page_size, Hkv] fp16 (raw bits)
 * q_dtype is DA_BF16 or DA_FP32.  Other arguments as decode_attn_split.
 */
int32_t decode_attn_split_int8(const void* q, int32_t q_dtype, const int8_t* k_pool,
                               const int8_t* v_pool, const uint16_t* k_scale,
                               const uint16_t* v_scale, const int32_t* page_table,
                               int32_t page_table_stride, int32_t max_pages,
                               const int32_t* cache_seqlens, const int32_t* batch_order,
                               int32_t batch, int32_t q_per_req,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t num_pages, int32_t kv_layout,
                               int32_t num_splits, const int32_t* split_counts,
                               const int32_t* work_list, int32_t work_capacity,
                               float softmax_scale, int32_t causal, float* o_partial,
                               float* lse_partial, void* stream);

/*
 * Stage 1 over an INT4 cache (LightLLM PR #1549, "Covered decode kernels":
 * INT4 KV flash decode stage 1; with q_per_req > 1 and causal it is the MTP
 * verify decode of the same page).  Per group of 32 elements along D:
 * x = (nibble - zero) * scale.
 *   k_pool, v_pool            [num_pages, page_size, Hkv, D/2] uint8
 *   k_scale_zero, v_scale_zero [num_pages, page_size, Hkv, D/32, 2] fp16 bits,
 *                              (scale, zero) pairs
 * Other arguments as decode_attn_split_int8.
 */
int32_t decode_attn_split_int4(const void* q, int32_t q_dtype, const uint8_t* k_pool,
                               const uint8_t* v_pool, const uint16_t* k_scale_zero,
                               const uint16_t* v_scale_zero, const int32_t* page_table,
                               int32_t page_table_stride, int32_t max_pages,
                               const int32_t* cache_seqlens, const int32_t* batch_order,
                               int32_t batch, int32_t q_per_req,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t num_pages, int32_t kv_layout,
                               int32_t num_splits, const int32_t* split_counts,
                               const int32_t* work_list, int32_t work_capacity,
                               float softmax_scale, int32_t causal, float* o_partial,
                               float* lse_partial, void* stream);

/*
 * KV append with quantise-on-write: writes the new tokens' K and V rows to
 * their token slots before attention runs (SGLang PR #29843 digest, test
 * listing: one out_cache_loc slot per new token; LightLLM PR #1549, "Covered
 * decode kernels": INT8 / INT4 KV caches).
 *   k_new, v_new   [num_tokens, Hkv, head_dim], new_dtype DA_BF16 or DA_FP32
 *   out_cache_loc  [num_tokens] int64 token slots; slot = page * page_size +
 *                  offset.  A negative slot, or one >= num_pages * page_size,
 *                  writes nothing (the -1 sentinel of padded batches).  Slots
 *                  are the caller's to keep distinct; with repeats the result
 *                  is unspecified.
 *   cache_format   DA_CACHE_DENSE: pools hold new_dtype, rows copied bit for bit;
 *                  DA_CACHE_INT8: per row s = fp16(max|x| / 127) (1 if that is
 *                    0), code = clamp(rne(x / s), -127, 127), scale -> k/v_scale;
 *                  DA_CACHE_INT4: per 32-group s = fp16((max - min) / 15) (1 if
 *                    0), z = fp16(clamp(rne(-min / s), 0, 15)) (+0 for 0),
 *                    nibble = clamp(rne(x / s) + z, 0, 15), (s, z) -> k/v_scale.
 *                  All decisions in IEEE fp32 (the codes are reproducible).
 *   pools / scales in the layouts of the split calls (kv_layout NHD or HND);
 *   k_scale, v_scale may be NULL for DA_CACHE_DENSE.
 *   head_dim in {64, 128}.  num_tokens == 0 enqueues nothing.
 */
int32_t decode_attn_append_kv(const void* k_new, const void* v_new, int32_t new_dtype,
                              const int64_t* out_cache_loc, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t cache_format,
                              void* k_pool, void* v_pool, uint16_t* k_scale, uint16_t* v_scale,
                              int32_t page_size, int32_t num_pages, int32_t kv_layout,
                              void* stream);

/*
 * Stage 2: LSE merge (LightLLM PR #1549, "Covered decode kernels": the
 * stage 2 of the two-stage attention; "Validation": stage-2 inputs are
 * reused).  For every query row: m = max_s lse_s, w_s = exp(lse_s - m),
 * out = sum_s w_s O_s / sum_s w_s, lse = m + ln(sum_s w_s); a row whose
 * splits are all empty gives out 0, lse -inf.
 *   out_dtype DA_BF16 (round to nearest even) or DA_FP32; lse_out may be NULL.
 *   split_counts (nullable) [batch] int32: the rows of request b combine only
 *   their first split_counts[b] slots (clamped to [1, num_splits]); the
 *   other slots are not read.  NULL: all num_splits slots.
 */
int32_t decode_attn_merge(const float* o_partial, const float* lse_partial, int32_t batch,
                          int32_t q_per_req, int32_t num_q_heads, int32_t head_dim,
                          int32_t num_splits, const int32_t* split_counts, void* out,
                          int32_t out_dtype, float* lse_out, void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it: stage 1 and the merge in one call, with the split partials in a scratch
 * array the library keeps on each GPU instead of caller buffers.  The result
 * is that of decode_attn_split / decode_attn_split_int8 / decode_attn_split_int4
 * (by cache_format: DA_CACHE_DENSE, _INT8, _INT4; k_scale / v_scale are the
 * scales or (scale, zero) pairs of the quantised formats, NULL for dense)
 * followed by decode_attn_merge into out / lse_out, with the same kernels;
 * every argument means what it means there.  With a work list, the merge
 * takes split_counts.
 *   Scratch: DA_STATIC_SCRATCH_BYTES (64 MiB) per GPU, allocated when the
 *   library is loaded on that GPU and held until the process ends.  The
 *   partials need 4 * B * q_per_req * Hq * num_splits * (D + 1) bytes (the
 *   output part rounded up to 256); a call that needs more returns
 *   DA_ERR_TOO_LARGE and enqueues nothing (e.g. B = 64, Hq = 40, D = 128:
 *   up to 48 splits; B = 64 with 4 MTP tokens and Hq = 32: up to 15).
 *   Calls on one GPU share its array, which keeps the last call's partials:
 *   two calls whose work overlaps on one GPU (different streams, threads or
 *   a graph replayed beside an eager call) race.  Nothing in it needs
 *   clearing (stage 1 writes every slot the merge reads).
 *   No allocation, free or synchronisation; capturable in a HIP graph.
 */
int32_t decode_attn_decode_static(const void* q, int32_t q_dtype, int32_t cache_format,
                                  const void* k_pool, const void* v_pool,
                                  const uint16_t* k_scale, const uint16_t* v_scale,
                                  const int32_t* page_table, int32_t page_table_stride,
                                  int32_t max_pages, const int32_t* cache_seqlens,
                                  const int32_t* batch_order, int32_t batch, int32_t q_per_req,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t page_size, int32_t num_pages, int32_t kv_layout,
                                  int32_t num_splits, const int32_t* split_counts,
                                  const int32_t* work_list, int32_t work_capacity,
                                  float softmax_scale, int32_t causal, void* out,
                                  int32_t out_dtype, float* lse_out, void* stream);

/*
 * Host-only: split count for a launch (LightLLM PR #1549: num_splits is the
 * tuned config of the KV-cache decode kernel; run keys are KV-length
 * buckets while the real length selects the config at run time).
 *   table      host [n_batch_keys, n_buckets] int32 split counts
 *   batch_keys host [n_batch_keys] int32, ascending
 *   bucket = clamp(ceil(kv_len / bucket_tokens), 1, n_buckets); the batch key
 *   is the nearest one to `batch` (ties -> the smaller key).
 * Returns the split count (>= 1), or -DA_ERR_INVALID_ARG.
 */
int32_t decode_attn_pick_splits(const int32_t* table, const int32_t* batch_keys,
                                int32_t n_batch_keys, int32_t n_buckets, int32_t bucket_tokens,
                                int32_t batch, int32_t kv_len);

/*
 * Test hook: dense copy of every request's tokens from a paged pool.
 * out [total_tokens, Hkv, row_bytes]: entry (cu_seqlens_k[b] + t, g) = the
 * pool row of (page page_table[b][t / page_size], slot t % page_size,
 * kv-head g) for t < cache_seqlens[b], in either kv_layout; row_bytes is
 * even (e.g. D*2 for bf16 K, 2 for int8 scales, 16 for int4 scale/zero).
 */
int32_t decode_attn_gather_kv(const void* pool, int64_t row_bytes, int32_t num_kv_heads,
                              int32_t kv_layout, int32_t page_size, int32_t num_pages,
                              const int32_t* page_table, int32_t page_table_stride,
                              int32_t max_pages, const int32_t* cache_seqlens,
                              const int32_t* cu_seqlens_k, int32_t batch, void* out,
                              void* stream);

/*
 * Contract checks (the conventions above leave device data unchecked in the
 * normal library).  A build compiled with -DDA_CHECKED
 * (libdecode_attn_checked.so, `python -m decode_attention_paged_gqa_amd.build
 * --checked`) makes the kernels record every violation of the device-data
 * contract they meet -- the DA_CHECK_* conditions -- in check words the
 * library keeps per device, while still clamping the data exactly as the
 * normal build does (identical results).  Each workgroup that meets a bad
 * value counts it, so `count` is a number of observations, not of bad
 * entries.
 *   flags, count  HOST out (nullable): OR of DA_CHECK_* bits, observations
 *   reset         != 0: clear the words after reading
 * Synchronises the current device (hipDeviceSynchronize) before reading.
 * Returns DA_ERR_UNSUPPORTED in the normal build, DA_ERR_LAUNCH when a HIP
 * call fails.
 */
int32_t decode_attn_checks(uint32_t* flags, uint64_t* count, int32_t reset);

/* Human-readable text for a status code (static storage). */
const char* decode_attn_strerror(int32_t status);

/* ABI version (major * 100 + minor). */
int32_t decode_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
