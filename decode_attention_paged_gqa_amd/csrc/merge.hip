// Stage 2: log-sum-exp merge of the split partials (LightLLM PR #1549,
// "Covered decode kernels": the second stage of the two-stage decode
// attention).  For one query row with split results (O_s, lse_s):
//   m = max_s lse_s, w_s = exp(lse_s - m),
//   out = sum_s w_s O_s / sum_s w_s,  lse = m + ln(sum_s w_s).
// A row whose splits are all empty (every lse_s = -inf) yields 0 / -inf.
//
// One wave per query row; the reduction over splits stays in registers:
// every lane owns D/64 output elements and walks all splits itself, the
// split weights being wave-uniform.  Split rows are loaded kPrefetch at a
// time ahead of their use (the first group before the split count is known).  With per-request split counts, the rows
// of request b combine only their first counts[b] split slots (clamped to
// [1, S]); the other slots are never read.
#include "common.h"

namespace {

constexpr int kWaves = 4;
constexpr int kPrefetch = 16;  // split rows loaded before the weights are known
static_assert(DA_MAX_SPLITS == 256, "four lse registers per lane");

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kWaves) void merge_kernel(const float* __restrict__ op,
                                                           const float* __restrict__ lp,
                                                           int rows, int S,
                                                           const int32_t* __restrict__ counts,
                                                           int rows_per_req, void* __restrict__ out,
                                                           float* __restrict__ lse_out,
                                                           unsigned long long* checks) {
  constexpr int E = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int slots = S;  // split slots per row in the buffers
  const float* l = lp + (long long)row * slots;
  const float* o = op + (long long)row * slots * D + lane * E;
  // Every load below stays inside the row's slots and is issued before the
  // row's split count is known: the first kPrefetch split rows, and the
  // lse of slot lane + 64 k in lane `lane`.
  float pre[kPrefetch][E];
#pragma unroll
  for (int s = 0; s < kPrefetch; ++s)
#pragma unroll
    for (int e = 0; e < E; ++e) pre[s][e] = s < slots ? o[(long long)s * D + e] : 0.f;
  float lv[DA_MAX_SPLITS / 64];
#pragma unroll
  for (int k = 0; k < DA_MAX_SPLITS / 64; ++k)
    lv[k] = 64 * k + lane < slots ? l[64 * k + lane] : da::kNegInf;
  if (counts) {
    const int cnt = counts[row / rows_per_req];
    da::note(checks, lane != 0 || (cnt >= 1 && cnt <= slots), DA_CHECK_COUNTS);
    S = min(max(cnt, 1), slots);
  }
  float m = da::kNegInf;
#pragma unroll
  for (int k = 0; k < DA_MAX_SPLITS / 64; ++k)
    if (64 * k + lane < S) m = fmaxf(m, lv[k]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m != da::kNegInf) {
    const float ml = m * da::kLog2e;
    // exp(lse_s - m); 0 for an empty split (lse -inf), whose row holds zeros.
    // lse_s is read from the lane that loaded it.
#pragma unroll
    for (int s = 0; s < kPrefetch; ++s) {
      if (s < S) {
        const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv[0]), s));
        const float w = da::fast_exp2(fmaf(ls, da::kLog2e, -ml));
        wsum += w;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(w, pre[s][e], acc[e]);
      }
    }
    // the rest in groups of kPrefetch: a group's rows are all loaded before
    // any is used, so a row costs a fraction of a memory round trip
    for (int s0 = kPrefetch; s0 < S; s0 += kPrefetch) {
      float buf[kPrefetch][E];
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e)
          buf[u][e] = s0 + u < S ? o[(long long)(s0 + u) * D + e] : 0.f;
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        const int s = s0 + u;
        if (s < S) {
          const int k = s >> 6;
          const float lk = k == 0 ? lv[0] : k == 1 ? lv[1] : k == 2 ? lv[2] : lv[3];
          const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lk), s & 63));
          const float w = da::fast_exp2(fmaf(ls, da::kLog2e, -ml));
          wsum += w;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = fmaf(w, buf[u][e], acc[e]);
        }
      }
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= inv;
  }
  if (OUT_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(out) + (long long)row * D + lane * E;
    if constexpr (E == 2) {
      *reinterpret_cast<uint32_t*>(dst) =
          (uint32_t)da::float_to_bf16_rne(acc[0]) | ((uint32_t)da::float_to_bf16_rne(acc[1]) << 16);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = da::float_to_bf16_rne(acc[e]);
    }
  } else {
    float* dst = reinterpret_cast<float*>(out) + (long long)row * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = acc[e];
  }
  if (lse_out && lane == 0) lse_out[row] = (m == da::kNegInf) ? m : m + logf(wsum);
}

template <int D, bool B16>
int32_t launch(const float* op, const float* lp, int rows, int S, const int32_t* counts,
               int rows_per_req, void* out, float* lse_out, hipStream_t st) {
  const int blocks = (rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((merge_kernel<D, B16>), dim3(blocks), dim3(64 * kWaves), 0, st, op, lp, rows,
                     S, counts, rows_per_req, out, lse_out, da_host::check_words());
  return da_host::launch_status();
}

}  // namespace

extern "C" int32_t decode_attn_merge(const float* o_partial, const float* lse_partial,
                                     int32_t batch, int32_t q_per_req, int32_t num_q_heads,
                                     int32_t head_dim, int32_t num_splits,
                                     const int32_t* split_counts, void* out,
                                     int32_t out_dtype, float* lse_out, void* stream) {
  if (!o_partial || !lse_partial || !out) return DA_ERR_INVALID_ARG;
  // bf16 outputs leave as pairs (4-byte stores); see "Alignment" in the header
  if (!da_host::aligned(out, 4) || !da_host::aligned(o_partial, 4) ||
      !da_host::aligned(lse_partial, 4) || !da_host::aligned(lse_out, 4))
    return DA_ERR_INVALID_ARG;
  if (batch <= 0 || q_per_req <= 0 || num_q_heads <= 0 || num_splits <= 0 ||
      num_splits > DA_MAX_SPLITS || q_per_req > DA_MAX_Q_PER_REQ)
    return DA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return DA_ERR_UNSUPPORTED;
  if (out_dtype != DA_BF16 && out_dtype != DA_FP32) return DA_ERR_UNSUPPORTED;
  const long long rows_ll = (long long)batch * q_per_req * num_q_heads;
  if (rows_ll > (1ll << 30)) return DA_ERR_INVALID_ARG;
  const int rows = (int)rows_ll;
  const int rpr = q_per_req * num_q_heads;
  hipStream_t st = (hipStream_t)stream;
  const bool b16 = out_dtype == DA_BF16;
  const int32_t* cn = split_counts;
  if (head_dim == 128)
    return b16 ? launch<128, true>(o_partial, lse_partial, rows, num_splits, cn, rpr, out, lse_out, st)
               : launch<128, false>(o_partial, lse_partial, rows, num_splits, cn, rpr, out, lse_out, st);
  return b16 ? launch<64, true>(o_partial, lse_partial, rows, num_splits, cn, rpr, out, lse_out, st)
             : launch<64, false>(o_partial, lse_partial, rows, num_splits, cn, rpr, out, lse_out, st);
}
