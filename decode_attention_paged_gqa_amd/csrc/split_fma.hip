// Stage 1 of split-KV decode attention over an fp32 cache with fp32 Q and up
// to 4 query rows per kv-head (more go to split_f32_mfma.hip), vector-ALU path (GQA flash decode "stage 1" and the num_splits KV-cache
// decode of LightLLM PR #1549, section "Covered decode kernels").  The
// stage-1 entry points that validate a call and pick its kernel are in
// stage1.cpp.
//
// One workgroup (4 waves) per (kv-head g, split s, request b).  The G*q
// query rows that read kv-head g are all served by that workgroup, so each
// K/V byte of the split is fetched from HBM exactly once.
//
// Lane layout inside a wave: 16 lanes per token row, 4 tokens per step,
// 4 steps per 16-token tile.  Lane (tl, c) owns elements [c*E, c*E + E) of
// its token's row (E = D/16), loaded as one contiguous vector, so a wave's
// load of 4 rows touches whole 64-to-512-byte row segments (coalesced).
// Tiles of the split are dealt round-robin to the 4 waves; each wave keeps
// its own online-softmax state (running max m, sum l, output acc) and the
// four states are combined through LDS at the end.
//
// Scores are kept in log2 units: q is pre-multiplied by softmax_scale*log2(e)
// and exponentials are exp2; the stored LSE is converted back to natural log.
#include "common.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct SplitArgs {
  const float* q;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* pt;
  const int32_t* seqlens;
  da::Stage1Sched sched;  // (request, split) of every workgroup
  float* o;
  float* lse;
  int pt_stride, max_pages;
  int qn, Hq, Hkv, G, R;
  int page_size, log2_ps, num_pages;
  int slot_stride, head_stride;  // rows (see da_host::KvStrides)
  float scale_log2;
  int causal;
};

// A lane's piece of a K or V row: D/16 fp32 values, read once per launch
// with non-temporal loads (see da::kStreamPolicy).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int E>
__device__ __forceinline__ void load_row(const uint8_t* p, float (&f)[E]) {
  static_assert(E % 4 == 0, "whole 16-byte pieces");
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i);
    f[4 * i] = __uint_as_float(a[0]);
    f[4 * i + 1] = __uint_as_float(a[1]);
    f[4 * i + 2] = __uint_as_float(a[2]);
    f[4 * i + 3] = __uint_as_float(a[3]);
  }
}

template <int D, int RT>
__global__ __launch_bounds__(kThreads) void split_fma_kernel(const SplitArgs a) {
  constexpr int E = D / 16;       // elements per lane
  constexpr int kRowBytes = 4 * D;

  __shared__ float sm_m[kWaves][RT];
  __shared__ float sm_l[kWaves][RT];
  __shared__ float sm_acc[kWaves][RT][D];

  da::Stage1Item it;
  if (!da::stage1_item<false>(a.sched, a.Hkv, it)) return;
  const int g = it.g, s = it.s, b = it.b, r0 = it.r0, nr = it.nr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = lane >> 4, c = lane & 15;

  const int ps = a.page_size;
  const int L = min(max(a.seqlens[b], 0), a.max_pages * ps);
  da::note(a.sched.checks,
           threadIdx.x != 0 || (a.seqlens[b] >= 0 && a.seqlens[b] <= a.max_pages * ps),
           DA_CHECK_SEQLEN);
  const int n = (L + ps - 1) >> a.log2_ps;
  const int cpg = (n + it.S - 1) / it.S;
  const int p0 = min(s * cpg, n), p1 = min((s + 1) * cpg, n);
  const int t0 = p0 * ps, t1 = min(p1 * ps, L);

  // ---- query rows r0 + r = i*G + hh (query token i, head g*G + hh), pre-scaled
  float qf[RT][E];
  int tend[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    if (r < nr) {
      const int i = (r0 + r) / a.G, h = g * a.G + ((r0 + r) % a.G);
      const float* qp = a.q + (((long long)b * a.qn + i) * a.Hq + h) * D + c * E;
#pragma unroll
      for (int e = 0; e < E; ++e) qf[r][e] = qp[e] * a.scale_log2;
      tend[r] = a.causal ? L - (a.qn - 1 - i) : L;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) qf[r][e] = 0.f;
      tend[r] = 0;
    }
  }

  float m[RT], l[RT], acc[RT][E];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m[r] = da::kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[r][e] = 0.f;
  }

  const int ntiles = t1 > t0 ? (t1 - t0 + 15) >> 4 : 0;

  for (int tile = wave; tile < ntiles; tile += kWaves) {
    const int tb = t0 + (tile << 4);
    int pid = a.pt[(long long)b * a.pt_stride + (tb >> a.log2_ps)];
    da::note(a.sched.checks, lane != 0 || (unsigned)pid < (unsigned)a.num_pages, DA_CHECK_PAGE_ID);
    if ((unsigned)pid >= (unsigned)a.num_pages) pid = 0;
    const int slot0 = tb & (ps - 1);

    // rows past the split end are not read (their values stay 0)
    float kf[4][E], vf[4][E];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int t = tb + st * 4 + tl;
      if (t < t1) {
        const long long row = (long long)pid * ps * a.Hkv +
                              (long long)(slot0 + st * 4 + tl) * a.slot_stride +
                              (long long)g * a.head_stride;
        load_row<E>(a.k + row * kRowBytes + c * E * 4, kf[st]);
        load_row<E>(a.v + row * kRowBytes + c * E * 4, vf[st]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) kf[st][e] = vf[st][e] = 0.f;
      }
    }

    // ---- scores (log2 units); invisible tokens -> -inf
    float sc[4][RT];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int t = tb + st * 4 + tl;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) d = fmaf(qf[r][e], kf[st][e], d);
        d += da::xor_shfl<1>(d);
        d += da::xor_shfl<2>(d);
        d += da::xor_shfl<4>(d);
        d += da::xor_shfl<8>(d);
        sc[st][r] = (t < t1 && t < tend[r]) ? d : da::kNegInf;
      }
    }

    // ---- online softmax; the running max is wave-uniform
    float p[4][RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float mx = fmaxf(fmaxf(sc[0][r], sc[1][r]), fmaxf(sc[2][r], sc[3][r]));
      mx = fmaxf(mx, da::xor_shfl<16>(mx));
      mx = fmaxf(mx, da::xor_shfl<32>(mx));
      const float mn = fmaxf(m[r], mx);
      if (mn == da::kNegInf) {
#pragma unroll
        for (int st = 0; st < 4; ++st) p[st][r] = 0.f;
        continue;
      }
      const float alpha = da::fast_exp2(m[r] - mn);
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        p[st][r] = da::fast_exp2(sc[st][r] - mn);
        psum += p[st][r];
      }
      l[r] = fmaf(l[r], alpha, psum);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[r][e] *= alpha;
      m[r] = mn;
    }

    // ---- acc += p * V
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][e] = fmaf(p[st][r], vf[st][e], acc[r][e]);
      }
    }
  }

  // ---- sum the 4 token lanes of the wave (same running max)
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    l[r] += da::xor_shfl<16>(l[r]);
    l[r] += da::xor_shfl<32>(l[r]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      acc[r][e] += da::xor_shfl<16>(acc[r][e]);
      acc[r][e] += da::xor_shfl<32>(acc[r][e]);
    }
  }
  if (tl == 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm_acc[wave][r][c * E + e] = acc[r][e];
      if (c == 0) {
        sm_m[wave][r] = m[r];
        sm_l[wave][r] = l[r];
      }
    }
  }
  __syncthreads();

  // ---- combine the 4 waves and write this split's partial rows
  for (int idx = threadIdx.x; idx < nr * D; idx += kThreads) {
    const int r = idx / D, d = idx - r * D;
    float M = da::kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
    float lsum = 0.f, o = 0.f;
    if (M != da::kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = da::fast_exp2(sm_m[w][r] - M);
        lsum = fmaf(sm_l[w][r], f, lsum);
        o = fmaf(sm_acc[w][r][d], f, o);
      }
    }
    const int i = (r0 + r) / a.G, h = g * a.G + ((r0 + r) % a.G);
    const long long orow = (((long long)b * a.qn + i) * a.Hq + h) * a.sched.S + s;
    a.o[orow * D + d] = lsum > 0.f ? o / lsum : 0.f;
    if (d == 0) a.lse[orow] = lsum > 0.f ? (M + __log2f(lsum)) * da::kLn2 : da::kNegInf;
  }
}

template <int D, int RT>
int32_t launch_rt(const SplitArgs& a, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL((split_fma_kernel<D, RT>), dim3(grid), dim3(kThreads), 0, st, a);
  return da_host::launch_status();
}

// a.R: rows per block; the fp32 matrix-core kernel takes 5 or more
template <int D>
int32_t launch_d(const SplitArgs& a, unsigned grid, hipStream_t st) {
  if (a.R <= 1) return launch_rt<D, 1>(a, grid, st);
  if (a.R <= 2) return launch_rt<D, 2>(a, grid, st);
  return launch_rt<D, 4>(a, grid, st);
}

int32_t launch_f32(const da_host::SplitCall& c, const SplitArgs& a) {
  if (a.R > 4) return DA_ERR_UNSUPPORTED;
  const unsigned grid = c.grid(false);
  return c.D == 128 ? launch_d<128>(a, grid, c.stream) : launch_d<64>(a, grid, c.stream);
}

SplitArgs make_args(const da_host::SplitCall& c) {
  SplitArgs a;
  a.q = (const float*)c.q; a.k = (const uint8_t*)c.k; a.v = (const uint8_t*)c.v; a.pt = c.pt;
  a.seqlens = c.seqlens; a.sched = c.sched();
  a.o = c.o; a.lse = c.lse;
  a.pt_stride = c.pt_stride; a.max_pages = c.max_pages;
  a.qn = c.qn; a.Hq = c.Hq; a.Hkv = c.Hkv; a.G = c.Hq / c.Hkv; a.R = c.rb_rows;
  a.page_size = c.ps; a.log2_ps = __builtin_ctz((unsigned)c.ps); a.num_pages = c.num_pages;
  a.slot_stride = c.kv.slot; a.head_stride = c.kv.head;
  a.scale_log2 = c.scale * da::kLog2e;
  a.causal = c.causal;
  return a;
}

}  // namespace

// fp32 cache and fp32 Q with up to 4 query rows per row block on the vector
// ALU; -1 for any other shape (see da_split_f32_mfma for 5 or more rows).
int32_t da_split_f32_fma(const da_host::SplitCall& c) {
  if (c.q_bf16 || (c.D != 128 && c.D != 64)) return -1;
  const SplitArgs a = make_args(c);
  if (a.R > 4) return -1;
  return launch_f32(c, a);
}
