// The vector-ALU stage-1 pipeline shared by the dense bf16 (split_bf16.hip)
// and fp32 (split_fma.hip) caches for small query groups: the GQA
// flash-decode stage 1 of LightLLM PR #1549, "Covered decode kernels".  Each
// of those files wraps split_vec_body in its own kernel and dispatch; the
// entry point that validates a call is in stage1.cpp.
//
// Work decomposition: one workgroup (4 waves) per (kv-head g, split s,
// request b); the split's tokens are cut into 8-token tiles dealt
// round-robin to the waves (or, with HQ = 4, one kv-head per wave over every
// tile: see split_vec_body).  With a batch order or a work list (requests by
// descending length, from the metadata prelude) the grid walks requests
// longest first, so the long splits are dispatched before the short ones.
//
// Lane layout: 8 lanes per token, 8 tokens per wave.  A token's K (or V) row
// is cut into 128-byte pieces (CPL of them: 2 for bf16 D = 128, 4 for fp32
// D = 128, half that at D = 64); lane (t = lane/8, c = lane%8) owns the
// 16-byte chunk c of every piece of its token's rows.  One 64-lane 16-byte
// load therefore covers the same 128-byte piece of 8 rows (whole cache
// lines), and the products need no data movement between lanes except the
// 8-lane sum of the q.k partial dots, done with three DPP adds (quad_perm
// xor 1, quad_perm xor 2, row_half_mirror).
//   q.k : bf16 - v_dot2 on bf16 pairs, fp32 accumulate (the bf16 products
//         are exact); fp32 - fp32 FMA
//   p.v : fp32 FMA with p kept in fp32
//
// Memory pipeline: tiles are fetched with global_load_lds_dwordx4 straight
// into a per-wave ring of STAGES LDS stages (2*CPL KB each), STAGES - 1 tiles
// ahead of the one being computed, so no VGPRs hold data in flight.  Each
// lane reads back exactly the 16-byte slots its own loads filled (lane i of
// a load lands at stage + 16*i), which is conflict-free.  The compiler would
// drain every outstanding LDS-DMA before any LDS read it can see, so the
// read-back is inline asm and the vmcnt wait before it is explicit: it
// waits only for the tile about to be read.  The split's page ids are staged
// in LDS once and read back with the tile, so the load addresses are formed
// in scalar registers (per-lane offsets are constant).
//
// Softmax: the wave keeps one running reference m per query row (uniform
// over its lanes).  Scores are exponentiated against m; m is raised (and
// l, acc rescaled) only when some score in the tile exceeds m + kRescaleSlack,
// so exponentials never exceed 2^kRescaleSlack and the common path has no
// max reduction.  The final (m, l, acc) are exact up to rounding and the LSE
// is m + log2(l) whatever m was.  Scores are in log2 units
// (softmax_scale * log2(e) folded into the dot product).
#pragma once

#include <type_traits>

#include "common.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define DA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
// sum over the 8 lanes of a token group (every lane receives the total)
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  return x;
}

// value held by lane ^ 8, ^ 16, ^ 32
__device__ __forceinline__ float xor8(float x) { return dpp<0x128>(x); }  // row_ror:8
__device__ __forceinline__ float xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  const bool odd_row = (threadIdx.x & 16) != 0;  // r[0]: lane^16 in odd rows, r[1]: in even rows
  return __builtin_bit_cast(float, odd_row ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  const bool upper = (threadIdx.x & 32) != 0;
  return __builtin_bit_cast(float, upper ? r[0] : r[1]);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, xor8(x));
  x = fmaxf(x, xor16(x));
  return fmaxf(x, xor32(x));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// This lane's slots of one stage (NCH 16-byte chunks, 1 KB apart) plus one
// page id, read where the compiler cannot see them (see above).
template <int NCH>
__device__ __forceinline__ int32_t lds_read_stage(uint32_t addr, uint32_t pid_addr,
                                                  u32x4 (&x)[NCH]) {
  static_assert(NCH == 2 || NCH == 4 || NCH == 8, "2, 4 or 8 chunks per stage");
  int32_t pid;
  if constexpr (NCH == 8) {
    asm volatile(
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b128 %1, %9 offset:1024\n\t"
        "ds_read_b128 %2, %9 offset:2048\n\t"
        "ds_read_b128 %3, %9 offset:3072\n\t"
        "ds_read_b128 %4, %9 offset:4096\n\t"
        "ds_read_b128 %5, %9 offset:5120\n\t"
        "ds_read_b128 %6, %9 offset:6144\n\t"
        "ds_read_b128 %7, %9 offset:7168\n\t"
        "ds_read_b32 %8, %10\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
          "=&v"(x[6]), "=&v"(x[7]), "=&v"(pid)
        : "v"(addr), "v"(pid_addr)
        : "memory");
  } else if constexpr (NCH == 4) {
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %5 offset:1024\n\t"
        "ds_read_b128 %2, %5 offset:2048\n\t"
        "ds_read_b128 %3, %5 offset:3072\n\t"
        "ds_read_b32 %4, %6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(pid)
        : "v"(addr), "v"(pid_addr)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b128 %1, %3 offset:1024\n\t"
        "ds_read_b32 %2, %4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(pid)
        : "v"(addr), "v"(pid_addr)
        : "memory");
  }
  return __builtin_amdgcn_readfirstlane(pid);
}

__device__ __forceinline__ int32_t lds_read_i32(uint32_t addr) {
  int32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}

struct VecArgs {
  const void* q;  // bf16 or fp32, the cache's element type
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

// largest split (in pages) whose page ids fit the LDS table
constexpr int kMaxSplitPages = 1024;

// EB: bytes per element (2: bf16, 4: fp32)
template <int EB, int D, int RT, int STAGES>
struct VecSmem {
  static constexpr int CPL = D * EB / 128;  // 128-byte pieces per row
  static constexpr int STAGE_BYTES = 2 * CPL * 1024;
  static constexpr int RING_BYTES = kWaves * STAGES * STAGE_BYTES;
  static constexpr int EPI_BYTES = (kWaves * 4 * RT * (D + 1) + kWaves * RT) * 4;
  static constexpr int MAIN_BYTES = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
  static constexpr int BYTES = MAIN_BYTES + kMaxSplitPages * 4;
};

// One workgroup's (kv-head, split, request) over a bf16 (F32 = false) or
// fp32 cache; smem: the kernel's VecSmem<...>::BYTES of LDS, 16-byte aligned.
// HQ: kv-heads per workgroup.  HQ = 1: the four waves share one kv-head and
// take its tiles in turn.  HQ = 4 (token-major pools): wave w takes kv-head
// HQ*g' + w and every tile of the split, and the waves meet at a barrier
// before each tile, so the four kv-heads' neighbouring rows of a token are
// requested by one CU together.
template <bool F32, int D, int RT, int STAGES, int HQ>
__device__ __forceinline__ void split_vec_body(const VecArgs& a, uint8_t* smem) {
  static_assert(HQ == 1 || HQ == kWaves, "one kv-head per workgroup or one per wave");
  constexpr int EB = F32 ? 4 : 2;
  using SM = VecSmem<EB, D, RT, STAGES>;
  constexpr int CPL = SM::CPL;
  constexpr int NCH = 2 * CPL;    // 16-byte loads per tile (K chunks, then V chunks)
  constexpr int EPC = 16 / EB;    // elements per chunk
  constexpr int E = EPC * CPL;    // elements per lane
  static_assert(CPL >= 1 && STAGES >= 2, "whole 128-byte pieces, one tile ahead");

  int32_t* s_pid = reinterpret_cast<int32_t*>(smem + SM::MAIN_BYTES);

  da::Stage1Item it;
  if (!da::stage1_item<false>(a.sched, a.Hkv / HQ, it)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = HQ == 1 ? it.g : HQ * it.g + wave;  // this wave's kv-head
  const int s = it.s, b = it.b, r0 = it.r0, nr = it.nr;
  // the wave's tiles: toff, toff + tstep, ... of the split
  constexpr int tstep = HQ == 1 ? kWaves : 1;
  const int toff = HQ == 1 ? wave : 0;
  const int tq = lane >> 3, c = lane & 7;

  const int ps = a.page_size;
  const int L = min(max(a.seqlens[b], 0), a.max_pages * ps);
  da::note(a.sched.checks,
           threadIdx.x != 0 || (a.seqlens[b] >= 0 && a.seqlens[b] <= a.max_pages * ps),
           DA_CHECK_SEQLEN);
  const int n = (L + ps - 1) >> a.log2_ps;
  const int cpg = (n + it.S - 1) / it.S;
  const int p0 = min(s * cpg, n), p1 = min((s + 1) * cpg, n);
  const int t1 = min(p1 * ps, L);  // the split's tokens end here
  // The split's page ids are staged in LDS kMaxSplitPages at a time: a longer
  // split runs as consecutive chunks (the pipeline drains at each chunk's end,
  // the softmax state carries over).  pc, c0, nmine: the current chunk's first
  // page and first token, and this wave's tile count in it.
  int pc = p0, c0 = p0 * ps, nmine = 0;
  auto stage_pids = [&](int pe) {  // page ids of pages pc .. pe - 1 into s_pid
    const int32_t* ptrow = a.pt + (long long)b * a.pt_stride;
    for (int j = threadIdx.x; j < pe - pc; j += kThreads) {
      const int pid = ptrow[pc + j];
      da::note(a.sched.checks, (unsigned)pid < (unsigned)a.num_pages, DA_CHECK_PAGE_ID);
      s_pid[j] = (unsigned)pid < (unsigned)a.num_pages ? pid : 0;
    }
  };
  stage_pids(min(p0 + kMaxSplitPages, p1));  // the first chunk's, before the query setup

  // ---- query rows r0 + r = i*G + hh; lane keeps its NCH/2 chunks of every row
  uint32_t qv[RT][4 * CPL];
  int tlim[RT];
  int tfull = t1;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int rr = r0 + (r < nr ? r : 0);
    const int i = rr / a.G, h = g * a.G + (rr % a.G);
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                        (((long long)b * a.qn + i) * a.Hq + h) * (D * EB) + 16 * c;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const uint4 x = *reinterpret_cast<const uint4*>(qp + 128 * cc);
      qv[r][4 * cc + 0] = x.x; qv[r][4 * cc + 1] = x.y;
      qv[r][4 * cc + 2] = x.z; qv[r][4 * cc + 3] = x.w;
    }
    // visibility limit of the row: split end, and the causal limit of query i
    tlim[r] = r < nr ? min(t1, a.causal ? L - (a.qn - 1 - i) : L) : 0;
    if (r < nr) tfull = min(tfull, tlim[r]);
  }
  // Make the query registers "produced" here, so the compiler waits for the
  // query loads once, before the pipeline, instead of draining the LDS-DMA
  // queue (vmcnt(0)) at their first use inside the loop.
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int w = 0; w < 4 * CPL; w += 4)
      asm volatile("" : "+v"(qv[r][w]), "+v"(qv[r][w + 1]), "+v"(qv[r][w + 2]), "+v"(qv[r][w + 3]));
  }

  float m[RT], l[RT], acc[RT][E];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m[r] = da::kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[r][e] = 0.f;
  }

  // ---- addressing: per-lane byte offsets are fixed; per-tile bases are scalar
  const long long slot_bytes = (long long)a.slot_stride * D * EB;  // between token slots
  const uint32_t voff = (uint32_t)(tq * slot_bytes + 16 * c);
  const long long head_base = (long long)g * a.head_stride * D * EB;
  const long long page_bytes = (long long)ps * a.Hkv * D * EB;
  DA_LDS uint8_t* ring = (DA_LDS uint8_t*)smem + wave * (STAGES * SM::STAGE_BYTES);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const uint32_t pid_lds = (uint32_t)(uintptr_t)(DA_LDS void*)s_pid;

  auto tile_base = [&](int j) { return c0 + ((toff + tstep * j) << 3); };
  auto pid_addr = [&](int j) { return pid_lds + 4 * ((tile_base(j) >> a.log2_ps) - pc); };
  auto issue = [&](int j, int pid) {
    const int tb = tile_base(j);
    const long long base = pid * page_bytes + (tb & (ps - 1)) * slot_bytes + head_base;
    DA_LDS uint8_t* st = ring + (j % STAGES) * SM::STAGE_BYTES;
    const uint8_t* kb = a.k + base + voff;
    const uint8_t* vb = a.v + base + voff;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc)
      __builtin_amdgcn_global_load_lds((const void*)(kb + 128 * cc), (DA_LDS void*)(st + cc * 1024),
                                       16, 0, da::kStreamPolicy);
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc)
      __builtin_amdgcn_global_load_lds((const void*)(vb + 128 * cc),
                                       (DA_LDS void*)(st + (CPL + cc) * 1024), 16, 0,
                                       da::kStreamPolicy);
  };

  auto scores = [&](const u32x4 (&x)[NCH], float (&d)[RT]) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      float t = 0.f;
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (F32)
            t = fmaf(__uint_as_float(qv[r][4 * cc + w]), __uint_as_float(x[cc][w]), t);
          else
            t = dot2_bf16(qv[r][4 * cc + w], x[cc][w], t);
        }
      }
      d[r] = sum8(t);
    }
  };

  // z = score - m (log2 units); p = exp2(z).  m starts at -inf, so the first
  // visible score always takes the (rare) rescale branch, which sets m.
  auto compute = [&](int j, const u32x4 (&x)[NCH], auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int t = tile_base(j) + tq;
    float z[RT];
    scores(x, z);
    bool need = false;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      z[r] = fmaf(z[r], a.scale_log2, -m[r]);
      if (MASKED && !(t < tlim[r])) z[r] = da::kNegInf;
      need |= z[r] > kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need)) {
      // raise the wave's reference of each row to the tile max (rare)
      float d[RT];
      scores(x, d);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const bool vis = !MASKED || t < tlim[r];
        const float sabs = vis ? d[r] * a.scale_log2 : da::kNegInf;
        const float mn = fmaxf(m[r], wave_max(sabs));
        const float al = mn == da::kNegInf ? 1.f : da::fast_exp2(m[r] - mn);  // 0 when m was -inf
        l[r] *= al;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][e] *= al;
        m[r] = mn;
        z[r] = vis ? sabs - mn : da::kNegInf;
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      z[r] = da::fast_exp2(z[r]);  // p
      l[r] += z[r];
    }
    uint32_t vw[4 * CPL];
    const bool vvalid = !MASKED || t < t1;  // V rows past the split end may hold NaN
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
      for (int w = 0; w < 4; ++w) vw[4 * cc + w] = vvalid ? x[CPL + cc][w] : 0u;
    }
#pragma unroll
    for (int w = 0; w < 4 * CPL; ++w) {
      if constexpr (F32) {
        const float v0 = __uint_as_float(vw[w]);
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][w] = fmaf(z[r], v0, acc[r][w]);
      } else {
        const float v0 = da::bf16_lo(vw[w]);
        const float v1 = da::bf16_hi(vw[w]);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          acc[r][2 * w] = fmaf(z[r], v0, acc[r][2 * w]);
          acc[r][2 * w + 1] = fmaf(z[r], v1, acc[r][2 * w + 1]);
        }
      }
    }
  };

  // ---- pipeline: STAGES - 1 tiles in flight ahead of the one computed.
  // Tiles j < jfull lie entirely below every row's visibility limit and run
  // without masks; the rest (the split's tail) run masked.  Two loops, so
  // each has a single straight-line body.
  auto step = [&](int j, u32x4 (&x)[NCH]) {
    // HQ > 1: the waves (each its own kv-head, every wave the same number of
    // tiles) meet before each tile, so their reads leave the CU together
    if constexpr (HQ > 1) __builtin_amdgcn_s_barrier();
    // wait for tile j; tiles j+1 .. min(j+STAGES-2, nmine-1) may stay in flight
    const int ahead = min(STAGES - 2, nmine - 1 - j);
    if (ahead >= 2) wait_vmcnt<2 * NCH>();
    else if (ahead == 1) wait_vmcnt<NCH>();
    else wait_vmcnt<0>();
    const int jn = min(j + STAGES - 1, nmine - 1);  // the tile to issue next
    const int pid = lds_read_stage<NCH>(ring_lds + (j % STAGES) * SM::STAGE_BYTES + lane * 16,
                                        pid_addr(jn), x);
    if (j + STAGES - 1 < nmine) issue(j + STAGES - 1, pid);  // into the stage read last iteration
  };
  for (; pc < p1; pc += kMaxSplitPages) {
    const int pe = min(pc + kMaxSplitPages, p1);
    c0 = pc * ps;
    const int c1 = min(pe * ps, t1);
    if (pc != p0) {
      __syncthreads();  // the previous chunk's page ids are no longer read
      stage_pids(pe);
    }
    __syncthreads();  // s_pid visible
    const int ntiles = (c1 - c0 + 7) >> 3;
    nmine = ntiles > toff ? (ntiles - toff + tstep - 1) / tstep : 0;
    const int lim = tfull - c0 - 8 * toff - 8;
    const int jfull = lim < 0 ? 0 : min(nmine, lim / (8 * tstep) + 1);
#pragma unroll
    for (int u = 0; u < STAGES - 1; ++u)
      if (u < nmine) issue(u, lds_read_i32(pid_addr(u)));
    for (int j = 0; j < jfull; ++j) {
      u32x4 x[NCH];
      step(j, x);
      compute(j, x, std::false_type{});
    }
    for (int j = jfull; j < nmine; ++j) {
      u32x4 x[NCH];
      step(j, x);
      compute(j, x, std::true_type{});
    }
  }

  // ---- the 8 token groups share m.  Pairs of groups are summed with one DPP
  // add (lanes ^ 8); the 4 pair sums of every wave go to LDS and are added
  // in the final pass together with the cross-wave rescale.
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    l[r] += xor8(l[r]);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[r][e] += xor8(acc[r][e]);
  }
  __syncthreads();  // ring no longer read by any wave; reuse it
  constexpr int NP = kWaves * 4;                   // partial states per row
  float* sm_acc = reinterpret_cast<float*>(smem);  // [NP][RT][D]
  float* sm_l = sm_acc + NP * RT * D;              // [NP][RT]
  float* sm_m = sm_l + NP * RT;                    // [kWaves][RT]
  if ((tq & 1) == 0) {
    const int pidx = wave * 4 + (tq >> 1);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
        for (int e = 0; e < EPC; e += 4)
          *reinterpret_cast<float4*>(sm_acc + (pidx * RT + r) * D + 8 * EPC * cc + EPC * c + e) =
              make_float4(acc[r][EPC * cc + e], acc[r][EPC * cc + e + 1],
                          acc[r][EPC * cc + e + 2], acc[r][EPC * cc + e + 3]);
      if (c == 0) {
        sm_l[pidx * RT + r] = l[r];
        if (tq == 0) sm_m[wave * RT + r] = m[r];
      }
    }
  }
  __syncthreads();

  // ---- combine the partial states and write this split's partial rows:
  // HQ = 1, the four waves' states of the kv-head; else each wave's own (its
  // kv-head's whole split), wave hw for kv-head HQ*g' + hw
  constexpr int NW = HQ == 1 ? kWaves : 1;  // waves per kv-head
  for (int idx = threadIdx.x; idx < HQ * nr * D; idx += kThreads) {
    int hw = 0, rem = idx;
    if constexpr (HQ > 1) {
      hw = idx / (nr * D);
      rem = idx - hw * (nr * D);
    }
    const int r = rem / D, d = rem - r * D;
    float M = da::kNegInf;
#pragma unroll
    for (int w = hw; w < hw + NW; ++w) M = fmaxf(M, sm_m[w * RT + r]);
    float lsum = 0.f, o = 0.f;
    if (M != da::kNegInf) {
#pragma unroll
      for (int w = hw; w < hw + NW; ++w) {
        const float f = da::fast_exp2(sm_m[w * RT + r] - M);
        float lw = 0.f, ow = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lw += sm_l[(w * 4 + k) * RT + r];
          ow += sm_acc[((w * 4 + k) * RT + r) * D + d];
        }
        lsum = fmaf(lw, f, lsum);
        o = fmaf(ow, f, o);
      }
    }
    const int gh = HQ == 1 ? g : HQ * it.g + hw;
    const int i = (r0 + r) / a.G, h = gh * a.G + ((r0 + r) % a.G);
    const long long orow = (((long long)b * a.qn + i) * a.Hq + h) * a.sched.S + s;
    a.o[orow * D + d] = lsum > 0.f ? o / lsum : 0.f;
    if (d == 0) a.lse[orow] = lsum > 0.f ? (M + __log2f(lsum)) * da::kLn2 : da::kNegInf;
  }
}

VecArgs make_vec_args(const da_host::SplitCall& c) {
  VecArgs a;
  a.q = c.q; a.k = (const uint8_t*)c.k; a.v = (const uint8_t*)c.v;
  a.pt = c.pt; a.seqlens = c.seqlens; a.sched = c.sched(); a.o = c.o; a.lse = c.lse;
  a.pt_stride = c.pt_stride; a.max_pages = c.max_pages;
  a.qn = c.qn; a.Hq = c.Hq; a.Hkv = c.Hkv; a.G = c.Hq / c.Hkv; a.R = c.rb_rows;
  a.page_size = c.ps; a.log2_ps = __builtin_ctz((unsigned)c.ps); a.num_pages = c.num_pages;
  a.slot_stride = c.kv.slot; a.head_stride = c.kv.head;
  a.scale_log2 = c.scale * da::kLog2e;
  a.causal = c.causal;
  return a;
}

}  // namespace
