// Stage 1 over a dense fp32 cache with fp32 Q on the matrix cores (the GQA
// flash decode of LightLLM PR #1549, "Covered decode kernels", at fp32), for
// 5 or more query rows per kv-head, in blocks of one or two 16-row tiles.
// Same contract as decode_attn_split.  On the vector ALU each query row costs
// a dot product and a cross-lane sum per token, so fp32 stops being
// memory-bound there beyond 4 rows; the fp32 matrix product takes up to 16
// rows per tile at one cost.
//
// One workgroup (4 waves) per (kv-head g, split s, request b); 16-token
// tiles dealt round-robin to the waves.  Per tile and wave:
//   S^T[16 tok x 16 rows] = K[16 x D] . Q^T     D/4 x v_mfma_f32_16x16x4_f32
//   O^T[D x 16 rows]     += V^T[D x 16] . P^T   D/4 x v_mfma_f32_16x16x4_f32
// Products of fp32 values accumulated in fp32, P in fp32: nothing is
// rounded to a narrower type.  Lane l = 16*lg + lm.
//   * QK: product (x, e) takes, in lane (lm, lg), element 4*(4x + lg) + e of
//     token lm's K row and of query row lm: lane lg reads 16-byte chunks
//     lg, 4 + lg, ... of the row.
//   * PV: product (block bb, token slot jj) takes, in lane (lm, lg), element
//     d = (D/16)*lm + bb of token 4*lg + jj's V row and that token's weight
//     for query row lm, which the lane holds from S^T; output row m of
//     block bb is d = (D/16)*m + bb.
//
// Memory pipeline as in the bf16 kernel: global_load_lds (16 bytes per lane)
// into a per-wave LDS ring of 32 KB (two 16 KB stages at D = 128, four 8 KB
// ones at D = 64; one workgroup per CU), a stage read back by one inline asm
// block after an explicit vmcnt wait and refilled at once with the tile
// kStages ahead.  A row's 16-byte chunks are stored rotated by the token
// index within the tile, so the K reads (one chunk of each of 16 tokens)
// spread over the banks.
//
// Softmax: one running reference m per query row, uniform over the lanes
// holding that row; raised lazily when a score exceeds m + 8 (log2 units).
#include <type_traits>

#include "mfma_util.h"

namespace {

using namespace da_mfma;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;
constexpr int kMaxSplitPages = 512;

template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head dim");
  static constexpr int kChunks = D / 4;       // 16-byte chunks per row
  static constexpr int kKq = D / 16;          // K chunks per lane and tile
  static constexpr int kVc = D / 64;          // V chunks per token and lane
  static constexpr int kBlocks = D / 16;      // PV output blocks of 16 d-rows
  static constexpr int kRowBytes = 4 * D;
  static constexpr int kStageK = 0;
  static constexpr int kStageV = 16 * kRowBytes;
  static constexpr int kStageBytes = 32 * kRowBytes;
  static constexpr int kStages = 32768 / kStageBytes;  // per wave: 32 KB
  static constexpr int kDma = 16 * kRowBytes / 1024;   // 1 KB DMA instructions per tensor and tile
  static constexpr int kLoads = 2 * kDma;
  static constexpr int kRingBytes = kWaves * kStages * kStageBytes;  // 128 KB
  // LDS position of 16-byte chunk c of tile row t
  __host__ __device__ static constexpr int chunk_pos(int t, int c) {
    return (c + t) & (kChunks - 1);
  }
};

template <int D>
struct StageData {
  float4_t k[Geo<D>::kKq];       // token lm: chunks 4x + lg
  float4_t v[4][Geo<D>::kVc];    // token 4*lg + jj: chunks (D/64)*lm + x
};

// All reads of one stage plus a page id, in one asm block.
__device__ __forceinline__ int32_t read_stage(const uint32_t (&ka)[8], const uint32_t (&va)[8],
                                              uint32_t pidaddr, StageData<128>& s) {
  int32_t pid;
  asm volatile(
      "ds_read_b128 %0, %17\n\t"
      "ds_read_b128 %1, %18\n\t"
      "ds_read_b128 %2, %19\n\t"
      "ds_read_b128 %3, %20\n\t"
      "ds_read_b128 %4, %21\n\t"
      "ds_read_b128 %5, %22\n\t"
      "ds_read_b128 %6, %23\n\t"
      "ds_read_b128 %7, %24\n\t"
      "ds_read_b128 %8, %25\n\t"
      "ds_read_b128 %9, %26\n\t"
      "ds_read_b128 %10, %27\n\t"
      "ds_read_b128 %11, %28\n\t"
      "ds_read_b128 %12, %29\n\t"
      "ds_read_b128 %13, %30\n\t"
      "ds_read_b128 %14, %31\n\t"
      "ds_read_b128 %15, %32\n\t"
      "ds_read_b32 %16, %33\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.k[2]), "=&v"(s.k[3]), "=&v"(s.k[4]),
        "=&v"(s.k[5]), "=&v"(s.k[6]), "=&v"(s.k[7]), "=&v"(s.v[0][0]), "=&v"(s.v[0][1]),
        "=&v"(s.v[1][0]), "=&v"(s.v[1][1]), "=&v"(s.v[2][0]), "=&v"(s.v[2][1]),
        "=&v"(s.v[3][0]), "=&v"(s.v[3][1]), "=&v"(pid)
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]),
        "v"(ka[7]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]),
        "v"(va[6]), "v"(va[7]), "v"(pidaddr)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}
__device__ __forceinline__ int32_t read_stage(const uint32_t (&ka)[4], const uint32_t (&va)[4],
                                              uint32_t pidaddr, StageData<64>& s) {
  int32_t pid;
  asm volatile(
      "ds_read_b128 %0, %9\n\t"
      "ds_read_b128 %1, %10\n\t"
      "ds_read_b128 %2, %11\n\t"
      "ds_read_b128 %3, %12\n\t"
      "ds_read_b128 %4, %13\n\t"
      "ds_read_b128 %5, %14\n\t"
      "ds_read_b128 %6, %15\n\t"
      "ds_read_b128 %7, %16\n\t"
      "ds_read_b32 %8, %17\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.k[2]), "=&v"(s.k[3]), "=&v"(s.v[0][0]),
        "=&v"(s.v[1][0]), "=&v"(s.v[2][0]), "=&v"(s.v[3][0]), "=&v"(pid)
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3]), "v"(pidaddr)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}

struct F32MfmaArgs {
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

// NT row tiles of 16 query rows (NT * 16 rows per workgroup): the K/V
// operands of a tile are read once and serve every row tile.  HQ: kv-heads
// per workgroup.  HQ = 1: the four waves share one kv-head and take its
// tiles in turn.  HQ = 4 (token-major pools at D = 64): wave w takes kv-head
// HQ*g' + w and every tile of the split, and the waves meet at a barrier
// before each tile, so the four kv-heads' neighbouring rows of a token are
// requested by one CU together.
template <int D, int NT, int HQ>
__global__ __launch_bounds__(kThreads, 1) void split_f32_mfma_kernel(const F32MfmaArgs a) {
  static_assert(HQ == 1 || HQ == kWaves, "one kv-head per workgroup or one per wave");
  using Gm = Geo<D>;
  constexpr int kKq = Gm::kKq, kVc = Gm::kVc, kBlocks = Gm::kBlocks, kStages = Gm::kStages;
  constexpr int kStageK = Gm::kStageK, kStageV = Gm::kStageV, kStageBytes = Gm::kStageBytes;
  constexpr int kRingBytes = Gm::kRingBytes, kRow = Gm::kRowBytes, kC = Gm::kChunks;
  constexpr int ROWS = 16 * NT;
  constexpr int kEpiBytes = (kWaves * ROWS * D + 2 * kWaves * ROWS) * 4;
  constexpr int kMainBytes = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMainBytes + kMaxSplitPages * 4];
  int32_t* s_pid = reinterpret_cast<int32_t*>(smem + kMainBytes);

  da::Stage1Item it;
  if (!da::stage1_item<false>(a.sched, a.Hkv / HQ, it)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = HQ == 1 ? it.g : HQ * it.g + wave;  // this wave's kv-head
  const int s = it.s, b = it.b, r0 = it.r0, nr = it.nr;
  // the wave's tiles: toff, toff + tstep, ... of the split
  constexpr int tstep = HQ == 1 ? kWaves : 1;
  const int toff = HQ == 1 ? wave : 0;
  const int lm = lane & 15, lg = lane >> 4;

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

  // ---- Q^T operands: row tile rt, row lm, elements 4*(4x + lg) + e (rows
  // past the block: zero)
  float4_t qv[NT][kKq];
  int tlim[NT];  // tokens t < tlim are visible to this lane's row of tile rt
  int lim_live = t1;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const bool live = 16 * rt + lm < nr;
    const int r = r0 + (live ? 16 * rt + lm : 0);  // this lane's query row of the kv-head
    const int i = r / a.G, h = g * a.G + r % a.G;
    const float4* qp =
        reinterpret_cast<const float4*>(a.q + (((long long)b * a.qn + i) * a.Hq + h) * D) + lg;
#pragma unroll
    for (int x = 0; x < kKq; ++x) {
      const float4 y = qp[4 * x];
      qv[rt][x] = live ? float4_t{y.x, y.y, y.z, y.w} : float4_t{0.f, 0.f, 0.f, 0.f};
    }
    tlim[rt] = live ? min(t1, a.causal ? L - (a.qn - 1 - i) : L) : 0;
    if (live) lim_live = min(lim_live, tlim[rt]);
  }
  // the query loads are waited for here, not inside the pipeline
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int x = 0; x < kKq; ++x) asm volatile("" : "+v"(qv[rt][x]));
  // tiles below every live row's limit need no masks (rows past the block
  // have tlim 0 and are never written, so they do not bound the unmasked region)
  int tfull;
  {
    for (int o = 1; o < 16; o <<= 1) lim_live = min(lim_live, __shfl_xor(lim_live, o, 64));
    tfull = __builtin_amdgcn_readfirstlane(lim_live);
  }

  float4_t acc[NT][kBlocks];
  float m[NT], l[NT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb) acc[rt][bb] = {0.f, 0.f, 0.f, 0.f};
    m[rt] = da::kNegInf;
    l[rt] = 0.f;
  }

  // ---- addressing
  const long long rowb = (long long)a.slot_stride * kRow;  // bytes between slots
  // DMA instruction h, lane i fills LDS chunk 64h + i of the tile: row
  // (64h + i) / chunks, position (64h + i) % chunks, holding the row's chunk c
  // with chunk_pos(row, c) = position
  uint32_t voff[Gm::kDma];
#pragma unroll
  for (int h = 0; h < Gm::kDma; ++h) {
    const int u = 64 * h + lane, t = u / kC, p = u % kC;
    voff[h] = (uint32_t)(t * rowb + 16 * ((p - Gm::chunk_pos(t, 0)) & (kC - 1)));
  }
  DA_LDS uint8_t* ring = (DA_LDS uint8_t*)smem + wave * (kStages * kStageBytes);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const uint32_t pid_lds = (uint32_t)(uintptr_t)(DA_LDS void*)s_pid;
  uint32_t rd_k[kKq], rd_v[4 * kVc];
#pragma unroll
  for (int x = 0; x < kKq; ++x) rd_k[x] = kStageK + kRow * lm + 16 * Gm::chunk_pos(lm, 4 * x + lg);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int x = 0; x < kVc; ++x) {
      const int t = 4 * lg + jj;
      rd_v[kVc * jj + x] = kStageV + kRow * t + 16 * Gm::chunk_pos(t, kVc * lm + x);
    }

  auto tile_base = [&](int j) { return c0 + ((toff + tstep * j) << 4); };
  auto pid_addr = [&](int j) { return pid_lds + 4 * ((tile_base(j) >> a.log2_ps) - pc); };
  const long long head_row = (long long)g * a.head_stride;
  auto issue = [&](int j, int pid) {
    const long long row0 = (long long)pid * ps * a.Hkv +
                           (long long)(tile_base(j) & (ps - 1)) * a.slot_stride + head_row;
    DA_LDS uint8_t* st = ring + (j % kStages) * kStageBytes;
#pragma unroll
    for (int h = 0; h < Gm::kDma; ++h)
      __builtin_amdgcn_global_load_lds((const void*)(a.k + row0 * kRow + voff[h]),
                                       (DA_LDS void*)(st + kStageK + 1024 * h), 16, 0,
                                       da::kStreamPolicy);
#pragma unroll
    for (int h = 0; h < Gm::kDma; ++h)
      __builtin_amdgcn_global_load_lds((const void*)(a.v + row0 * kRow + voff[h]),
                                       (DA_LDS void*)(st + kStageV + 1024 * h), 16, 0,
                                       da::kStreamPolicy);
  };

  auto compute = [&](int j, const StageData<D>& sd, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int tb = tile_base(j) + 4 * lg;
    float pw[NT][4];  // weight of token 4*lg + i for row lm of tile rt
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      // ---- S^T: dot[i] = q . k for token 4*lg + i, row lm of tile rt
      float4_t dot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < kKq; ++x)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dot = __builtin_amdgcn_mfma_f32_16x16x4f32(sd.k[x][e], qv[rt][x][e], dot, 0, 0, 0);
      float z[4];
      bool need = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = fmaf(dot[i], a.scale_log2, -m[rt]);
        if (MASKED && !(tb + i < tlim[rt])) z[i] = da::kNegInf;
        need |= z[i] > kRescaleSlack;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
        // raise each row's reference to its max over the tile (rare)
        float sabs[4], mx = da::kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sabs[i] = (!MASKED || tb + i < tlim[rt]) ? dot[i] * a.scale_log2 : da::kNegInf;
          mx = fmaxf(mx, sabs[i]);
        }
        mx = fmaxf(mx, xor16(mx));
        mx = fmaxf(mx, xor32(mx));
        const float mn = fmaxf(m[rt], mx);
        const float al = mn == da::kNegInf ? 1.f : da::fast_exp2(m[rt] - mn);
        l[rt] *= al;
#pragma unroll
        for (int bb = 0; bb < kBlocks; ++bb) acc[rt][bb] *= al;
        m[rt] = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = sabs[i] == da::kNegInf ? da::kNegInf : sabs[i] - mn;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[rt][i] = da::fast_exp2(z[i]);
        l[rt] += pw[rt][i];
      }
    }

    // ---- V^T operand: token 4*lg + jj, d = (D/16)*lm + bb.  Rows past the
    // split end may hold anything (even NaN): zero there.
    float4_t vw[4][kVc];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool ok = !MASKED || tb + jj < t1;
#pragma unroll
      for (int x = 0; x < kVc; ++x) vw[jj][x] = ok ? sd.v[jj][x] : float4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
          acc[rt][bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vw[jj][bb >> 2][bb & 3], pw[rt][jj],
                                                             acc[rt][bb], 0, 0, 0);
  };

  // ---- pipeline: tile j is read into registers and its stage refilled with
  // tile j + kStages at once; tiles j+1 .. j+kStages stay in flight during
  // compute(j)
  auto step = [&](int j, StageData<D>& sd) {
    // HQ > 1: the waves (each its own kv-head, every wave the same number of
    // tiles) meet before each tile, so their reads leave the CU together
    if constexpr (HQ > 1) __builtin_amdgcn_s_barrier();
    // the tiles after j issued so far may stay in flight
    wait_tiles_ahead<Gm::kLoads, kStages - 1>(min(kStages - 1, nmine - 1 - j));
    const int jn = min(j + kStages, nmine - 1);  // the tile to issue next
    const uint32_t base = ring_lds + (j % kStages) * kStageBytes;
    uint32_t ka[kKq], va[4 * kVc];
#pragma unroll
    for (int x = 0; x < kKq; ++x) ka[x] = base + rd_k[x];
#pragma unroll
    for (int x = 0; x < 4 * kVc; ++x) va[x] = base + rd_v[x];
    const int pid = read_stage(ka, va, pid_addr(jn), sd);
    if (j + kStages < nmine) issue(j + kStages, pid);  // into the stage just read
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
    const int ntiles = (c1 - c0 + 15) >> 4;
    nmine = ntiles > toff ? (ntiles - toff + tstep - 1) / tstep : 0;
    const int lim = tfull - c0 - 16 * toff - 16;
    const int jfull = lim < 0 ? 0 : min(nmine, lim / (16 * tstep) + 1);
#pragma unroll
    for (int u = 0; u < kStages; ++u)
      if (u < nmine) issue(u, lds_read_i32(pid_addr(u)));
    for (int j = 0; j < jfull; ++j) {
      StageData<D> sd;
      step(j, sd);
      compute(j, sd, std::false_type{});
    }
    for (int j = jfull; j < nmine; ++j) {
      StageData<D> sd;
      step(j, sd);
      compute(j, sd, std::true_type{});
    }
  }

  // ---- l is partial over the lane groups; acc and m are already per row
  __syncthreads();  // ring no longer read by any wave; reuse it
  float* sm_acc = reinterpret_cast<float*>(smem);  // [kWaves][ROWS][D]
  float* sm_m = sm_acc + kWaves * ROWS * D;        // [kWaves][ROWS]
  float* sm_l = sm_m + kWaves * ROWS;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    l[rt] += xor16(l[rt]);
    l[rt] += xor32(l[rt]);
    const int row = wave * ROWS + 16 * rt + lm;
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm_acc[row * D + kBlocks * (4 * lg + i) + bb] = acc[rt][bb][i];
    if (lg == 0) {
      sm_m[row] = m[rt];
      sm_l[row] = l[rt];
    }
  }
  __syncthreads();
  if constexpr (HQ == 1) {
    write_partials<kWaves, ROWS, D>(sm_acc, sm_m, sm_l, r0, nr, a.G, g, b, a.qn, a.Hq, a.sched.S,
                                    s, 0.f, a.o, a.lse);
  } else {  // every wave's state is its kv-head's whole split
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      write_partials<1, ROWS, D>(sm_acc + w * ROWS * D, sm_m + w * ROWS, sm_l + w * ROWS, r0, nr,
                                 a.G, HQ * it.g + w, b, a.qn, a.Hq, a.sched.S, s, 0.f, a.o, a.lse);
  }
}

template <int D>
void launch(const da_host::SplitCall& c, const F32MfmaArgs& a, int R) {
  // token-major pools at D = 64: four kv-heads per workgroup where they divide evenly
  const bool quad = D == 64 && c.kv.slot != 1 && c.Hkv % kWaves == 0;
  const dim3 grid(quad ? (unsigned)da_host::stage1_grid((long long)(c.Hkv / kWaves) * c.nrb,
                                                         c.units, c.nrb > 1)
                       : c.grid(false)),
      block(kThreads);
  if (R <= 16) {
    if (quad) hipLaunchKernelGGL((split_f32_mfma_kernel<D, 1, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_f32_mfma_kernel<D, 1, 1>), grid, block, 0, c.stream, a);
  } else {
    if (quad) hipLaunchKernelGGL((split_f32_mfma_kernel<D, 2, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_f32_mfma_kernel<D, 2, 1>), grid, block, 0, c.stream, a);
  }
}

}  // namespace

// fp32 stage 1 on the matrix cores for 5 or more query rows per kv-head (one
// row tile up to 16 rows, two for blocks of up to 32); -1 for fewer, which
// stay on the vector ALU (split_fma.hip).
int32_t da_split_f32_mfma(const da_host::SplitCall& call) {
  if (call.q_bf16 || (call.D != 128 && call.D != 64)) return -1;
  da_host::SplitCall c = call;
  if (c.rows > DA_MAX_ROWS) da_host::row_blocks(c.rows, 2 * DA_MAX_ROWS, c.nrb, c.rb_rows);
  const int G = c.Hq / c.Hkv, R = c.rb_rows;  // rows per block
  if (R < 5) return -1;
  F32MfmaArgs a;
  a.q = (const float*)c.q; a.k = (const uint8_t*)c.k; a.v = (const uint8_t*)c.v;
  a.pt = c.pt; a.seqlens = c.seqlens; a.sched = c.sched(); a.o = c.o; a.lse = c.lse;
  a.pt_stride = c.pt_stride; a.max_pages = c.max_pages;
  a.qn = c.qn; a.Hq = c.Hq; a.Hkv = c.Hkv; a.G = G; a.R = R;
  a.page_size = c.ps; a.log2_ps = __builtin_ctz((unsigned)c.ps); a.num_pages = c.num_pages;
  a.slot_stride = c.kv.slot; a.head_stride = c.kv.head;
  a.scale_log2 = c.scale * da::kLog2e;
  a.causal = c.causal;
  if (c.D == 128) launch<128>(c, a, R);
  else launch<64>(c, a, R);
  return da_host::launch_status();
}
