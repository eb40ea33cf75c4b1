// Stage 1 over a dense bf16 cache on the matrix cores, for D = 128 or 64 and 6
// or more query rows per kv-head, in blocks of one or two 16-row tiles (G * q:
// the MTP verify batches of LightLLM PR #1549,
// "Validation", MTP step 3, and the GQA flash decode of "Covered decode
// kernels" when G * q makes a dense 16-row tile).  Same contract as
// decode_attn_split.
//
// One workgroup (4 waves) per (kv-head g, split s, request b); 16-token tiles
// dealt round-robin to the waves (token-major pools at D = 64 with Hkv a
// multiple of 4: one kv-head per wave instead, see HQ below).  Per tile and
// wave:
//   S^T[16 tok x 16 rows] = K[16 x D] . Q^T       D/32 x v_mfma_f32_16x16x32_bf16
//   O^T[D x 16 rows]     += V^T[D x 16] . P^T     D/8 x v_mfma_f32_16x16x16_bf16
// S is computed transposed so each lane's four scores (4 tokens, one row)
// sit where the PV product wants its B operand.  Lane l = 16*lg + lm.
//
// Precision: Q, K and V enter as the bf16 values they are, so every product
// is exact in fp32 and accumulates in fp32.  The weights P are the only
// values that would need a rounding to enter the matrix core; a single bf16
// rounding of P would cost ~2e-3 rel-L2 on the output, so P goes in as two
// bf16 terms, hi = bf16(p) and lo = bf16(p - hi), in two PV products:
// |p - hi - lo| <= 2^-16 |p|.
//   * QK: MFMA kb, lane (lm, lg): token lm, elements 32*kb + 8*lg + 0..7,
//     i.e. 16-byte chunk 4*kb + lg of its row; Q^T likewise for row lm.
//   * PV: output block bb (of D/16), row m is d = (D/16)*m + bb: lane (lm, lg)
//     holds elements (D/16)*lm .. + D/16 - 1 of each of its four tokens
//     4*lg + j (a 16-byte chunk at D = 128, half of one at D = 64), and one
//     v_perm per token pair picks element bb of each.
//
// Memory pipeline: a 16-token tile is 32*D bytes of K and as many of V per
// wave.  The per-wave LDS ring holds 16 KB of such stages (two at D = 128,
// four at D = 64; two workgroups fit a CU); a stage is read into registers and
// at once refilled with the tile that many ahead, so the same number of bytes
// is in flight behind the tile being computed at either D.  Loads are
// global_load_lds (16 bytes per lane), read back by inline asm after an
// explicit vmcnt wait (the compiler would drain the queue before any LDS read
// it can see).  A row's 16-byte chunks are stored rotated by the token index
// within the tile (by half of it at D = 64, where two rows share a bank
// sweep), so both operand reads spread over the LDS banks.
//
// Softmax: one running reference m per query row, uniform over the lanes
// holding that row; raised lazily when a score exceeds m + 8 (log2 units).
#include <type_traits>

#include "mfma_util.h"

namespace {

using namespace da_mfma;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;
constexpr int kMaxSplitPages = 512;

// Per-head-dim geometry of a tile and of the LDS ring.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head dim");
  static constexpr int kChunks = D / 8;        // 16-byte chunks per K/V row
  static constexpr int kKb = D / 32;           // QK products per row tile
  static constexpr int kBlocks = D / 16;       // PV output blocks of 16 d-rows
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kStageK = 0;
  static constexpr int kStageV = 16 * kRowBytes;
  static constexpr int kStageBytes = 32 * kRowBytes;
  static constexpr int kStages = 16384 / kStageBytes;  // per wave: 16 KB
  static constexpr int kDma = D / 32;          // 1 KB DMA instructions per tensor and tile
  static constexpr int kLoads = 2 * kDma;      // per tile
  static constexpr int kRingBytes = kWaves * kStages * kStageBytes;  // 64 KB
  // LDS position of 16-byte chunk c of tile row t
  __host__ __device__ static constexpr int chunk_pos(int t, int c) {
    return (c + (D == 128 ? t : t >> 1)) & (kChunks - 1);
  }
};

template <int D>
struct StageData {
  using VT = std::conditional_t<D == 128, u32x4, u32x2>;
  u32x4 k[Geo<D>::kKb];  // token lm: chunk 4*kb + lg
  VT v[4];               // token 4*lg + j: elements (D/16)*lm .. + D/16 - 1
};

// All reads of one stage plus a page id, in one asm block.  At D = 64, token
// 4*lg + 2x + 1 sits one 128-byte row after token 4*lg + 2x, at the same
// rotation (va[x] addresses the even one).
__device__ __forceinline__ int32_t read_stage(const uint32_t (&ka)[2], const uint32_t (&va)[2],
                                              uint32_t pidaddr, StageData<64>& s) {
  int32_t pid;
  asm volatile(
      "ds_read_b128 %0, %7\n\t"
      "ds_read_b128 %1, %8\n\t"
      "ds_read_b64 %2, %9\n\t"
      "ds_read_b64 %3, %9 offset:128\n\t"
      "ds_read_b64 %4, %10\n\t"
      "ds_read_b64 %5, %10 offset:128\n\t"
      "ds_read_b32 %6, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.v[0]), "=&v"(s.v[1]), "=&v"(s.v[2]),
        "=&v"(s.v[3]), "=&v"(pid)
      : "v"(ka[0]), "v"(ka[1]), "v"(va[0]), "v"(va[1]), "v"(pidaddr)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}
__device__ __forceinline__ int32_t read_stage(const uint32_t (&ka)[4], const uint32_t (&va)[4],
                                              uint32_t pidaddr, StageData<128>& s) {
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
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.k[2]), "=&v"(s.k[3]), "=&v"(s.v[0]),
        "=&v"(s.v[1]), "=&v"(s.v[2]), "=&v"(s.v[3]), "=&v"(pid)
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(va[0]), "v"(va[1]), "v"(va[2]),
        "v"(va[3]), "v"(pidaddr)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}

struct Bf16MfmaArgs {
  const uint16_t* q;
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

__device__ __forceinline__ float bf16_to_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// two fp32 values -> packed bf16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)da::float_to_bf16_rne(lo) | ((uint32_t)da::float_to_bf16_rne(hi) << 16);
}

// NT row tiles of 16 query rows (NT * 16 rows per workgroup): the K/V
// operands of a tile are read once and serve every row tile.  HQ: kv-heads
// per workgroup.  HQ = 1: the four waves share one kv-head and take its
// tiles in turn.  HQ = 4 (token-major pools at D = 64): wave w takes kv-head
// HQ*g' + w and every tile of the split, and the waves meet at a barrier
// before each tile, so the four kv-heads' neighbouring 128-byte rows of a
// token (512 contiguous bytes) are requested by one CU together.  At D = 128
// (256-byte rows) the same mode measured slower, so it stays at HQ = 1.
template <int D, int NT, int HQ>
__global__ __launch_bounds__(kThreads, 2) void split_bf16_mfma_kernel(const Bf16MfmaArgs a) {
  static_assert(HQ == 1 || HQ == kWaves, "one kv-head per workgroup or one per wave");
  using Gm = Geo<D>;
  constexpr int kD = D, kKb = Gm::kKb, kBlocks = Gm::kBlocks, kStages = Gm::kStages;
  constexpr int kStageK = Gm::kStageK, kStageV = Gm::kStageV, kStageBytes = Gm::kStageBytes;
  constexpr int kRingBytes = Gm::kRingBytes;
  constexpr int ROWS = 16 * NT;
  constexpr int kEpiBytes = (kWaves * ROWS * kD + 2 * kWaves * ROWS) * 4;
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


  // ---- Q^T operands: row tile rt, row lm, elements 32*kb + 8*lg + e (rows
  // past the block: zero)
  u32x4 qv[NT][kKb];
  int tlim[NT];  // tokens t < tlim are visible to this lane's row of tile rt
  int lim_live = t1;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const bool live = 16 * rt + lm < nr;
    const int r = r0 + (live ? 16 * rt + lm : 0);  // this lane's query row of the kv-head
    const int i = r / a.G, h = g * a.G + r % a.G;
    const uint4* qp =
        reinterpret_cast<const uint4*>(a.q + (((long long)b * a.qn + i) * a.Hq + h) * kD + 8 * lg);
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      const uint4 x = qp[4 * kb];
      qv[rt][kb] = live ? u32x4{x.x, x.y, x.z, x.w} : u32x4{0u, 0u, 0u, 0u};
    }
    tlim[rt] = live ? min(t1, a.causal ? L - (a.qn - 1 - i) : L) : 0;
    if (live) lim_live = min(lim_live, tlim[rt]);
  }
  // the query loads are waited for here, not inside the pipeline
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) asm volatile("" : "+v"(qv[rt][kb]));
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
  const long long rowb = (long long)a.slot_stride * kD * 2;  // bytes between slots
  // DMA instruction h, lane i fills LDS chunk i of that 1 KB block: tile row
  // (64 / chunks) h + i / chunks, position i % chunks, holding the row's
  // chunk c with chunk_pos(row, c) = position
  constexpr int kC = Gm::kChunks;
  uint32_t voff[Gm::kDma];
#pragma unroll
  for (int h = 0; h < Gm::kDma; ++h) {
    const int t = (64 / kC) * h + lane / kC, p = lane % kC;
    voff[h] = (uint32_t)(t * rowb + 16 * ((p - Gm::chunk_pos(t, 0)) & (kC - 1)));
  }
  DA_LDS uint8_t* ring = (DA_LDS uint8_t*)smem + wave * (kStages * kStageBytes);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const uint32_t pid_lds = (uint32_t)(uintptr_t)(DA_LDS void*)s_pid;
  constexpr int kRow = Gm::kRowBytes;
  constexpr int kNv = D == 128 ? 4 : 2;  // V read addresses (D = 64: token pairs)
  uint32_t rd_k[kKb], rd_v[kNv];
#pragma unroll
  for (int x = 0; x < kKb; ++x) rd_k[x] = kStageK + kRow * lm + 16 * Gm::chunk_pos(lm, 4 * x + lg);
#pragma unroll
  for (int x = 0; x < kNv; ++x) {
    if constexpr (D == 128) {
      const int t = 4 * lg + x;
      rd_v[x] = kStageV + kRow * t + 16 * Gm::chunk_pos(t, lm);
    } else {
      const int t = 4 * lg + 2 * x;  // elements 4*lm .. 4*lm+3: half lm & 1 of chunk lm / 2
      rd_v[x] = kStageV + kRow * t + 16 * Gm::chunk_pos(t, lm >> 1) + 8 * (lm & 1);
    }
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
      __builtin_amdgcn_global_load_lds((const void*)(a.k + row0 * (kD * 2) + voff[h]),
                                       (DA_LDS void*)(st + kStageK + 1024 * h), 16, 0,
                                       da::kStreamPolicy);
#pragma unroll
    for (int h = 0; h < Gm::kDma; ++h)
      __builtin_amdgcn_global_load_lds((const void*)(a.v + row0 * (kD * 2) + voff[h]),
                                       (DA_LDS void*)(st + kStageV + 1024 * h), 16, 0,
                                       da::kStreamPolicy);
  };

  auto compute = [&](int j, const StageData<D>& sd, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int tb = tile_base(j) + 4 * lg;
    s16x4_t phi[NT], plo[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      // ---- S^T: dot[i] = q . k for token 4*lg + i, row lm of tile rt
      float4_t dot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb)
        dot = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, sd.k[kb]),
                                                      __builtin_bit_cast(bf16x8_t, qv[rt][kb]),
                                                      dot, 0, 0, 0);
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
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = da::fast_exp2(z[i]);
        l[rt] += p[i];
      }
      // P^T operand in two bf16 terms: hi = bf16(p), lo = bf16(p - hi)
      const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
      const uint32_t l01 = pack_bf16(p[0] - bf16_to_f(h01 & 0xffffu), p[1] - bf16_to_f(h01 >> 16));
      const uint32_t l23 = pack_bf16(p[2] - bf16_to_f(h23 & 0xffffu), p[3] - bf16_to_f(h23 >> 16));
      phi[rt] = __builtin_bit_cast(s16x4_t, u32x2{h01, h23});
      plo[rt] = __builtin_bit_cast(s16x4_t, u32x2{l01, l23});
    }

    // ---- V^T operand: tokens 4*lg + jj, d = (D/16)*lm + bb.  Rows past the
    // split end may hold anything (even NaN): zero there.
    using VT = typename StageData<D>::VT;
    VT vw[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool ok = !MASKED || tb + jj < t1;
      vw[jj] = ok ? sd.v[jj] : VT{};
    }
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb) {
      // element bb of each token's chunk: dword bb/2, half bb%2
      const uint32_t sel = (bb & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t x01 = __builtin_amdgcn_perm(vw[1][bb >> 1], vw[0][bb >> 1], sel);
      const uint32_t x23 = __builtin_amdgcn_perm(vw[3][bb >> 1], vw[2][bb >> 1], sel);
      const s16x4_t va = __builtin_bit_cast(s16x4_t, u32x2{x01, x23});
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        acc[rt][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi[rt], acc[rt][bb], 0, 0, 0);
        acc[rt][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo[rt], acc[rt][bb], 0, 0, 0);
      }
    }
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
    uint32_t ka[kKb], va[kNv];
#pragma unroll
    for (int x = 0; x < kKb; ++x) ka[x] = base + rd_k[x];
#pragma unroll
    for (int x = 0; x < kNv; ++x) va[x] = base + rd_v[x];
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
  float* sm_acc = reinterpret_cast<float*>(smem);  // [kWaves][ROWS][kD]
  float* sm_m = sm_acc + kWaves * ROWS * kD;       // [kWaves][ROWS]
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
        sm_acc[row * kD + kBlocks * (4 * lg + i) + bb] = acc[rt][bb][i];
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
      write_partials<1, ROWS, D>(sm_acc + w * ROWS * kD, sm_m + w * ROWS, sm_l + w * ROWS, r0, nr,
                                 a.G, HQ * it.g + w, b, a.qn, a.Hq, a.sched.S, s, 0.f, a.o, a.lse);
  }
}

template <int D>
void launch(const da_host::SplitCall& c, const Bf16MfmaArgs& a, int R) {
  // token-major pools at D = 64: four kv-heads per workgroup where they divide evenly
  const bool quad = D == 64 && c.kv.slot != 1 && c.Hkv % kWaves == 0;
  const dim3 grid(quad ? (unsigned)da_host::stage1_grid((long long)(c.Hkv / kWaves) * c.nrb,
                                                         c.units, c.nrb > 1)
                       : c.grid(false)),
      block(kThreads);
  if (R <= 16) {
    if (quad) hipLaunchKernelGGL((split_bf16_mfma_kernel<D, 1, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_bf16_mfma_kernel<D, 1, 1>), grid, block, 0, c.stream, a);
  } else {
    if (quad) hipLaunchKernelGGL((split_bf16_mfma_kernel<D, 2, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_bf16_mfma_kernel<D, 2, 1>), grid, block, 0, c.stream, a);
  }
}

}  // namespace

// bf16 stage 1 on the matrix cores (D = 128 or 64) for 6..16 query rows per
// kv-head (one row tile) and for more (two row tiles: blocks of up to 32
// rows, so that G * q in 17..32 reads each page once); -1 when the shape is
// not covered (the caller then reports the call as unsupported).
int32_t da_split_bf16_mfma(const da_host::SplitCall& call) {
  if (!call.q_bf16 || (call.D != 128 && call.D != 64)) return -1;
  da_host::SplitCall c = call;
  if (c.rows > DA_MAX_ROWS) da_host::row_blocks(c.rows, 2 * DA_MAX_ROWS, c.nrb, c.rb_rows);
  const int G = c.Hq / c.Hkv, R = c.rb_rows;  // rows per block
  if (R < 6) return -1;
  Bf16MfmaArgs a;
  a.q = (const uint16_t*)c.q; a.k = (const uint8_t*)c.k; a.v = (const uint8_t*)c.v;
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
