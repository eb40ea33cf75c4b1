// Stage 1 over an INT8 cache on the matrix cores (LightLLM PR #1549,
// "Covered decode kernels": INT8 KV flash decode stage 1), for D = 128 or 64,
// bf16 or fp32 Q and G * q query rows per kv-head in blocks of up to 32 (one
// or two 16-row tiles per workgroup).  Same contract as
// decode_attn_split_int8: K = k_pool * k_scale, V = v_pool * v_scale, one
// fp16 scale per (page, slot, kv-head).
//
// One workgroup (4 waves) per (kv-head g, split s, request b); 16-token tiles
// dealt round-robin to the waves (token-major pools with Hkv a multiple of
// 4: one kv-head per wave instead, see HQ below).  Per tile and wave:
//   S^T[16 tok x 16 rows] = K[16 x D] . Q^T     D/32 x v_mfma_f32_16x16x32_f16
//   O^T[D x 16 rows]     += V^T[D x 16] . P^T   D/16 x v_mfma_f32_16x16x16_f16
// Computing S transposed leaves each lane's four scores (4 tokens, one row)
// where the PV product wants its B operand.  Lane l = 16*lg + lm.
//
// Scores are exact up to fp32 rounding.  A code b (-128..127) enters the QK
// product as the fp16 subnormal whose bit pattern is b + 128, i.e. the value
// (b + 128) * 2^-24: an xor with 0x80 per byte and one byte permute per
// element pair form it.  Q is scaled per row by a power of two (largest
// element in [2^14, 2^15)) and held in fp16, exact for bf16 values, so the
// products are exact in fp32.  An fp32 Q is held as two fp16 terms, hi =
// fp16(q') and lo = fp16(q' - hi) (22 significant bits; hi + lo is exact in
// fp32), each taken through the QK product into the same accumulator.  The offset is taken out with the row's fp32
// sum of scaled Q, and the token's scale multiplies the result:
//   q.k = s * 2^-sh * 2^24 * (dot - 2^-24 * 128 * sum_d q'_d).
// The PV product takes V' = fp16(b * s) (b exact in fp16; one rounding;
// below |b s| = 2^-14 an fp16 subnormal, absolute error <= 2^-25) and P =
// fp16(p * 2^7) (one rounding; p <= 2^8 under the lazy rescale, so p * 2^7 <
// 2^15, and the factor keeps small weights out of fp16's subnormal range);
// l carries the same 2^7.  Where |b s| passes 65504, V' overflows and the
// split's sums turn inf or NaN: each wave checks its sums at the end, and the
// workgroup then computes the split again with V' = fp16((b / 2^7) * s),
// which stays below 127 * 65504 / 2^7 < 65504 for any fp16 scale (absolute
// error <= 2^-25 in V', 2^-18 in v, below |b s| = 2^-7), the factor taken out
// when the partials are written.
//   * QK: MFMA kb, lane (lm, lg): token lm, elements (D/4)*lg + 8*kb + 0..7;
//     the lane reads its D/4 contiguous bytes of the row.
//   * PV: output block bb row m is d = (D/16)*m + bb: lane (lm, lg) reads
//     bytes (D/16)*lm .. + D/16 - 1 of each of its four tokens 4*lg + j.
//
// Memory pipeline: global_load_lds into a per-wave LDS ring of 16-token
// stages (K 16*D bytes, V as many, scales 256 B; 4 stages at D = 128, 8 at
// D = 64, so that about as many bytes are in flight), read back by inline
// asm after an explicit vmcnt wait.  Codes stream non-temporal, scales with
// the default policy (their lines have several readers).  At D = 128 a row's eight 16-byte chunks
// are rotated by ((token / 2) mod 8), at D = 64 its four by ((token / 4) mod
// 4), and there row 4*lg + j sits in row slot 4*lg + ((j + lg) mod 4): 64-byte
// rows 256 bytes apart would put the four lane groups' V reads on the same
// banks, and the rotation spreads the K reads.  A token's fp16 scale comes in the aligned dword
// that holds it (in bounds: a scale array holds num_pages * page_size * Hkv
// entries, an even count) and the parity of its index picks the half.
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
constexpr float kPScale = 7.0f;  // P (and l) carry a factor 2^7
constexpr int kVShift = 7;       // scaled pass: V' = v / 2^7, the output sums carry 2^-7 against l
constexpr int kMaxSplitPages = 512;

// Per-head-dim geometry of a tile and of the LDS ring.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head dim");
  static constexpr int kChunks = D / 16;     // 16-byte chunks per code row
  static constexpr int kKb = D / 32;         // QK products per row tile
  static constexpr int kBlocks = D / 16;     // PV output blocks of 16 d-rows
  static constexpr int kHw = D / 64;         // V dwords per token and lane
  static constexpr int kStageK = 0;
  static constexpr int kStageV = 16 * D;
  static constexpr int kStageSc = 32 * D;    // dwords: [0, 16) K scales, [16, 32) V scales
  static constexpr int kStageBytes = 32 * D + 256;
  static constexpr int kStages = D == 128 ? 4 : 8;
  static constexpr int kDma = D / 64;        // 1 KB DMA instructions per tensor and tile
  static constexpr int kLoads = 2 * kDma + 1;  // per tile, with the scales
  static constexpr int kRingBytes = kWaves * kStages * kStageBytes;  // 68 / 72 KB
  // rotation of token t's chunks, and the LDS row slot of token t
  __host__ __device__ static constexpr int rot(int t) { return D == 128 ? t >> 1 : t >> 2; }
  __host__ __device__ static constexpr int slot(int t) {
    return D == 128 ? t : (t & ~3) | (((t & 3) + (t >> 2)) & 3);
  }
  __host__ __device__ static constexpr int token_of_slot(int r) {
    return D == 128 ? r : (r & ~3) | (((r & 3) - (r >> 2)) & 3);
  }
  // LDS position of 16-byte chunk c of token t's row
  __host__ __device__ static constexpr int chunk_pos(int t, int c) {
    return (c + rot(t)) & (kChunks - 1);
  }
};

template <int D>
struct StageData {
  using VT = std::conditional_t<D == 128, u32x2, uint32_t>;
  u32x4 k[Geo<D>::kKb / 2];  // token lm: bytes (D/4)*lg .. + D/4 - 1
  VT v[4];                   // token 4*lg + j: bytes (D/16)*lm .. + D/16 - 1
  u32x4 ks;                  // dwords holding the K scales of tokens 4*lg + i
  u32x4 vs;                  // dwords holding the V scales of tokens 4*lg + j
};

// dword hw of a token's V bytes in a lane
__device__ __forceinline__ uint32_t vdw(u32x2 v, int hw) { return v[hw]; }
__device__ __forceinline__ uint32_t vdw(uint32_t v, int) { return v; }

// All reads of one stage plus the next page id, in one asm block (the
// compiler would otherwise drain the LDS-DMA queue before them).  D = 64:
// the four V rows sit at lane-dependent slots, so each has its own address.
__device__ __forceinline__ int32_t read_stage(const uint32_t (&ka)[1], const uint32_t (&va)[4],
                                              uint32_t sc, uint32_t pidaddr, StageData<64>& s) {
  int32_t pid;
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b32 %1, %9\n\t"
      "ds_read_b32 %2, %10\n\t"
      "ds_read_b32 %3, %11\n\t"
      "ds_read_b32 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %13 offset:64\n\t"
      "ds_read_b32 %7, %14\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.v[0]), "=&v"(s.v[1]), "=&v"(s.v[2]), "=&v"(s.v[3]),
        "=&v"(s.ks), "=&v"(s.vs), "=&v"(pid)
      : "v"(ka[0]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(sc), "v"(pidaddr)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}
// D = 128: token 4*lg + 2x + 1 sits one 128-byte row after token 4*lg + 2x,
// at the same rotation (va[x] addresses the even one).
__device__ __forceinline__ int32_t read_stage(const uint32_t (&ka)[2], const uint32_t (&va)[2],
                                              uint32_t sc, uint32_t pidaddr, StageData<128>& s) {
  const uint32_t k0 = ka[0], k1 = ka[1], v0 = va[0], v2 = va[1];
  int32_t pid;
  asm volatile(
      "ds_read_b128 %0, %9\n\t"
      "ds_read_b128 %1, %10\n\t"
      "ds_read_b64 %2, %11\n\t"
      "ds_read_b64 %3, %11 offset:128\n\t"
      "ds_read_b64 %4, %12\n\t"
      "ds_read_b64 %5, %12 offset:128\n\t"
      "ds_read_b128 %6, %13\n\t"
      "ds_read_b128 %7, %13 offset:64\n\t"
      "ds_read_b32 %8, %14\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.v[0]), "=&v"(s.v[1]), "=&v"(s.v[2]),
        "=&v"(s.v[3]), "=&v"(s.ks), "=&v"(s.vs), "=&v"(pid)
      : "v"(k0), "v"(k1), "v"(v0), "v"(v2), "v"(sc), "v"(pidaddr)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}

struct Int8Args {
  const void* q;  // bf16 or fp32
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* ks;
  const uint8_t* vs;
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

// bytes of a pair of tokens' codes (byte kk of each dword) as fp16 subnormal
// pair [b0 + 128, b1 + 128] * 2^-24, from dwords already offset by 0x80
__device__ __forceinline__ uint32_t code_pair_lo(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, 0x0C010C00u);
}
__device__ __forceinline__ uint32_t code_pair_hi(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, 0x0C030C02u);
}

// NT row tiles of 16 query rows (NT * 16 rows per workgroup): the K and V
// operands of a tile are formed once and serve every row tile.  QF: fp32 Q.
// HQ: kv-heads per workgroup.  HQ = 1: the four waves share one kv-head and
// take its tiles in turn.  HQ = 4 (token-major pools): wave w takes kv-head
// HQ*g' + w and every tile of the split, and the waves meet at a barrier
// before each tile, so the four kv-heads' neighbouring code rows (512
// contiguous bytes of a token) and their shared scale lines are requested by
// one CU together.
template <int D, int NT, bool QF, int HQ>
__global__ __launch_bounds__(kThreads, 2) void split_int8_mfma_kernel(const Int8Args a) {
  static_assert(HQ == 1 || HQ == kWaves, "one kv-head per workgroup or one per wave");
  using Gm = Geo<D>;
  constexpr int kD = D, kKb = Gm::kKb, kBlocks = Gm::kBlocks, kStages = Gm::kStages;
  constexpr int kStageK = Gm::kStageK, kStageV = Gm::kStageV, kStageSc = Gm::kStageSc;
  constexpr int kStageBytes = Gm::kStageBytes, kRingBytes = Gm::kRingBytes;
  constexpr int ROWS = 16 * NT;
  constexpr int kEpiBytes = (kWaves * ROWS * kD + 2 * kWaves * ROWS) * 4;
  constexpr int kMainBytes = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMainBytes + kMaxSplitPages * 4];
  int32_t* s_pid = reinterpret_cast<int32_t*>(smem + kMainBytes);
  __shared__ int s_redo;  // a wave's V operand left fp16's range

  da::Stage1Item it;
  if (!da::stage1_item<true>(a.sched, a.Hkv / HQ, it)) return;
  if (threadIdx.x == 0) s_redo = 0;  // ordered before any write by the loop's barriers
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


  // ---- Q^T operands: row tile rt, row lm, elements (D/4)*lg + 8*kb + e,
  // scaled by 2^sh, fp16
  uint32_t qv[NT][kKb][4];  // [rt][kb][pair]
  uint32_t ql[NT][QF ? kKb : 1][4];  // fp32 Q: the lo terms
  float rowfac[NT];       // score (log2 units) = s * (rowfac * dot - qoff)
  float qoff[NT];         // rowfac * 128 * 2^-24 * sum of the row's scaled Q
  int tlim[NT];           // tokens t < tlim are visible to this lane's row
  int lim_live = t1;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const bool live = 16 * rt + lm < nr;
    const int r = r0 + (live ? 16 * rt + lm : 0);  // this lane's query row of the kv-head
    const int i = r / a.G, h = g * a.G + r % a.G;
    const long long qoff_el = (((long long)b * a.qn + i) * a.Hq + h) * kD + (kD / 4) * lg;
    float qf[kKb][8];
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      load_q8<QF>(a.q, qoff_el + 8 * kb, qf[kb]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kb][e] = live ? qf[kb][e] : 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qf[kb][e]));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const int sh = q_row_shift(mx);
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      float lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = ldexpf(qf[kb][e], sh);
        qf[kb][e] = (float)(_Float16)x;
        sum += qf[kb][e];
        if constexpr (QF) {
          lo[e] = (float)(_Float16)(x - qf[kb][e]);
          sum += lo[e];
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        qv[rt][kb][x] = pack_h2(qf[kb][2 * x], qf[kb][2 * x + 1]);
        if constexpr (QF) ql[rt][kb][x] = pack_h2(lo[2 * x], lo[2 * x + 1]);
      }
    }
    sum += xor16(sum);
    sum += xor32(sum);
    rowfac[rt] = ldexpf(a.scale_log2, 24 - sh);
    qoff[rt] = rowfac[rt] * ldexpf(sum, -17);  // 128 * 2^-24 = 2^-17
    tlim[rt] = live ? min(t1, a.causal ? L - (a.qn - 1 - i) : L) : 0;
    if (live) lim_live = min(lim_live, tlim[rt]);
  }
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb) {
      asm volatile("" : "+v"(qv[rt][kb][0]), "+v"(qv[rt][kb][1]), "+v"(qv[rt][kb][2]),
                   "+v"(qv[rt][kb][3]));
      if constexpr (QF)
        asm volatile("" : "+v"(ql[rt][kb][0]), "+v"(ql[rt][kb][1]), "+v"(ql[rt][kb][2]),
                     "+v"(ql[rt][kb][3]));
    }
  // tiles below every live row's limit need no masks (rows past the block
  // have tlim 0 and are never written, so they do not bound the unmasked region)
  int tfull;
  {
    for (int o = 1; o < 16; o <<= 1) lim_live = min(lim_live, __shfl_xor(lim_live, o, 64));
    tfull = __builtin_amdgcn_readfirstlane(lim_live);
  }

  float4_t acc[NT][kBlocks];
  float m[NT], l[NT];
  auto reset_state = [&]() {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
      for (int bb = 0; bb < kBlocks; ++bb) acc[rt][bb] = {0.f, 0.f, 0.f, 0.f};
      m[rt] = da::kNegInf;
      l[rt] = 0.f;
    }
  };
  reset_state();

  // ---- addressing
  const long long rowb = (long long)a.slot_stride * kD;  // bytes between slots (codes)
  // DMA lane i of 1 KB block h fills LDS chunk i of that block: row slot
  // (64 / chunks) h + i / chunks, position i % chunks, holding chunk c of the
  // slot's token with chunk_pos(token, c) = position
  constexpr int kC = Gm::kChunks;
  uint32_t voff_kv[Gm::kDma];
#pragma unroll
  for (int h = 0; h < Gm::kDma; ++h) {
    const int t = Gm::token_of_slot((64 / kC) * h + lane / kC), p = lane % kC;
    voff_kv[h] = (uint32_t)(t * rowb + 16 * ((p - Gm::rot(t)) & (kC - 1)));
  }
  // scale DMA: lanes 0..15 K scale of token i, 16..31 V scale of token i-16,
  // 32..63 repeat lanes 0..31 (their LDS words are not read)
  const int sc_tok = lane & 15;
  const uint8_t* sc_base = ((lane >> 4) & 1) ? a.vs : a.ks;
  DA_LDS uint8_t* ring = (DA_LDS uint8_t*)smem + wave * (kStages * kStageBytes);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const uint32_t pid_lds = (uint32_t)(uintptr_t)(DA_LDS void*)s_pid;
  // K: the lane's D/4 bytes of token lm are chunks (D/64) lg .. + D/64 - 1.
  // V: bytes (D/16) lm .. of token t are in chunk lm / (16 / (D/16)).
  constexpr int kRow = D;  // bytes per code row
  constexpr int kNk = kKb / 2, kNv = D == 128 ? 2 : 4;
  uint32_t rd_k[kNk], rd_v[kNv];
#pragma unroll
  for (int x = 0; x < kNk; ++x)
    rd_k[x] = kStageK + kRow * Gm::slot(lm) + 16 * Gm::chunk_pos(lm, kNk * lg + x);
#pragma unroll
  for (int x = 0; x < kNv; ++x) {
    constexpr int kVb = D / 16;            // V bytes per token and lane
    constexpr int kPer = 16 / kVb;         // lanes per chunk
    const int t = D == 128 ? 4 * lg + 2 * x : 4 * lg + x;
    rd_v[x] = kStageV + kRow * Gm::slot(t) + 16 * Gm::chunk_pos(t, lm / kPer) + kVb * (lm % kPer);
  }
  const uint32_t rd_sc = kStageSc + 16 * lg;

  auto tile_base = [&](int j) { return c0 + ((toff + tstep * j) << 4); };
  auto pid_addr = [&](int j) { return pid_lds + 4 * ((tile_base(j) >> a.log2_ps) - pc); };
  const long long head_row = (long long)g * a.head_stride;
  auto issue = [&](int j, int pid) {
    // row of the tile's first slot
    const long long row0 = (long long)pid * ps * a.Hkv +
                           (long long)(tile_base(j) & (ps - 1)) * a.slot_stride + head_row;
    DA_LDS uint8_t* st = ring + (j % kStages) * kStageBytes;
#pragma unroll
    for (int h = 0; h < Gm::kDma; ++h)
      __builtin_amdgcn_global_load_lds((const void*)(a.k + row0 * kD + voff_kv[h]),
                                       (DA_LDS void*)(st + kStageK + 1024 * h), 16, 0,
                                       da::kStreamPolicy);
#pragma unroll
    for (int h = 0; h < Gm::kDma; ++h)
      __builtin_amdgcn_global_load_lds((const void*)(a.v + row0 * kD + voff_kv[h]),
                                       (DA_LDS void*)(st + kStageV + 1024 * h), 16, 0,
                                       da::kStreamPolicy);
    // The scales keep the default policy: a 2-byte scale per token puts
    // several readers on one cache line (head-major: the four waves' tiles;
    // token-major: the eight kv-heads' workgroups), and a non-temporal read
    // would evict the line before the next reader comes.
    const long long e = row0 + (long long)sc_tok * a.slot_stride;  // scale index
    __builtin_amdgcn_global_load_lds((const void*)(sc_base + ((2 * e) & ~3ll)),
                                     (DA_LDS void*)(st + kStageSc), 4, 0, 0);
  };

  // Half of the scale dword holding token 4*lg + i's scale.  Its index is
  // pid * page_size * Hkv + (slot0 + 4*lg + i) * slot_stride + g * head_stride
  // with page_size even and slot0 a multiple of 16, so its parity is that
  // of i * slot_stride + g * head_stride.
  int sc_shift[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc_shift[i] = ((i * a.slot_stride + g * a.head_stride) & 1) << 4;

  auto compute = [&](int j, const StageData<D>& sd, auto masked_tag, auto scaled_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool SCALED = decltype(scaled_tag)::value;  // V formed as v / 2^7
    // ---- dot[rt][i] = 2^-24 * sum_d q'_d (b_d + 128) for token 4*lg + i, row lm
    // of tile rt
    float4_t dot[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) dot[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
    {
      uint32_t kw[2 * kKb];
#pragma unroll
      for (int x = 0; x < 2 * kKb; ++x) kw[x] = sd.k[x >> 2][x & 3] ^ 0x80808080u;
#pragma unroll
      for (int kb = 0; kb < kKb; ++kb) {
        const half2_t c0 = as_h2(code_pair_lo(kw[2 * kb])), c1 = as_h2(code_pair_hi(kw[2 * kb]));
        const half2_t c2 = as_h2(code_pair_lo(kw[2 * kb + 1]));
        const half2_t c3 = as_h2(code_pair_hi(kw[2 * kb + 1]));
        const half8_t ka = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          const half2_t q0 = as_h2(qv[rt][kb][0]), q1 = as_h2(qv[rt][kb][1]);
          const half2_t q2 = as_h2(qv[rt][kb][2]), q3 = as_h2(qv[rt][kb][3]);
          const half8_t qb = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
          dot[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb, dot[rt], 0, 0, 0);
          if constexpr (QF) {
            const half2_t l0 = as_h2(ql[rt][kb][0]), l1 = as_h2(ql[rt][kb][1]);
            const half2_t l2 = as_h2(ql[rt][kb][2]), l3 = as_h2(ql[rt][kb][3]);
            const half8_t lb = {l0[0], l0[1], l1[0], l1[1], l2[0], l2[1], l3[0], l3[1]};
            dot[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, lb, dot[rt], 0, 0, 0);
          }
        }
      }
    }
    const int tb = tile_base(j) + 4 * lg;
    uint32_t ksc[4], vsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ksc[i] = sd.ks[i] >> sc_shift[i];
      vsc[i] = sd.vs[i] >> sc_shift[i];
    }
    half4_t pb[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      float z[4], tq[4];
      bool need = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tq[i] = fmaf(dot[rt][i], rowfac[rt], -qoff[rt]);
        z[i] = fmaf(h_lo(ksc[i]), tq[i], kPScale - m[rt]);
        if (MASKED && !(tb + i < tlim[rt])) z[i] = da::kNegInf;
        need |= z[i] > kRescaleSlack + kPScale;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
        float sabs[4], mx = da::kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sabs[i] = (!MASKED || tb + i < tlim[rt]) ? h_lo(ksc[i]) * tq[i] : da::kNegInf;
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
        for (int i = 0; i < 4; ++i)
          z[i] = sabs[i] == da::kNegInf ? da::kNegInf : sabs[i] - (mn - kPScale);
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = da::fast_exp2(z[i]);
        l[rt] += p[i];
      }
      pb[rt] = half4_t{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    }

    // ---- V operand: tokens 4*lg + j, d = (D/16)*lm + block.  Rows past the
    // split end may hold anything (even NaN scales): code 0, scale 0 there.
    constexpr int kHw = Gm::kHw;
    uint32_t vw[4][kHw], vs[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool ok = !MASKED || tb + jj < t1;
#pragma unroll
      for (int hw = 0; hw < kHw; ++hw) vw[jj][hw] = ok ? vdw(sd.v[jj], hw) : 0u;
      vs[jj] = ok ? vsc[jj] : 0u;
    }
    const half2_t s01 = as_h2(__builtin_amdgcn_perm(vs[1], vs[0], 0x05040100u));
    const half2_t s23 = as_h2(__builtin_amdgcn_perm(vs[3], vs[2], 0x05040100u));
    // the code byte b + 128 in the mantissa of 1024 + (b + 128) (ulp 1), minus
    // 1152: b exactly, and times s: fp16(b s); on the scaled pass in that of
    // 8 + (b + 128) / 2^7 (ulp 2^-7), minus 9: b / 2^7, and fp16(b s / 2^7),
    // which no fp16 scale can overflow
    constexpr uint32_t kHi = SCALED ? 0x48804880u : 0x64806480u;
    const half2_t kOff = SCALED ? half2_t{9, 9} : half2_t{1152, 1152};
#pragma unroll
    for (int hw = 0; hw < kHw; ++hw) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int bb = 4 * hw + kk;
        // [t0.byte kk, 0, t1.byte kk, 0], then bytes ^ 0x80 and the exponent
        // byte above them
        const uint32_t sel = (uint32_t)kk | 0x0C00u | ((uint32_t)(4 + kk) << 16) | 0x0C000000u;
        const uint32_t x01 = __builtin_amdgcn_perm(vw[1][hw], vw[0][hw], sel) ^ kHi;
        const uint32_t x23 = __builtin_amdgcn_perm(vw[3][hw], vw[2][hw], sel) ^ kHi;
        const half2_t a01 = (as_h2(x01) - kOff) * s01;
        const half2_t a23 = (as_h2(x23) - kOff) * s23;
        const half4_t va = {a01[0], a01[1], a23[0], a23[1]};
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
          acc[rt][bb] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb[rt], acc[rt][bb], 0, 0, 0);
      }
    }
  };

  auto step = [&](int j, StageData<D>& sd) {
    // HQ > 1: the waves (each its own kv-head, every wave the same number of
    // tiles) meet before each tile, so their reads of neighbouring rows and
    // shared lines leave the CU together
    if constexpr (HQ > 1) __builtin_amdgcn_s_barrier();
    // the tiles after j issued so far may stay in flight
    wait_tiles_ahead<Gm::kLoads, kStages - 2>(min(kStages - 2, nmine - 1 - j));
    const int jn = min(j + kStages - 1, nmine - 1);
    const uint32_t base = ring_lds + (j % kStages) * kStageBytes;
    uint32_t ka[kNk], va[kNv];
#pragma unroll
    for (int x = 0; x < kNk; ++x) ka[x] = base + rd_k[x];
#pragma unroll
    for (int x = 0; x < kNv; ++x) va[x] = base + rd_v[x];
    const int pid = read_stage(ka, va, base + rd_sc, pid_addr(jn), sd);
    if (j + kStages - 1 < nmine) issue(j + kStages - 1, pid);
  };
  auto run_split = [&](auto sc) {
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
      for (int u = 0; u < kStages - 1; ++u)
        if (u < nmine) issue(u, lds_read_i32(pid_addr(u)));
      for (int j = 0; j < jfull; ++j) {
        StageData<D> sd;
        step(j, sd);
        compute(j, sd, std::false_type{}, sc);
      }
      for (int j = jfull; j < nmine; ++j) {
        StageData<D> sd;
        step(j, sd);
        compute(j, sd, std::true_type{}, sc);
      }
    }
  };
  run_split(std::false_type{});

  // ---- V formed as fp16(b s) overflows where |b s| passes 65504, leaving
  // inf or NaN in the output sums; then the split is computed again with V
  // formed as fp16(b s / 2^7), which no fp16 scale can overflow, and the
  // factor is taken out again when the partials are written.
  int vshift = 0;
  {
    bool bad = false;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad |= !(fabsf(acc[rt][bb][i]) <= 3.0e38f);
    if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) s_redo = 1;
  }
  __syncthreads();
  if (s_redo) {  // uniform over the workgroup
    vshift = kVShift;
    reset_state();
    pc = p0;
    stage_pids(min(p0 + kMaxSplitPages, p1));  // every wave is past its last LDS read
    run_split(std::true_type{});
  }

  // ---- l is partial over the lane groups; acc and m are already per row
  __syncthreads();
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
                                    s, kPScale, a.o, a.lse, vshift);
  } else {  // every wave's state is its kv-head's whole split
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      write_partials<1, ROWS, D>(sm_acc + w * ROWS * kD, sm_m + w * ROWS, sm_l + w * ROWS, r0, nr,
                                 a.G, HQ * it.g + w, b, a.qn, a.Hq, a.sched.S, s, kPScale, a.o,
                                 a.lse, vshift);
  }
}

template <int D, bool QF>
void launch(const da_host::SplitCall& c, const Int8Args& a, int R) {
  // token-major pools: four kv-heads per workgroup where they divide evenly
  const bool quad = c.kv.slot != 1 && c.Hkv % kWaves == 0;
  const dim3 grid(quad ? (unsigned)da_host::stage1_grid((long long)(c.Hkv / kWaves) * c.nrb,
                                                         c.units, true)
                       : c.grid(true)),
      block(kThreads);
  if (R <= 16) {
    if (quad) hipLaunchKernelGGL((split_int8_mfma_kernel<D, 1, QF, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_int8_mfma_kernel<D, 1, QF, 1>), grid, block, 0, c.stream, a);
  } else {
    if (quad) hipLaunchKernelGGL((split_int8_mfma_kernel<D, 2, QF, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_int8_mfma_kernel<D, 2, QF, 1>), grid, block, 0, c.stream, a);
  }
}

}  // namespace

// INT8 stage 1 on the matrix cores (D = 128 or 64, bf16 or fp32 Q), one row
// tile (up to 16 query rows per kv-head) or two (blocks of up to 32 rows, so
// that G * q in 17..32 forms each tile's operands once); -1 when the shape is
// not covered (the caller then reports the call as unsupported).
int32_t da_split_int8_mfma(const da_host::SplitCall& call) {
  if (call.D != 128 && call.D != 64) return -1;
  da_host::SplitCall c = call;
  if (c.rows > DA_MAX_ROWS) da_host::row_blocks(c.rows, 2 * DA_MAX_ROWS, c.nrb, c.rb_rows);
  const int G = c.Hq / c.Hkv, R = c.rb_rows;  // rows per block
  Int8Args a;
  a.q = c.q; a.k = (const uint8_t*)c.k; a.v = (const uint8_t*)c.v;
  a.ks = (const uint8_t*)c.ks; a.vs = (const uint8_t*)c.vs;
  a.pt = c.pt; a.seqlens = c.seqlens; a.sched = c.sched(); a.o = c.o; a.lse = c.lse;
  a.pt_stride = c.pt_stride; a.max_pages = c.max_pages;
  a.qn = c.qn; a.Hq = c.Hq; a.Hkv = c.Hkv; a.G = G; a.R = R;
  a.page_size = c.ps; a.log2_ps = __builtin_ctz((unsigned)c.ps); a.num_pages = c.num_pages;
  a.slot_stride = c.kv.slot; a.head_stride = c.kv.head;
  a.scale_log2 = c.scale * da::kLog2e;
  a.causal = c.causal;
  if (c.q_bf16) {
    if (c.D == 128) launch<128, false>(c, a, R);
    else launch<64, false>(c, a, R);
  } else {
    if (c.D == 128) launch<128, true>(c, a, R);
    else launch<64, true>(c, a, R);
  }
  return da_host::launch_status();
}
