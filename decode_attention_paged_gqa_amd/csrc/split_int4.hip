// Stage 1 over an INT4 cache on the matrix cores, for D = 128 or 64 and any
// number of query rows per kv-head (G*q, in blocks of up to 32: one or two 16-row tiles per
// workgroup; a partly filled tile still beats the vector ALU, whose 4-bit
// expansion cannot keep pace with the memory stream; e.g. the MTP verify
// batches of LightLLM
// PR #1549 "Covered decode kernels": INT4 KV flash decode stage 1, MTP
// attention; SGLang #36219 digest code listing: several tokens per request).
// Same contract as decode_attn_split_int4.
//
// One workgroup (4 waves) per (kv-head g, split s, request b); 16-token
// tiles dealt round-robin to the waves (token-major pools with Hkv a
// multiple of 4: one kv-head per wave instead, see HQ below).  Per tile and
// wave:
//   S^T[16 tok x 16 rows] = K[16 x D] . Q^T   D/32 x v_mfma_f32_16x16x32_f16
//   O^T[D x 16 rows]     += V^T[D x 16] . P^T D/16 x v_mfma_f32_16x16x16_f16
// Computing S transposed puts each lane's four scores (4 tokens, one row)
// exactly where the PV product wants its B operand, so P never moves
// between lanes.  Lane l = 16*lg + lm: QK row (token) lm, PV row (d) lm.
//
// Scores are exact up to fp32 rounding: each QK product covers ONE
// quantisation group (32 elements of D), so the group's (scale, zero) is a
// per-token constant of that product:
//   q.k = sum_g s_g * (sum_{d in g} q_d n_d  -  z_g * sum_{d in g} q_d).
// The codes n (0..15) enter the matrix core as fp16 subnormals with the
// bit pattern n, i.e. the value n * 2^-24 (exact; the product with an fp16
// Q element is exact in fp32).  Q is scaled by a power of two per row so its
// largest element lies in [2^14, 2^15) before the (then exact, for bf16)
// conversion to fp16; the power of two and 2^24 are folded into the score
// factor.  An fp32 Q is held as two fp16 terms, hi = fp16(q') and lo =
// fp16(q' - hi) (22 significant bits; hi + lo is exact in fp32), each taken
// through the group's QK product into the same accumulator, and the group
// sums of Q add both.  The per-group terms are combined in fp32 with the group's s and
// z: the scale terms s_g * dot_g on the vector ALU (one mixed-precision fma
// each), the zero-point terms -sum_g (s_g z_g) sum_g(q) as one fp32 matrix
// product [16 tokens x 4 groups] . [4 groups x 16 rows] (s_g z_g is exact in
// fp32; at D = 64 groups 2 and 3 are zero), so any fp16 zero point is taken
// exactly.
//   * QK: MFMA kb is group kb.  Lane (lm, lg) supplies token lm's dword lg
//     of that group (elements 32*kb + 8*lg + 0..7); k-slots 2x, 2x+1 are
//     elements x and x+4 of the dword (nibble x of its two halves).  Pairs
//     0 and 2 are masked into bits 0..3 (n * 2^-24); pairs 1 and 3 are
//     masked where they lie, bits 4..7 (16 n * 2^-24, still exact), and
//     their Q elements are divided by 16 instead.
//   * PV: output block b row m is d = (D/16)*m + b: lane (lm, lg) reads, for
//     its four tokens 4*lg+j, elements (D/16)*lm .. + D/16 - 1 of each row
//     (D = 128: dword lm, in group lm/4; D = 64: half lm%2 of dword lm/2, in
//     group lm/8).  Every d-row of a lane lies in one group, so V = n*s - z*s
//     splits into two products: V^T operand fp16(n*s), one fma per element
//     pair on the exact code 1024 + n (fma(1024 + n, s, -1024 s); a high
//     nibble is taken in place as 1024 + 16 n, giving fp16(16 n s), and its
//     output blocks are divided by 16 at the end), and the zero-point term,
//     one product per tile of the tokens' -fp16(z*s) (the lane's group) with
//     P, accumulated apart and added at the end.
//     P enters as fp16(p * 2^7) (p <= 2^8 under the lazy rescale below, so
//     p * 2^7 < 2^15; the factor keeps small weights out of fp16's subnormal
//     range and cancels against the same factor in l): the roundings of
//     n*s, z*s and P are the only ones in the product.
//
// Memory pipeline as in the bf16 kernel: global_load_lds into a per-wave LDS
// ring, read back by inline asm after an explicit vmcnt wait.  D = 128: 4
// stages of K 1 KB, V 1 KB and the two scale/zero tiles of 256 B each per 16
// tokens; the K and V tiles are stored with their 16-byte chunks rotated by
// (token / 4) so that the dword reads of both operands (K: one group of
// token lm; V: dword lm of token 4*lg + j) hit distinct banks.  D = 64: 4
// stages of K 512 B, V 512 B (one DMA: lanes 0..31 fetch K, 32..63 V) and the
// scale/zero tiles of 128 B each (one DMA likewise); the 32-byte rows are
// stored transposed (token t in row slot 4 (t % 4) + t / 4) with their two
// chunks rotated by ((t / 2) mod 2), which again puts both operand reads on
// distinct banks.  With four kv-heads per workgroup (token-major pools) the
// waves fill one ring together instead, each DMA fetching whole token rows
// of all four heads (see the kernel).
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
constexpr int kMaxSplitPages = 512;

// Per-head-dim geometry of a tile and of the LDS ring.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head dim");
  static constexpr int kGroups = D / 32;     // quantisation groups per row
  static constexpr int kBlocks = D / 16;     // PV output blocks of 16 d-rows
  static constexpr int kRowBytes = D / 2;    // code bytes per row
  static constexpr int kSzBytes = 4 * kGroups;  // (scale, zero) bytes per row
  static constexpr int kStageK = 0;
  static constexpr int kStageV = 16 * kRowBytes;
  static constexpr int kStageKsz = 32 * kRowBytes;
  static constexpr int kStageVsz = kStageKsz + 16 * kSzBytes;
  static constexpr int kStageBytes = kStageVsz + 16 * kSzBytes;  // 2560 / 1280
  // four tiles per wave in the ring at either head dim (at D = 64 four ran
  // faster than six or eight, in both pool layouts)
  static constexpr int kStages = 4;
  static constexpr int kLoads = D == 128 ? 4 : 2;  // DMA instructions per tile
  static constexpr int kRingBytes = kWaves * kStages * kStageBytes;  // 40 KB / 20 KB
  // row slot of token t in a code tile, and the rotation of its chunks
  __host__ __device__ static constexpr int slot(int t) {
    return D == 128 ? t : 4 * (t & 3) + (t >> 2);  // an involution at D = 64
  }
  __host__ __device__ static constexpr int rot(int t) { return D == 128 ? t >> 2 : (t >> 1) & 1; }
};

template <int D>
struct StageData;
template <>
struct StageData<128> {
  uint32_t k[4];   // token lm, group kb: dword lg (elements 32*kb + 8*lg + 0..7)
  uint32_t v[4];   // dword lm of tokens 4*lg + j
  u32x4 ksz[4];    // (scale, zero) of token 4*lg + i, groups 0..3
  uint32_t vsz[4]; // (scale, zero) of token 4*lg + j, group lm/4
  uint32_t kz;     // (scale, zero) of token lm, group lg
};
template <>
struct StageData<64> {
  uint32_t k[2];   // token lm, group kb: dword lg (elements 32*kb + 8*lg + 0..7)
  uint32_t v[4];   // dword lm/2 of tokens 4*lg + j
  u32x2 ksz[4];    // (scale, zero) of token 4*lg + i, groups 0..1
  uint32_t vsz[4]; // (scale, zero) of token 4*lg + j, group lm/8
  uint32_t kz;     // (scale, zero) of token lm, group lg & 1
};

// D = 64: all reads of one stage (at a lane-specific address plus ST, the
// stage offset or 0 where the address already holds it) plus the next page
// id.  V rows of tokens 4*lg + 2x and 4*lg + 2x + 1 sit 128 bytes apart
// (va[x] addresses the first).
template <int ST, int SZS = 8>
__device__ __forceinline__ int32_t read_stage64(const uint32_t (&kaddr)[2],
                                                const uint32_t (&vaddr)[2], uint32_t kszaddr,
                                                uint32_t vszaddr, uint32_t kzaddr,
                                                uint32_t pidaddr, StageData<64>& s) {
  int32_t pid;
  asm volatile(
      "ds_read_b32 %0, %16 offset:%24\n\t"
      "ds_read_b32 %1, %17 offset:%24\n\t"
      "ds_read_b32 %2, %18 offset:%24\n\t"
      "ds_read_b32 %3, %18 offset:%24+128\n\t"
      "ds_read_b32 %4, %19 offset:%24\n\t"
      "ds_read_b32 %5, %19 offset:%24+128\n\t"
      "ds_read_b64 %6, %20 offset:%24\n\t"
      "ds_read_b64 %7, %20 offset:%24+%25\n\t"
      "ds_read_b64 %8, %20 offset:%24+2*%25\n\t"
      "ds_read_b64 %9, %20 offset:%24+3*%25\n\t"
      "ds_read_b32 %10, %21 offset:%24\n\t"
      "ds_read_b32 %11, %21 offset:%24+%25\n\t"
      "ds_read_b32 %12, %21 offset:%24+2*%25\n\t"
      "ds_read_b32 %13, %21 offset:%24+3*%25\n\t"
      "ds_read_b32 %14, %22 offset:%24\n\t"
      "ds_read_b32 %15, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.v[0]), "=&v"(s.v[1]), "=&v"(s.v[2]),
        "=&v"(s.v[3]), "=&v"(s.ksz[0]), "=&v"(s.ksz[1]), "=&v"(s.ksz[2]), "=&v"(s.ksz[3]),
        "=&v"(s.vsz[0]), "=&v"(s.vsz[1]), "=&v"(s.vsz[2]), "=&v"(s.vsz[3]), "=&v"(s.kz),
        "=&v"(pid)
      : "v"(kaddr[0]), "v"(kaddr[1]), "v"(vaddr[0]), "v"(vaddr[1]), "v"(kszaddr), "v"(vszaddr),
        "v"(kzaddr), "v"(pidaddr), "i"(ST), "i"(SZS)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}

// All reads of ring stage ST (its byte offset, a constant folded into the
// instructions' offset fields) plus the next page id, in one asm block (the
// compiler would otherwise drain the LDS-DMA queue before them).  The
// address operands are the lanes' fixed positions inside stage 0.
template <int ST>
__device__ __forceinline__ int32_t read_stage(const uint32_t (&kaddr)[4], uint32_t vaddr,
                                              uint32_t kszaddr, uint32_t vszaddr,
                                              uint32_t kzaddr, uint32_t pidaddr,
                                              StageData<128>& s) {
  int32_t pid;
  asm volatile(
      "ds_read_b32 %0, %18 offset:%27\n\t"
      "ds_read_b32 %1, %19 offset:%27\n\t"
      "ds_read_b32 %2, %20 offset:%27\n\t"
      "ds_read_b32 %3, %21 offset:%27\n\t"
      "ds_read_b32 %4, %22 offset:%27\n\t"
      "ds_read_b32 %5, %22 offset:%27+64\n\t"
      "ds_read_b32 %6, %22 offset:%27+128\n\t"
      "ds_read_b32 %7, %22 offset:%27+192\n\t"
      "ds_read_b128 %8, %23 offset:%27\n\t"
      "ds_read_b128 %9, %23 offset:%27+16\n\t"
      "ds_read_b128 %10, %23 offset:%27+32\n\t"
      "ds_read_b128 %11, %23 offset:%27+48\n\t"
      "ds_read_b32 %12, %24 offset:%27\n\t"
      "ds_read_b32 %13, %24 offset:%27+16\n\t"
      "ds_read_b32 %14, %24 offset:%27+32\n\t"
      "ds_read_b32 %15, %24 offset:%27+48\n\t"
      "ds_read_b32 %16, %25 offset:%27\n\t"
      "ds_read_b32 %17, %26\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.k[2]), "=&v"(s.k[3]), "=&v"(s.v[0]),
        "=&v"(s.v[1]), "=&v"(s.v[2]), "=&v"(s.v[3]), "=&v"(s.ksz[0]), "=&v"(s.ksz[1]),
        "=&v"(s.ksz[2]), "=&v"(s.ksz[3]), "=&v"(s.vsz[0]), "=&v"(s.vsz[1]), "=&v"(s.vsz[2]),
        "=&v"(s.vsz[3]), "=&v"(s.kz), "=&v"(pid)
      : "v"(kaddr[0]), "v"(kaddr[1]), "v"(kaddr[2]), "v"(kaddr[3]), "v"(vaddr), "v"(kszaddr),
        "v"(vszaddr), "v"(kzaddr), "v"(pidaddr), "i"(ST)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}

// D = 128 with four kv-heads per workgroup sharing each stage (see the
// kernel): as read_stage, but the four V rows sit at four addresses and a
// token's (scale, zero) rows are 64 bytes apart.
template <int ST>
__device__ __forceinline__ int32_t read_stage_shared(const uint32_t (&kaddr)[4],
                                                     const uint32_t (&vaddr)[4], uint32_t kszaddr,
                                                     uint32_t vszaddr, uint32_t kzaddr,
                                                     uint32_t pidaddr, StageData<128>& s) {
  int32_t pid;
  asm volatile(
      "ds_read_b32 %0, %18 offset:%30\n\t"
      "ds_read_b32 %1, %19 offset:%30\n\t"
      "ds_read_b32 %2, %20 offset:%30\n\t"
      "ds_read_b32 %3, %21 offset:%30\n\t"
      "ds_read_b32 %4, %22 offset:%30\n\t"
      "ds_read_b32 %5, %23 offset:%30\n\t"
      "ds_read_b32 %6, %24 offset:%30\n\t"
      "ds_read_b32 %7, %25 offset:%30\n\t"
      "ds_read_b128 %8, %26 offset:%30\n\t"
      "ds_read_b128 %9, %26 offset:%30+64\n\t"
      "ds_read_b128 %10, %26 offset:%30+128\n\t"
      "ds_read_b128 %11, %26 offset:%30+192\n\t"
      "ds_read_b32 %12, %27 offset:%30\n\t"
      "ds_read_b32 %13, %27 offset:%30+64\n\t"
      "ds_read_b32 %14, %27 offset:%30+128\n\t"
      "ds_read_b32 %15, %27 offset:%30+192\n\t"
      "ds_read_b32 %16, %28 offset:%30\n\t"
      "ds_read_b32 %17, %29\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s.k[0]), "=&v"(s.k[1]), "=&v"(s.k[2]), "=&v"(s.k[3]), "=&v"(s.v[0]),
        "=&v"(s.v[1]), "=&v"(s.v[2]), "=&v"(s.v[3]), "=&v"(s.ksz[0]), "=&v"(s.ksz[1]),
        "=&v"(s.ksz[2]), "=&v"(s.ksz[3]), "=&v"(s.vsz[0]), "=&v"(s.vsz[1]), "=&v"(s.vsz[2]),
        "=&v"(s.vsz[3]), "=&v"(s.kz), "=&v"(pid)
      : "v"(kaddr[0]), "v"(kaddr[1]), "v"(kaddr[2]), "v"(kaddr[3]), "v"(vaddr[0]), "v"(vaddr[1]),
        "v"(vaddr[2]), "v"(vaddr[3]), "v"(kszaddr), "v"(vszaddr), "v"(kzaddr), "v"(pidaddr),
        "i"(ST)
      : "memory");
  return __builtin_amdgcn_readfirstlane(pid);
}

struct MfmaArgs {
  const void* q;  // bf16 or fp32
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* ksz;
  const uint8_t* vsz;
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

// NT row tiles of 16 query rows (NT * 16 rows per workgroup): the K codes and
// the dequantised V of a tile are formed once and serve every row tile.
// One tile fits three workgroups per CU, two tiles two.  POLICY: the cache
// policy of the scale stream, and of the code stream with one kv-head per
// workgroup.  Non-temporal in the head-major layout, where every cache line
// belongs to one kv-head's workgroup; the default in the token-major one,
// where a code row (64 or 32 bytes) and a scale row (16 or 8) share their
// lines with the neighbouring kv-heads' rows, which other waves read moments
// later.  HQ: kv-heads per workgroup.  HQ = 1: the four waves share one
// kv-head and take its tiles in turn.  HQ = 4 (token-major pools, kv-heads
// 4g' .. 4g' + 3): wave w computes kv-head 4g' + w over every tile of the
// split, and the waves fill one LDS ring together (SHARED): a stage holds
// the tile of all four heads, wave w fetching its tokens 4w .. 4w + 3, whose
// four code rows are contiguous, so every code line is requested whole by
// one instruction and streams non-temporal; the (scale, zero) rows fill half
// of each line, whose other half the workgroup of the other four kv-heads
// reads (default policy).  Each wave waits for its own part of a tile, then
// the waves meet at a barrier before reading it.
template <int D, int NT, int POLICY, bool QF, int HQ>  // QF: fp32 Q
__global__ __launch_bounds__(kThreads, NT == 1 ? 3 : 2) void split_int4_mfma_kernel(const MfmaArgs a) {
  static_assert(HQ == 1 || HQ == kWaves, "one kv-head per workgroup or one per wave");
  using Gm = Geo<D>;
  constexpr int kD = D, kGroups = Gm::kGroups, kBlocks = Gm::kBlocks, kStages = Gm::kStages;
  constexpr int kStageK = Gm::kStageK, kStageV = Gm::kStageV, kStageKsz = Gm::kStageKsz;
  constexpr int kStageVsz = Gm::kStageVsz, kStageBytes = Gm::kStageBytes;
  constexpr int kRingBytes = Gm::kRingBytes;
  // four kv-heads per workgroup: the waves fill one ring together (SHARED
  // below), a stage holding all four heads' tile
  constexpr bool SHARED = HQ > 1;
  constexpr int kStageStride = SHARED ? kWaves * kStageBytes : kStageBytes;
  constexpr int ROWS = 16 * NT;
  constexpr int kEpiBytes = (kWaves * ROWS * kD + 2 * kWaves * ROWS) * 4;
  constexpr int kMainBytes = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMainBytes + kMaxSplitPages * 4];
  int32_t* s_pid = reinterpret_cast<int32_t*>(smem + kMainBytes);
  __shared__ int s_redo;         // a wave's V operand left fp16's range
  __shared__ float s_vmax[kWaves];

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


  // ---- Q^T operands (row tile rt, row lm): for MFMA kb, elements
  // 32*kb + 8*lg + e, e = 0..7, scaled by 2^sh and held in fp16
  uint32_t qv[NT][kGroups][4];  // [rt][kb][register]
  uint32_t ql[NT][QF ? kGroups : 1][4];  // fp32 Q: the lo terms
  float rowfac[NT];       // score (log2 units) = rowfac * sum_g s_g (dot_g - z_g qsum_g)
  float qsum_lg[NT];      // qsum of group lg: operand of the zero-point product
  int tlim[NT];           // tokens t < tlim are visible to this lane's row
  int lim_live = t1;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const bool live = 16 * rt + lm < nr;
    const int r = r0 + (live ? 16 * rt + lm : 0);  // this lane's query row of the kv-head
    float qsum[kGroups];  // 2^-24 * sum of the row's scaled fp16 Q over group kb
    const int i = r / a.G, h = g * a.G + r % a.G;
    const long long qoff = (((long long)b * a.qn + i) * a.Hq + h) * kD + 8 * lg;
    float qf[kGroups][8];
#pragma unroll
    for (int kb = 0; kb < kGroups; ++kb) {
      load_q8<QF>(a.q, qoff + 32 * kb, qf[kb]);  // 8 elements at 32*kb + 8*lg
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kb][e] = live ? qf[kb][e] : 0.f;
    }
    float mx = 0.f;
#pragma unroll
    for (int kb = 0; kb < kGroups; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qf[kb][e]));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const int sh = q_row_shift(mx);
#pragma unroll
    for (int kb = 0; kb < kGroups; ++kb) {
      float part = 0.f, lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = ldexpf(qf[kb][e], sh);
        qf[kb][e] = (float)(_Float16)y;
        part += qf[kb][e];
        if constexpr (QF) {
          lo[e] = (float)(_Float16)(y - qf[kb][e]);
          part += lo[e];
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // pairs 1 and 3 meet codes that sit 4 bits up (16 n), see the K operand
        const float f = (x & 1) ? 0.0625f : 1.f;
        qv[rt][kb][x] = pack_h2(qf[kb][x] * f, qf[kb][x + 4] * f);
        if constexpr (QF) ql[rt][kb][x] = pack_h2(lo[x] * f, lo[x + 4] * f);
      }
      part += xor16(part);
      part += xor32(part);
      qsum[kb] = ldexpf(part, -24);
    }
    rowfac[rt] = ldexpf(a.scale_log2, 24 - sh);
    qsum_lg[rt] = qsum[0];
#pragma unroll
    for (int kb = 1; kb < kGroups; ++kb) qsum_lg[rt] = lg == kb ? qsum[kb] : qsum_lg[rt];
    if (kGroups < 4 && lg >= kGroups) qsum_lg[rt] = 0.f;  // no such group
    tlim[rt] = live ? min(t1, a.causal ? L - (a.qn - 1 - i) : L) : 0;
    if (live) lim_live = min(lim_live, tlim[rt]);
  }
  // tiles below every live row's limit need no masks (rows past the block
  // have tlim 0 and are never written, so they do not bound the unmasked region)
  int tfull;
  {
    for (int o = 1; o < 16; o <<= 1) lim_live = min(lim_live, __shfl_xor(lim_live, o, 64));
    tfull = __builtin_amdgcn_readfirstlane(lim_live);
  }

  float4_t acc[NT][kBlocks];
  // zacc[rt]: -sum_t P_t z_t s_t for the lane's d-rows (one quantisation group
  // per d-row, the same in every output block); added to acc at the end
  float4_t zacc[NT];
  float m[NT], l[NT];
  auto reset_state = [&]() {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
      for (int bb = 0; bb < kBlocks; ++bb) acc[rt][bb] = {0.f, 0.f, 0.f, 0.f};
      zacc[rt] = {0.f, 0.f, 0.f, 0.f};
      m[rt] = da::kNegInf;
      l[rt] = 0.f;
    }
  };
  reset_state();
  // V is formed as v * 2^-vexp: 0 on the first pass, raised only when that
  // pass overflowed fp16 (see the end of the split)
  int vexp = 0;
  half2_t vdown = {1, 1};
  // fp16 exponent bits of 1024 in both halves, kept in a register so that
  // mask-and-or is one instruction
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));

  // ---- addressing
  constexpr int kRow = Gm::kRowBytes, kSz = Gm::kSzBytes;
  const long long rowb = (long long)a.slot_stride * kRow;  // bytes between slots (codes)
  const long long szb = (long long)a.slot_stride * kSz;    // (scale/zero)
  uint32_t voff_kv, voff_sz;
  const uint8_t* code_base = a.k;  // the tensor this lane's code DMA reads
  const uint8_t* sz_base = a.ksz;
  if constexpr (SHARED && D == 64) {
    // wave w fetches tokens 4w .. 4w + 3 of the tile for all four kv-heads,
    // whose rows of a token are contiguous (128 code bytes: one line; 32
    // scale bytes): lanes 0..31 the K codes, 32..63 the V codes, and one DMA
    // likewise for the (scale, zero) rows.  In LDS wave w's K codes (512 B)
    // and V codes (512 B) follow each other, a token's four code rows one
    // 128-byte row, kv-head h of token t in slot (h + t/4) mod 4 with its two
    // 16-byte groups rotated by (t/2) mod 2; after the four waves' codes, the
    // waves' K and V (scale, zero) rows (128 B each), a token's four in 32
    // bytes, kv-head h in slot (h + t/4) mod 4.  DMA lane i fills 16-byte
    // position i % 8 (codes) or dword i % 8 (scales) of token 4w + (i % 32)/8.
    const int li = lane & 31, t = 4 * wave + (li >> 3), pos = li & 7;
    const int hk = ((pos >> 1) - (t >> 2)) & 3, ck = ((pos & 1) - ((t >> 1) & 1)) & 1;
    voff_kv = (uint32_t)(t * rowb + kRow * hk + 16 * ck);
    voff_sz = (uint32_t)(t * szb + kSz * hk + 4 * (pos & 1));
    if (lane >= 32) {
      code_base = a.v;
      sz_base = a.vsz;
    }
  } else if constexpr (SHARED) {
    // wave w fetches tokens 4w .. 4w + 3 of the tile for all four kv-heads,
    // whose rows of a token are contiguous (256 code bytes, 64 scale bytes):
    // every 128-byte line is requested whole by one instruction.  In LDS a
    // token's four code rows fill one 256-byte row, kv-head h of token t in
    // slot (h + t + t/4) mod 4 with its 16-byte groups rotated by t/4; its
    // four (scale, zero) rows one 64-byte row, kv-head h in slot
    // (h + t/4) mod 4.  DMA lane i fills 16-byte position i % 16 (codes) or
    // dword i % 16 (scales) of token 4w + i/16.
    const int t = 4 * wave + (lane >> 4), pos = lane & 15;
    const int hk = ((pos >> 2) - t - (t >> 2)) & 3, ck = ((pos & 3) - (t >> 2)) & 3;
    voff_kv = (uint32_t)(t * rowb + kRow * hk + 16 * ck);
    const int hs = ((pos >> 2) - (t >> 2)) & 3;
    voff_sz = (uint32_t)(t * szb + kSz * hs + 4 * (pos & 3));
  } else if constexpr (D == 128) {
    // DMA lane i fills LDS chunk i (token i/4, position i%4) with the token's
    // 16-byte group (position - token/4) mod 4
    voff_kv = (uint32_t)((lane >> 2) * rowb + 16 * (((lane & 3) - (lane >> 4)) & 3));
    voff_sz = (uint32_t)((lane >> 2) * szb + 4 * (lane & 3));
  } else {
    // one DMA per tile for the codes: lanes 0..31 fill the K tile, 32..63
    // the V tile; lane i fills chunk i % 32 of it (row slot r = (i % 32) / 2,
    // position i % 2) with chunk (position - rot) mod 2 of token slot(r);
    // likewise one for the (scale, zero) rows, token (i % 32) / 2, group i % 2
    const int li = lane & 31, r = li >> 1, t = Gm::slot(r);
    voff_kv = (uint32_t)(t * rowb + 16 * (((li & 1) - Gm::rot(t)) & 1));
    voff_sz = (uint32_t)((li >> 1) * szb + 4 * (li & 1));
    if (lane >= 32) {
      code_base = a.v;
      sz_base = a.vsz;
    }
  }
  DA_LDS uint8_t* ring = (DA_LDS uint8_t*)smem + (SHARED ? 0 : wave * (kStages * kStageBytes));
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const uint32_t pid_lds = (uint32_t)(uintptr_t)(DA_LDS void*)s_pid;
  uint32_t rd_k[kGroups];
  uint32_t rd_v[SHARED && D == 128 ? 4 : D == 128 ? 1 : 2];
  uint32_t rd_ksz, rd_kz, rd_vsz;
  // shared stage, D = 128: K 4 KB, V 4 KB, then the two 1 KB (scale, zero)
  // tiles; D = 64: [K 512 B, V 512 B] per wave, then [K, V (scale, zero) 128
  // B each] per wave
  constexpr int kShV = 16 * 4 * kRow, kShKsz = 2 * kShV, kShVsz = kShKsz + 16 * 4 * kSz;
  constexpr int kSh64Sz = 4 * 1024;
  if constexpr (SHARED && D == 64) {
    const int h = wave;  // this wave's kv-head within the workgroup's four
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)  // token lm, group kb, dword lg
      rd_k[kb] = 1024 * (lm >> 2) + 128 * (lm & 3) + kRow * ((h + (lm >> 2)) & 3) +
                 16 * ((kb + ((lm >> 1) & 1)) & 1) + 4 * lg;
#pragma unroll
    for (int x = 0; x < 2; ++x)  // token 4 lg + 2x (+1 at 128 bytes), dword lm / 2
      rd_v[x] = 1024 * lg + 512 + 128 * (2 * x) + kRow * ((h + lg) & 3) +
                16 * (((lm >> 3) + x) & 1) + 4 * ((lm >> 1) & 3);
    rd_ksz = kSh64Sz + 256 * lg + kSz * ((h + lg) & 3);  // tokens 4 lg + i at 32 i
    rd_kz = kSh64Sz + 256 * (lm >> 2) + 32 * (lm & 3) + kSz * ((h + (lm >> 2)) & 3) + 4 * (lg & 1);
    rd_vsz = kSh64Sz + 128 + 256 * lg + kSz * ((h + lg) & 3) + 4 * (lm >> 3);
  } else if constexpr (SHARED) {
    const int h = wave;  // this wave's kv-head within the workgroup's four
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      rd_k[kb] = 4 * kRow * lm + kRow * ((h + lm + (lm >> 2)) & 3) + 16 * ((kb + (lm >> 2)) & 3) +
                 4 * lg;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)  // token 4 lg + jj, dword lm
      rd_v[jj] = kShV + 4 * kRow * (4 * lg + jj) + kRow * ((h + jj + lg) & 3) +
                 16 * (((lm >> 2) + lg) & 3) + 4 * (lm & 3);
    rd_ksz = kShKsz + 4 * kSz * (4 * lg) + kSz * ((h + lg) & 3);
    rd_kz = kShKsz + 4 * kSz * lm + kSz * ((h + (lm >> 2)) & 3) + 4 * lg;
    rd_vsz = kShVsz + 4 * kSz * (4 * lg) + kSz * ((h + lg) & 3) + 4 * (lm >> 2);
  } else if constexpr (D == 128) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) rd_k[kb] = kStageK + 64 * lm + 16 * ((kb + (lm >> 2)) & 3) + 4 * lg;
    rd_v[0] = kStageV + 64 * (4 * lg) + 16 * (((lm >> 2) + lg) & 3) + 4 * (lm & 3);
    rd_ksz = kStageKsz + 64 * lg;
    rd_kz = kStageKsz + 16 * lm + 4 * lg;
    rd_vsz = kStageVsz + 16 * (4 * lg) + 4 * (lm >> 2);
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      rd_k[kb] = kStageK + kRow * Gm::slot(lm) + 16 * ((kb + Gm::rot(lm)) & 1) + 4 * lg;
#pragma unroll
    for (int x = 0; x < 2; ++x) {  // tokens 4*lg + 2x (+1 at 128 bytes: slot + 4)
      const int t = 4 * lg + 2 * x;
      rd_v[x] = kStageV + kRow * Gm::slot(t) + 16 * (((lm >> 3) + Gm::rot(t)) & 1) +
                4 * ((lm >> 1) & 3);
    }
    rd_ksz = kStageKsz + 32 * lg;
    rd_kz = kStageKsz + 8 * lm + 4 * (lg & 1);
    rd_vsz = kStageVsz + 32 * lg + 4 * (lm >> 3);
  }

  auto tile_base = [&](int j) { return c0 + ((toff + tstep * j) << 4); };
  auto pid_addr = [&](int j) { return pid_lds + 4 * ((tile_base(j) >> a.log2_ps) - pc); };
  // shared stage: the workgroup's first kv-head, and this wave's part of it
  const int g_dma = SHARED ? HQ * it.g : g;
  const int dst_kv = SHARED ? 1024 * wave : 0,
            dst_sz = !SHARED ? 0 : D == 128 ? 256 * wave : kSh64Sz + 256 * wave;
  auto issue = [&](int j, int pid) {
    const int tb = tile_base(j);
    const long long row0 = (long long)pid * ps * a.Hkv + (long long)(tb & (ps - 1)) * a.slot_stride +
                           (long long)g_dma * a.head_stride;
    DA_LDS uint8_t* st = ring + (j % kStages) * kStageStride;
    if constexpr (SHARED && D == 64) {
      __builtin_amdgcn_global_load_lds((const void*)(code_base + row0 * kRow + voff_kv),
                                       (DA_LDS void*)(st + dst_kv), 16, 0, da::kStreamPolicy);
      __builtin_amdgcn_global_load_lds((const void*)(sz_base + row0 * kSz + voff_sz),
                                       (DA_LDS void*)(st + dst_sz), 4, 0, POLICY);
    } else if constexpr (SHARED) {
      __builtin_amdgcn_global_load_lds((const void*)(a.k + row0 * (kD / 2) + voff_kv),
                                       (DA_LDS void*)(st + dst_kv), 16, 0, da::kStreamPolicy);
      __builtin_amdgcn_global_load_lds((const void*)(a.v + row0 * (kD / 2) + voff_kv),
                                       (DA_LDS void*)(st + kShV + dst_kv), 16, 0, da::kStreamPolicy);
      __builtin_amdgcn_global_load_lds((const void*)(a.ksz + row0 * 16 + voff_sz),
                                       (DA_LDS void*)(st + kShKsz + dst_sz), 4, 0, POLICY);
      __builtin_amdgcn_global_load_lds((const void*)(a.vsz + row0 * 16 + voff_sz),
                                       (DA_LDS void*)(st + kShVsz + dst_sz), 4, 0, POLICY);
    } else if constexpr (D == 128) {
      __builtin_amdgcn_global_load_lds((const void*)(a.k + row0 * (kD / 2) + voff_kv),
                                       (DA_LDS void*)(st + kStageK), 16, 0, POLICY);
      __builtin_amdgcn_global_load_lds((const void*)(a.v + row0 * (kD / 2) + voff_kv),
                                       (DA_LDS void*)(st + kStageV), 16, 0, POLICY);
      __builtin_amdgcn_global_load_lds((const void*)(a.ksz + row0 * 16 + voff_sz),
                                       (DA_LDS void*)(st + kStageKsz), 4, 0, POLICY);
      __builtin_amdgcn_global_load_lds((const void*)(a.vsz + row0 * 16 + voff_sz),
                                       (DA_LDS void*)(st + kStageVsz), 4, 0, POLICY);
    } else {
      __builtin_amdgcn_global_load_lds((const void*)(code_base + row0 * kRow + voff_kv),
                                       (DA_LDS void*)(st + kStageK), 16, 0, POLICY);
      __builtin_amdgcn_global_load_lds((const void*)(sz_base + row0 * kSz + voff_sz),
                                       (DA_LDS void*)(st + kStageKsz), 4, 0, POLICY);
    }
  };

  auto compute = [&](int j, const StageData<D>& sd, auto masked_tag, auto scaled_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool SCALED = decltype(scaled_tag)::value;  // V scaled by 2^-vexp
    // ---- K operands, shared by the row tiles: elements (x, x+4) are nibble x
    // of the dword's two halves; pairs 1 and 3 are masked in place
    // (16 n * 2^-24, exact), their Q is / 16
    half8_t ka[kGroups];
#pragma unroll
    for (int kb = 0; kb < kGroups; ++kb) {
      const uint32_t w = sd.k[kb], wh = w >> 8;
      const half2_t k0 = as_h2(w & 0x000F000Fu), k1 = as_h2(w & 0x00F000F0u);
      const half2_t k2 = as_h2(wh & 0x000F000Fu), k3 = as_h2(wh & 0x00F000F0u);
      ka[kb] = half8_t{k0[0], k0[1], k1[0], k1[1], k2[0], k2[1], k3[0], k3[1]};
    }
    // -s z of token lm, group lg: the A operand of the zero-point product
    // (0, as is its B operand qsum_lg, for a group past D)
    float nsz = -(h_lo(sd.kz) * h_hi(sd.kz));
    if (kGroups < 4 && lg >= kGroups) nsz = 0.f;
    const int tb = tile_base(j) + 4 * lg;
    half4_t pb[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      // ---- zero-point terms: zt[i] = -sum_g s_g z_g qsum_g for token 4*lg + i,
      // row lm of tile rt (B: qsum of group lg, row lm)
      const float4_t zt = __builtin_amdgcn_mfma_f32_16x16x4f32(nsz, qsum_lg[rt],
                                                              float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      // ---- per-group dot products of the raw codes: dot[kb][i] =
      // 2^-24 * sum_{d in group kb} q'_d n_d for token 4*lg + i, row lm
      float4_t dot[kGroups];
#pragma unroll
      for (int kb = 0; kb < kGroups; ++kb) {
        const half2_t q0 = as_h2(qv[rt][kb][0]), q1 = as_h2(qv[rt][kb][1]);
        const half2_t q2 = as_h2(qv[rt][kb][2]), q3 = as_h2(qv[rt][kb][3]);
        const half8_t qb = {q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
        dot[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[kb], qb, float4_t{0.f, 0.f, 0.f, 0.f},
                                                         0, 0, 0);
        if constexpr (QF) {
          const half2_t l0 = as_h2(ql[rt][kb][0]), l1 = as_h2(ql[rt][kb][1]);
          const half2_t l2 = as_h2(ql[rt][kb][2]), l3 = as_h2(ql[rt][kb][3]);
          const half8_t lb = {l0[0], l0[1], l1[0], l1[1], l2[0], l2[1], l3[0], l3[1]};
          dot[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[kb], lb, dot[kb], 0, 0, 0);
        }
      }
      float4_t st;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc_s = zt[i];
#pragma unroll
        for (int kb = 0; kb < kGroups; ++kb) acc_s = fmaf(h_lo(sd.ksz[i][kb]), dot[kb][i], acc_s);
        st[i] = acc_s;
      }
      // st[i] = score of token 4*lg + i for row lm
      float z[4];
      bool need = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = fmaf(st[i], rowfac[rt], kPScale - m[rt]);
        if (MASKED && !(tb + i < tlim[rt])) z[i] = da::kNegInf;
        need |= z[i] > kRescaleSlack + kPScale;
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
        float sabs[4], mx = da::kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sabs[i] = (!MASKED || tb + i < tlim[rt]) ? st[i] * rowfac[rt] : da::kNegInf;
          mx = fmaxf(mx, sabs[i]);
        }
        mx = fmaxf(mx, xor16(mx));
        mx = fmaxf(mx, xor32(mx));
        const float mn = fmaxf(m[rt], mx);
        const float al = mn == da::kNegInf ? 1.f : da::fast_exp2(m[rt] - mn);
        l[rt] *= al;
#pragma unroll
        for (int bb = 0; bb < kBlocks; ++bb) acc[rt][bb] *= al;
        zacc[rt] *= al;
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

    // ---- V operand: tokens 4*lg + j, d = (D/16)*lm + block
    // rows past the split end may hold anything (even NaN scales): give them
    // code 0, scale 0, zero 0, i.e. the value 0
    uint32_t vw[4], vsz[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool ok = !MASKED || tb + jj < t1;
      vw[jj] = ok ? sd.v[jj] : 0u;
      vsz[jj] = ok ? sd.vsz[jj] : 0u;
    }
    // per token pair: s and -z*s (fp16, one per token); on the scaled pass
    // s * 2^-vexp (exact unless it falls below fp16's normal range)
    half2_t s01 = as_h2(__builtin_amdgcn_perm(vsz[1], vsz[0], 0x05040100u));
    half2_t s23 = as_h2(__builtin_amdgcn_perm(vsz[3], vsz[2], 0x05040100u));
    if constexpr (SCALED) {
      s01 = s01 * vdown;
      s23 = s23 * vdown;
    }
    const half2_t nzs01 = -(as_h2(__builtin_amdgcn_perm(vsz[1], vsz[0], 0x07060302u)) * s01);
    const half2_t nzs23 = -(as_h2(__builtin_amdgcn_perm(vsz[3], vsz[2], 0x07060302u)) * s23);
    // the zero-point term of every d-row of the lane's group: one product
    {
      const half4_t za = {nzs01[0], nzs01[1], nzs23[0], nzs23[1]};
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
        zacc[rt] = __builtin_amdgcn_mfma_f32_16x16x16f16(za, pb[rt], zacc[rt], 0, 0, 0);
    }
    // n s from the code t = 1024 + n: fma(t, s, -1024 s), one rounding (1024 s
    // is exact in fp16 while |s| < 64; a larger scale overflows it and the
    // split takes the scaled pass).  A high nibble is taken in place as
    // t = 1024 + 16 n, which gives 16 n s; its output blocks (odd bb) are
    // divided by 16 when the pass ends.
    const half2_t o01 = s01 * half2_t{-1024, -1024}, o23 = s23 * half2_t{-1024, -1024};
#pragma unroll
    for (int kk = 0; kk < kBlocks / 2; ++kk) {
      // byte kk of each token's dword (D = 64: byte 2 (lm % 2) + kk, the
      // lane's half): [t0.byte, 0, t1.byte, 0]
      const uint32_t by = D == 128 ? (uint32_t)kk : (uint32_t)(2 * (lm & 1) + kk);
      const uint32_t sel = by | 0x0C00u | ((4 + by) << 16) | 0x0C000000u;
      const uint32_t x01 = __builtin_amdgcn_perm(vw[1], vw[0], sel);
      const uint32_t x23 = __builtin_amdgcn_perm(vw[3], vw[2], sel);
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int bb = 2 * kk + hi;
        // fp16 1024 + n (low nibble) or 1024 + 16 n (high nibble), exact
        const uint32_t mask = hi ? 0x00F000F0u : 0x000F000Fu;
        const half2_t t01 = as_h2((x01 & mask) | magic);
        const half2_t t23 = as_h2((x23 & mask) | magic);
        const half2_t a01 = __builtin_elementwise_fma(t01, s01, o01);
        const half2_t a23 = __builtin_elementwise_fma(t23, s23, o23);
        half4_t va = {a01[0], a01[1], a23[0], a23[1]};
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
          acc[rt][bb] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb[rt], acc[rt][bb], 0, 0, 0);
      }
    }
  };

  // the lanes' read positions inside stage 0; stage j % kStages adds a constant
  uint32_t ka[kGroups];
#pragma unroll
  for (int kb = 0; kb < kGroups; ++kb) ka[kb] = ring_lds + rd_k[kb];
  const uint32_t va = ring_lds + rd_v[0], ksza = ring_lds + rd_ksz, vsza = ring_lds + rd_vsz,
                 kza = ring_lds + rd_kz;
  const uint32_t va2 = ring_lds + rd_v[D == 128 ? 0 : 1];
  constexpr int kVsh = SHARED && D == 128 ? 4 : 1;
  uint32_t vsh[kVsh];
#pragma unroll
  for (int jj = 0; jj < kVsh; ++jj) vsh[jj] = ring_lds + rd_v[jj];
  // wait for tile j, read it (stage offset ST + off bytes), refill its stage
  auto step = [&](int j, StageData<D>& sd, uint32_t off, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    // HQ > 1: the waves (each its own kv-head, every wave the same number of
    // tiles) meet before each tile, so their reads of the lines they share
    // leave the CU together
    if constexpr (HQ > 1 && !SHARED) __builtin_amdgcn_s_barrier();
    // the tiles after j issued so far may stay in flight
    wait_tiles_ahead<Gm::kLoads, kStages - 2>(min(kStages - 2, nmine - 1 - j));
    // shared stage: every wave's part of tile j has landed, and every wave has
    // read tile j - 1, whose stage the issue below refills
    if constexpr (SHARED) __builtin_amdgcn_s_barrier();
    const int jn = min(j + kStages - 1, nmine - 1);
    int pid;
    if constexpr (SHARED && D == 64) {
      const uint32_t k2[2] = {ka[0] + off, ka[1] + off}, v2[2] = {va + off, va2 + off};
      pid = read_stage64<ST, 32>(k2, v2, ksza + off, vsza + off, kza + off, pid_addr(jn), sd);
    } else if constexpr (SHARED) {
      const uint32_t k4[4] = {ka[0] + off, ka[1] + off, ka[2] + off, ka[3] + off};
      const uint32_t v4[4] = {vsh[0] + off, vsh[1] + off, vsh[2] + off, vsh[3] + off};
      pid = read_stage_shared<ST>(k4, v4, ksza + off, vsza + off, kza + off, pid_addr(jn), sd);
    } else if constexpr (D == 128) {
      const uint32_t k4[4] = {ka[0] + off, ka[1] + off, ka[2] + off, ka[3] + off};
      pid = read_stage<ST>(k4, va + off, ksza + off, vsza + off, kza + off, pid_addr(jn), sd);
    } else {
      const uint32_t k2[2] = {ka[0] + off, ka[1] + off}, v2[2] = {va + off, va2 + off};
      pid = read_stage64<ST>(k2, v2, ksza + off, vsza + off, kza + off, pid_addr(jn), sd);
    }
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
      using C0 = std::integral_constant<int, 0>;
      int j = 0;
      {
        // unmasked tiles, kStages per trip so that each one's stage is a constant
        static_assert(kStages == 4, "one unrolled trip per ring cycle");
        using C1 = std::integral_constant<int, kStageStride>;
        using C2 = std::integral_constant<int, 2 * kStageStride>;
        using C3 = std::integral_constant<int, 3 * kStageStride>;
        for (; j + kStages <= jfull; j += kStages) {
          StageData<D> sd0, sd1, sd2, sd3;
          step(j, sd0, 0u, C0{});
          compute(j, sd0, std::false_type{}, sc);
          step(j + 1, sd1, 0u, C1{});
          compute(j + 1, sd1, std::false_type{}, sc);
          step(j + 2, sd2, 0u, C2{});
          compute(j + 2, sd2, std::false_type{}, sc);
          step(j + 3, sd3, 0u, C3{});
          compute(j + 3, sd3, std::false_type{}, sc);
        }
      }
      // the rest (fewer than kStages unmasked tiles; then the masked ones)
      for (; j < nmine; ++j) {
        StageData<D> sd;
        step(j, sd, (uint32_t)((j % kStages) * kStageStride), C0{});
        compute(j, sd, std::true_type{}, sc);
      }
    }
    // high-nibble blocks carry 16 n s; then the zero-point term
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int bb = 0; bb < kBlocks; ++bb)
        acc[rt][bb] = (bb & 1 ? acc[rt][bb] * 0.0625f : acc[rt][bb]) + zacc[rt];
  };
  run_split(std::false_type{});

  // ---- An fp16 V operand out of range (a scale of 64 or more, so that 1024 s
  // overflows, or z*s past 65504) leaves inf or NaN in the output sums.  Then
  // the split is computed again with V formed as v * 2^-vexp, vexp the
  // smallest power that brings the bound |s| * max(1024, 15 + |z|) of every
  // V group of the split below 2^15 (so 1024 s, n*s and z*s all stay in
  // range); the factor is taken out again when the partials are written.
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
    float vm = 0.f;
    const int32_t* ptrow = a.pt + (long long)b * a.pt_stride;
    // (HQ = 1: the workgroup's threads over the tokens; else each wave over its kv-head's)
    for (int t = p0 * ps + (HQ == 1 ? (int)threadIdx.x : lane); t < t1;
         t += HQ == 1 ? kThreads : 64) {
      const int pid0 = ptrow[t >> a.log2_ps];
      const int pid = (unsigned)pid0 < (unsigned)a.num_pages ? pid0 : 0;
      const long long row = (long long)pid * ps * a.Hkv + (long long)(t & (ps - 1)) * a.slot_stride +
                            (long long)g * a.head_stride;
      const uint32_t* sz = reinterpret_cast<const uint32_t*>(a.vsz + row * kSz);
#pragma unroll
      for (int k = 0; k < kGroups; ++k)
        vm = fmaxf(vm, fabsf(h_lo(sz[k])) * fmaxf(1024.f, 15.f + fabsf(h_hi(sz[k]))));
    }
    for (int o = 32; o > 0; o >>= 1) vm = fmaxf(vm, __shfl_xor(vm, o, 64));
    if (lane == 0) s_vmax[wave] = vm;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) vm = fmaxf(vm, s_vmax[w]);
    // |s| < 2^16 and |z| < 2^16, so the bound is below 2^33: vexp <= 18
    int ex = 33;
    if (vm <= 3.0e38f) (void)frexpf(vm, &ex);  // vm < 2^ex
    vexp = __builtin_amdgcn_readfirstlane(min(max(ex - 15, 0), 18));
    vdown = half2_t{(_Float16)ldexpf(1.f, -vexp), (_Float16)ldexpf(1.f, -vexp)};
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
                                    s, kPScale, a.o, a.lse, vexp);
  } else {  // every wave's state is its kv-head's whole split
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      write_partials<1, ROWS, D>(sm_acc + w * ROWS * kD, sm_m + w * ROWS, sm_l + w * ROWS, r0, nr,
                                 a.G, HQ * it.g + w, b, a.qn, a.Hq, a.sched.S, s, kPScale, a.o,
                                 a.lse, vexp);
  }
}

template <int D, bool QF>
void launch(const da_host::SplitCall& c, const MfmaArgs& a, int R) {
  const bool hnd = c.kv.slot == 1;  // head-major pool layout
  // token-major pools: four kv-heads per workgroup where they divide evenly
  const bool quad = !hnd && c.Hkv % kWaves == 0;
  const dim3 grid(quad ? (unsigned)da_host::stage1_grid((long long)(c.Hkv / kWaves) * c.nrb,
                                                         c.units, true)
                       : c.grid(true)),
      block(kThreads);
  constexpr int kNt = da::kStreamPolicy;
  if (R <= 16) {
    if (hnd) hipLaunchKernelGGL((split_int4_mfma_kernel<D, 1, kNt, QF, 1>), grid, block, 0, c.stream, a);
    else if (quad) hipLaunchKernelGGL((split_int4_mfma_kernel<D, 1, 0, QF, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_int4_mfma_kernel<D, 1, 0, QF, 1>), grid, block, 0, c.stream, a);
  } else {
    if (hnd) hipLaunchKernelGGL((split_int4_mfma_kernel<D, 2, kNt, QF, 1>), grid, block, 0, c.stream, a);
    else if (quad) hipLaunchKernelGGL((split_int4_mfma_kernel<D, 2, 0, QF, kWaves>), grid, block, 0, c.stream, a);
    else hipLaunchKernelGGL((split_int4_mfma_kernel<D, 2, 0, QF, 1>), grid, block, 0, c.stream, a);
  }
}

}  // namespace

// INT4 stage 1 on the matrix cores (D = 128 or 64, bf16 or fp32 Q), one row
// tile (up to 16 query rows per kv-head) or two (blocks of up to 32 rows, so
// that G * q in 17..32 forms each tile's operands once); -1 when the shape is
// not covered (the caller then reports the call as unsupported).
int32_t da_split_int4_mfma(const da_host::SplitCall& call) {
  if (call.D != 128 && call.D != 64) return -1;
  da_host::SplitCall c = call;
  if (c.rows > DA_MAX_ROWS) da_host::row_blocks(c.rows, 2 * DA_MAX_ROWS, c.nrb, c.rb_rows);
  const int G = c.Hq / c.Hkv, R = c.rb_rows;  // rows per block
  MfmaArgs a;
  a.q = c.q; a.k = (const uint8_t*)c.k; a.v = (const uint8_t*)c.v;
  a.ksz = (const uint8_t*)c.ks; a.vsz = (const uint8_t*)c.vs;
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
