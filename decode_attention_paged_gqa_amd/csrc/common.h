// Shared device / host helpers of libdecode_attn (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_attn.h"

namespace da {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------- conversions
// bf16 is the upper half of an fp32 word, so widening is a shift / mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  _Float16 h;
  uint16_t b = (uint16_t)bits16;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t float_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// signed byte k (0..3) of a word, exactly as float
__device__ __forceinline__ float sbyte_to_float(uint32_t w, int k) {
  return (float)(int32_t)((int32_t)(w << (24 - 8 * k)) >> 24);
}

// ---------------------------------------------------------------- wave helpers
template <int MASK>
__device__ __forceinline__ float xor_shfl(float x) {
  return __shfl_xor(x, MASK, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cache policy of the stage-1 K/V (and scale) streams, the aux operand of
// global_load_lds: non-temporal (nt).  Each byte is read once per launch;
// marked so, it is not kept in the caches on its way, and a plain 4 GiB
// stream on MI355X reads at 81 % of 8 TB/s instead of 73 % (the stage-1
// kernels gain the same ~8 points).
constexpr int kStreamPolicy = 2;

// ---------------------------------------------------------------- contract checks
// Device data the host cannot see without a sync (page ids, lengths, batch
// order, work lists, split counts, request rows) is the caller's contract;
// kernels clamp it to in-bounds values.  A checked build (-DDA_CHECKED) also
// records every violation in the library's check words chk = [flag bits
// (DA_CHECK_*), count], read back by decode_attn_checks; an unchecked build
// compiles the checks away.  Either way the results are the same.
__device__ __forceinline__ void note(unsigned long long* chk, bool ok, unsigned bit) {
#ifdef DA_CHECKED
  if (!ok && chk) {
    atomicOr(chk, (unsigned long long)bit);
    atomicAdd(chk + 1, 1ull);
  }
#else
  (void)chk; (void)ok; (void)bit;
#endif
}

// ---------------------------------------------------------------- stage-1 work units
// Stage 1 runs one workgroup per (kv-head g, work unit u) on a 1-D grid.  A
// unit is one (request, split).  Without a work list, unit u = z * S + s is
// split s of the request in dispatch slot z (order[z] with a batch order,
// else z), every request having S splits.  With a work list (built by the
// metadata prelude from per-request split counts), unit u is the list's
// entry u = b * 256 + s, request b having counts[b] splits; -1 entries are
// padding.  Either way the partials keep S slots per query row.
//
// Workgroups reach the chip's 8 XCDs round-robin by linear id, and each XCD
// has its own L2.  Two orders of (g, u):
//  * spread: id = g + Hkv * u.  With Hkv a multiple of 8 every XCD gets one
//    kv-head of every unit, the best balance; used where a kv-head's rows
//    fill whole cache lines (dense caches).
//  * grouped: units are dealt to the XCDs in rounds of 8, in snake order
//    (round r sends unit 8r + j to XCD j for even r and to XCD 7 - j for odd
//    r, keeping a longest-first order balanced), and a unit's Hkv heads are
//    that XCD's next Hkv workgroups.  Short rows of neighbouring kv-heads
//    (4-bit and 8-bit codes, their scales) share cache lines; this way each
//    such line is brought into one L2, once, by workgroups that run side by
//    side.
// Units keep their order (longest requests first with a batch order or a
// work list).
//
// Row blocks: a kv-head serves R = G * q_per_req query rows.  A kernel holds
// at most 16 of them, so R > 16 is cut into nrb = ceil(R / 16) blocks of
// ceil(R / nrb) rows (the last may be shorter), and each (kv-head, block)
// pair is a workgroup of its own, as if it were a kv-head: the grid carries
// Hkv * nrb "heads".  Every block reads the kv-head's pages; the grouped
// order is then used for every kernel, which puts the nrb blocks of a
// kv-head on one XCD as consecutive workgroups, so the later blocks find the
// pages in that XCD's L2.
constexpr int kXcds = 8;
constexpr int kItemShift = 8;  // work item = b << 8 | s

struct Stage1Sched {
  unsigned long long* checks;  // contract-check words (checked builds; else null)
  const int32_t* order;   // nullable: batch order (no work list)
  const int32_t* work;    // nullable: work list of `units` entries
  const int32_t* counts;  // per-request split counts (with a work list)
  int S;                  // split slots per query row; the split count without a work list
  int B;                  // requests
  int units;              // S * B, or the work list's capacity
  int rows;               // R = G * q_per_req query rows per kv-head
  int nrb;                // row blocks per kv-head
  int rb_rows;            // rows per block (the last block may have fewer)
};

struct Stage1Item {
  int g, b, s, S;  // kv-head, request, split, the request's split count
  int r0, nr;      // this workgroup's query rows: r0 .. r0 + nr - 1 of the kv-head
};

// false for padding workgroups: the last round of the grouped order, -1
// entries of a work list, and entries that name no valid (request, split)
template <bool GROUPED>
__device__ __forceinline__ bool stage1_item(const Stage1Sched& sc, int Hkv, Stage1Item& it) {
  const int i = (int)blockIdx.x;
  const int Hv = Hkv * sc.nrb;  // (kv-head, row block) pairs
  int u, gv;
  if (!GROUPED && sc.nrb == 1) {
    u = i / Hv;
    gv = i - u * Hv;
  } else {
    const int x = i % kXcds, k = i / kXcds;
    const int r = k / Hv;
    u = r * kXcds + ((r & 1) ? kXcds - 1 - x : x);
    gv = k - r * Hv;
    if (u >= sc.units) return false;
  }
  it.g = gv / sc.nrb;
  it.r0 = (gv - it.g * sc.nrb) * sc.rb_rows;
  it.nr = min(sc.rb_rows, sc.rows - it.r0);  // >= 1 for every R <= 2^24 (entry check)
  if (it.nr <= 0) return false;
  const bool first = threadIdx.x == 0;  // one note per workgroup
  if (!sc.work) {
    const int z = u / sc.S;
    it.s = u - z * sc.S;
    const int b = sc.order ? sc.order[z] : z;
    note(sc.checks, !first || (unsigned)b < (unsigned)sc.B, DA_CHECK_ORDER);
    it.b = (unsigned)b < (unsigned)sc.B ? b : z;
    it.S = sc.S;
    return true;
  }
  const int item = sc.work[u];
  if (item < 0) return false;
  it.b = item >> kItemShift;
  it.s = item & ((1 << kItemShift) - 1);
  if (it.b >= sc.B) {
    note(sc.checks, !first, DA_CHECK_WORK);
    return false;
  }
  const int cnt = sc.counts[it.b];
  note(sc.checks, !first || (cnt >= 1 && cnt <= sc.S), DA_CHECK_COUNTS);
  it.S = min(max(cnt, 1), sc.S);
  note(sc.checks, !first || it.s < it.S, DA_CHECK_WORK);
  return it.s < it.S;
}

}  // namespace da

// ---------------------------------------------------------------- host side
namespace da_host {

inline int32_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DA_OK : DA_ERR_LAUNCH;
}

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool aligned(const void* p, unsigned bytes) { return ((uintptr_t)p & (bytes - 1)) == 0; }

// The current device's contract-check words (checked builds; null otherwise).
unsigned long long* check_words();

// Rows between consecutive slots and between consecutive kv-heads of a
// page, for the two pool layouts; a page is page_size * Hkv rows.  Row of
// (page p, slot t, head g) = p * page_size * Hkv + t * slot + g * head.
struct KvStrides {
  int slot, head;
};
inline bool kv_strides(int32_t kv_layout, int Hkv, int page_size, KvStrides& st) {
  if (kv_layout == DA_KV_NHD) {
    st.slot = Hkv;
    st.head = 1;
    return true;
  }
  if (kv_layout == DA_KV_HND) {
    st.slot = 1;
    st.head = page_size;
    return true;
  }
  return false;
}

// Everything a stage-1 launch needs, checked by the entry point; the
// specialised kernels take it whole and return -1 for shapes they do not
// cover (the entry point then tries the next one, or reports the call as
// unsupported).
struct SplitCall {
  const void* q;
  int q_bf16;
  const void* k;
  const void* v;
  const uint16_t* ks;  // scales (int8) or (scale, zero) pairs (int4); null for dense
  const uint16_t* vs;
  const int32_t* pt;
  int pt_stride, max_pages;
  const int32_t* seqlens;
  const int32_t* order;
  const int32_t* work;    // nullable: work list (then counts is required)
  const int32_t* counts;
  int units;              // grid units: S * batch, or the work list's capacity
  unsigned long long* checks;  // contract-check words (checked builds; else null)
  int batch, qn, Hq, Hkv, D, ps, num_pages, S;
  int rows, nrb, rb_rows;  // query rows per kv-head, row blocks, rows per block
  KvStrides kv;
  float scale;
  int causal;
  float* o;
  float* lse;
  hipStream_t stream;

  da::Stage1Sched sched() const {
    da::Stage1Sched sc;
    sc.checks = checks;
    sc.order = order; sc.work = work; sc.counts = counts;
    sc.S = S; sc.B = batch; sc.units = units;
    sc.rows = rows; sc.nrb = nrb; sc.rb_rows = rb_rows;
    return sc;
  }

  // grid of the launch for a kernel whose own order is `grouped` (see
  // da::stage1_item; row blocks always take the grouped order)
  unsigned grid(bool grouped) const;
};

// 1-D grid of stage 1 (see da::stage1_item) over `units` work units; the
// grouped order pads to whole rounds of 8 units
inline long long stage1_grid(long long heads, long long units, bool grouped) {
  if (!grouped) return units * heads;
  return da::kXcds * heads * ((units + da::kXcds - 1) / da::kXcds);
}

inline unsigned SplitCall::grid(bool grouped) const {
  return (unsigned)stage1_grid((long long)Hkv * nrb, units, grouped || nrb > 1);
}

// Row blocks of R query rows per kv-head, at most max_rows each (see
// da::stage1_item): ceil(R / max_rows) blocks of equal size but the last.
inline void row_blocks(int R, int max_rows, int& nrb, int& rb_rows) {
  nrb = (R + max_rows - 1) / max_rows;
  rb_rows = (R + nrb - 1) / nrb;
}

}  // namespace da_host
