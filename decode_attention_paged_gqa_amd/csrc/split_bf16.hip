// Stage 1 for a dense bf16 cache and small query groups (G*q <= 5): the
// vector-ALU path of the GQA flash-decode stage 1 (LightLLM PR #1549,
// "Covered decode kernels").  Same contract as decode_attn_split (entry
// point in stage1.cpp); built to stream K/V at HBM speed.  The pipeline
// (lane layout, LDS-DMA ring, lazy softmax rescale) is split_vec_body in
// split_vec.h, shared with the fp32 cache's kernel.
#include "split_vec.h"

namespace {

// token-major pools take four kv-heads per workgroup at D = 64, where a
// token's four neighbouring kv-head rows are 512 contiguous bytes (ragged
// G = 5 batch 246 -> 220 us); at D = 128 it measured slower on the ragged
// batch (423 -> 442 us), so that head dim keeps one kv-head per workgroup
template <int D>
constexpr bool kQuadLayout = D == 64;

// 4 LDS stages of 2*CPL KB per wave: 64 KB of ring at D = 128, so two
// workgroups share a CU
template <int D, int RT, int STAGES, int HQ>
__global__ __launch_bounds__(kThreads, 2) void split_bf16_kernel(const VecArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[VecSmem<2, D, RT, STAGES>::BYTES];
  split_vec_body<false, D, RT, STAGES, HQ>(a, smem);
}

template <int D, int RT>
int32_t launch(const VecArgs& a, const da_host::SplitCall& c, hipStream_t st) {
  // token-major pools: four kv-heads per workgroup where they divide evenly
  if (kQuadLayout<D> && c.kv.slot != 1 && c.Hkv % kWaves == 0) {
    const unsigned grid =
        (unsigned)da_host::stage1_grid((long long)(c.Hkv / kWaves) * c.nrb, c.units, c.nrb > 1);
    hipLaunchKernelGGL((split_bf16_kernel<D, RT, 4, kWaves>), dim3(grid), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((split_bf16_kernel<D, RT, 4, 1>), dim3(c.grid(false)), dim3(kThreads), 0, st,
                       a);
  }
  return da_host::launch_status();
}

}  // namespace

// Called by the split entry point after argument validation; returns -1
// when this kernel does not cover the shape (more than 5 rows per block:
// the caller then uses the matrix-core kernel).
int32_t da_split_bf16_fast(const da_host::SplitCall& c) {
  const int R = c.rb_rows, D = c.D;  // rows per block
  if (!c.q_bf16 || R > 5 || (D != 128 && D != 64)) return -1;
  const VecArgs a = make_vec_args(c);
  hipStream_t st = c.stream;
  if (D == 128) {
    switch (R) {
      case 1: return launch<128, 1>(a, c, st);
      case 2: return launch<128, 2>(a, c, st);
      case 3: case 4: return launch<128, 4>(a, c, st);
      default: return launch<128, 5>(a, c, st);
    }
  }
  switch (R) {
    case 1: return launch<64, 1>(a, c, st);
    case 2: return launch<64, 2>(a, c, st);
    case 3: case 4: return launch<64, 4>(a, c, st);
    default: return launch<64, 5>(a, c, st);
  }
}
