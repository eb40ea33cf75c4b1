// Stage 1 for a dense fp32 cache with fp32 Q and up to 4 query rows per
// kv-head (more go to split_f32_mfma.hip): the vector-ALU path of the GQA
// flash-decode stage 1 (LightLLM PR #1549, "Covered decode kernels"); the
// entry point that validates a call and picks its kernel is in stage1.cpp.
// The pipeline (lane layout, LDS-DMA ring, lazy softmax rescale) is
// split_vec_body in split_vec.h, shared with the bf16 cache's kernel; here
// the products are plain fp32 FMAs.
#include "split_vec.h"

namespace {

// LDS ring: STAGES stages of 2*CPL KB per wave (CPL = D/32 pieces of 128
// bytes per fp32 row).  D = 64 has the byte geometry of the bf16 kernel at
// D = 128 (4 stages, 64 KB, two workgroups per CU).  D = 128 stages are
// 8 KB: 2 stages (one tile in flight per wave, 64 KB of ring) keep two
// workgroups on a CU and measure a little faster than 4 stages with one
// workgroup per CU (B = 16, 8K tokens: 80-81 % of 8 TB/s against 76-82 %).
constexpr int FP32_D128_STAGES = 2;

// token-major pools take four kv-heads per workgroup at D = 64 (B = 16, 8K,
// G = 4: 87.6 -> 85.5 us; G = 1: 89.3 -> 85.8 us); D = 128 rows are 512
// bytes, and that head dim keeps one kv-head per workgroup
template <int D>
constexpr bool kQuadLayout = D == 64;

// two workgroups per CU where their LDS fits (160 KB per CU), else one
template <int D, int RT, int STAGES, int HQ>
__global__ __launch_bounds__(kThreads, (VecSmem<4, D, RT, STAGES>::BYTES <= 80 * 1024 ? 2 : 1))
void split_fma_kernel(const VecArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[VecSmem<4, D, RT, STAGES>::BYTES];
  split_vec_body<true, D, RT, STAGES, HQ>(a, smem);
}

template <int D, int RT>
int32_t launch(const VecArgs& a, const da_host::SplitCall& c, hipStream_t st) {
  constexpr int STAGES = D == 128 ? FP32_D128_STAGES : 4;
  if (kQuadLayout<D> && c.kv.slot != 1 && c.Hkv % kWaves == 0) {
    const unsigned grid =
        (unsigned)da_host::stage1_grid((long long)(c.Hkv / kWaves) * c.nrb, c.units, c.nrb > 1);
    hipLaunchKernelGGL((split_fma_kernel<D, RT, STAGES, kWaves>), dim3(grid), dim3(kThreads), 0, st,
                       a);
  } else {
    hipLaunchKernelGGL((split_fma_kernel<D, RT, STAGES, 1>), dim3(c.grid(false)), dim3(kThreads), 0,
                       st, a);
  }
  return da_host::launch_status();
}

template <int D>
int32_t launch_d(const VecArgs& a, const da_host::SplitCall& c, hipStream_t st) {
  if (a.R <= 1) return launch<D, 1>(a, c, st);
  if (a.R <= 2) return launch<D, 2>(a, c, st);
  return launch<D, 4>(a, c, st);
}

}  // namespace

// fp32 cache and fp32 Q with up to 4 query rows per row block on the vector
// ALU; -1 for any other shape (see da_split_f32_mfma for 5 or more rows).
int32_t da_split_f32_fma(const da_host::SplitCall& c) {
  if (c.q_bf16 || c.rb_rows > 4 || (c.D != 128 && c.D != 64)) return -1;
  const VecArgs a = make_vec_args(c);
  return c.D == 128 ? launch_d<128>(a, c, c.stream) : launch_d<64>(a, c, c.stream);
}
