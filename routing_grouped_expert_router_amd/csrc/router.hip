// Router logits on gfx950: logits[t, e] = sum_h x[t, h] * W_r[e, h] (+ bias[e]),
// fp32 accumulation (vllbc blog, routing section: one logit per expert per
// token; the bias of the synthetic workloads is added before selection).
//
// Two kernels, both with a fixed summation order (bit-reproducible):
//  * router_small (any E, fp32 or bf16 x): one workgroup per token and group of
//    up to 64 experts (one expert when T * E <= 1024, so that few tokens still
//    spread over many workgroups); thread i takes 8 consecutive h per 2048-wide stride and
//    keeps one partial sum per expert, then a wave butterfly and a fixed-order
//    sum over the four waves.  W_r rows are read from L2 by every workgroup.
//  * router_mfma (E > 64, bf16 x): a workgroup owns 16 experts x 16*MR tokens
//    (MR = 1, 2 or 4 picked so the grid has at least 256 workgroups);
//    its 16 waves split H, each runs v_mfma_f32_16x16x32_bf16 over its slice
//    with operands loaded straight to registers (next slice in flight), and
//    the 16 partial tiles are summed in wave order through LDS.
#include "router_dev.hpp"

namespace moe {

template <bool XF32, int EB>
__global__ __launch_bounds__(256) void router_small_kernel(RouterArgs a) {
  router_small_item<XF32, EB>(a, blockIdx.x, blockIdx.y);
}

template <int MR>
__global__ __launch_bounds__(kRouterWaves * 64) void router_mfma_kernel(RouterArgs a) {
  __shared__ f32x4 red[kRouterWaves][MR][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16 * MR;
  f32x4 acc[MR];
  router_mfma_slice<MR>(a, e0, t0, wave, acc);
#pragma unroll
  for (int m = 0; m < MR; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  router_mfma_store<MR>(a, e0, t0, red);
}

bool router_uses_mfma(int E, int H, int x_f32) { return E > 64 && !x_f32 && H % 1024 == 0; }

constexpr int kRouterOneExpertMax = 1024;   // T * E up to which each workgroup takes one expert

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (router_uses_mfma(a.E, a.H, a.x_f32)) {
    // 16*MR tokens per workgroup: the largest MR that still gives >= 256
    // workgroups (weights are re-read once per token block, activations once
    // per 16-expert block either way)
    const int eb = (a.E + 15) / 16;
    if ((int64_t)eb * ((a.T + 63) / 64) >= 256)
      hipLaunchKernelGGL(router_mfma_kernel<4>, dim3(eb, (a.T + 63) / 64), dim3(kRouterWaves * 64), 0, s, a);
    else if ((int64_t)eb * ((a.T + 31) / 32) >= 256)
      hipLaunchKernelGGL(router_mfma_kernel<2>, dim3(eb, (a.T + 31) / 32), dim3(kRouterWaves * 64), 0, s, a);
    else
      hipLaunchKernelGGL(router_mfma_kernel<1>, dim3(eb, (a.T + 15) / 16), dim3(kRouterWaves * 64), 0, s, a);
  } else if ((int64_t)a.T * a.E <= kRouterOneExpertMax) {
    // few tokens: one workgroup per (token, expert), so the W_r rows are read
    // in parallel (each expert's sum runs in the same order for any EB)
    const dim3 g(a.T, a.E), b(256);
    if (a.x_f32) hipLaunchKernelGGL((router_small_kernel<true, 1>), g, b, 0, s, a);
    else hipLaunchKernelGGL((router_small_kernel<false, 1>), g, b, 0, s, a);
  } else {
    const dim3 g(a.T, a.E > 32 ? (a.E + 63) / 64 : 1), b(256);
    if (a.x_f32) {
      if (a.E <= 8) hipLaunchKernelGGL((router_small_kernel<true, 8>), g, b, 0, s, a);
      else if (a.E <= 16) hipLaunchKernelGGL((router_small_kernel<true, 16>), g, b, 0, s, a);
      else if (a.E <= 32) hipLaunchKernelGGL((router_small_kernel<true, 32>), g, b, 0, s, a);
      else hipLaunchKernelGGL((router_small_kernel<true, 64>), g, b, 0, s, a);
    } else {
      if (a.E <= 8) hipLaunchKernelGGL((router_small_kernel<false, 8>), g, b, 0, s, a);
      else if (a.E <= 16) hipLaunchKernelGGL((router_small_kernel<false, 16>), g, b, 0, s, a);
      else if (a.E <= 32) hipLaunchKernelGGL((router_small_kernel<false, 32>), g, b, 0, s, a);
      else hipLaunchKernelGGL((router_small_kernel<false, 64>), g, b, 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
