// Router logits for fp32 activations (the tiny fp32 workload):
// logits[t, e] = sum_h x[t, h] * W_r[e, h] (+ bias[e]) in fp32, one wave per
// (token, expert), lanes striding over h, then a fixed-order wave reduction.
// (vllbc blog, routing section: one logit per expert per token.)
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void router_f32_kernel(RouterF32Args a) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* xr = a.x + (int64_t)t * a.H;
  for (int e = blockIdx.y * 4 + wave; e < a.E; e += gridDim.y * 4) {
    const uint16_t* wr = a.w + (int64_t)e * a.H;
    float s = 0.f;
    for (int h = lane; h < a.H; h += kWave) s += xr[h] * bf16_to_f32(wr[h]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
    if (lane == 0) a.logits[(int64_t)t * a.E + e] = s + (a.bias ? a.bias[e] : 0.f);
  }
}

hipError_t launch_router_f32(const RouterF32Args& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int gy = (a.E + 3) / 4 < 64 ? (a.E + 3) / 4 : 64;
  hipLaunchKernelGGL(router_f32_kernel, dim3(a.T, gy), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
