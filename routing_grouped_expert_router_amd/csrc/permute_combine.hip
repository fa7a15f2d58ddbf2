// Gather into expert-grouped rows and the route-weighted combine, on gfx950.
//
// Both are row copies bound by HBM: one wave moves one H-wide row in 16-byte
// vectors, so every wave instruction touches 1 KiB of contiguous memory.
//
// permute (vllbc blog, vLLM forward path: tokens sorted into expert order;
//   MoonEP online plan: dispatch into expert-grouped slots):
//   xg[slot_of[t*K + k]] = x[t]  and  xg[shared_base + t] = x[t].
// combine (vllbc blog, combine: weight each expert output by g_i, then sum
//   the K results; the shared expert enters with weight 1):
//   out[t] = sum_k w[t, k] * y[slot_of[t*K + k]] + y[shared_base + t],
//   accumulated in fp32 with k ascending (then the shared row), K-split
//   partial planes of y summed in split order first.
#include "combine_dev.hpp"

namespace moe {

constexpr int kRowsPerBlock = 4;   // one wave per row

__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a) {
  const int64_t TK = (int64_t)a.T * a.K;
  const int64_t n = TK + (int64_t)a.n_shared * a.T;
  const int64_t i = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  int t;
  int64_t dst;
  if (i < TK) { t = int(i / a.K); dst = a.slot_of[i]; }
  else { t = int(i - TK); dst = a.shared_base + t; }
  if (dst < 0 || dst >= a.rows) return;
  const int nv = a.H / 8;
  u32x4* drow = reinterpret_cast<u32x4*>(a.xg + dst * a.H);
  if (a.act_f32) {
    const f32x4* srow = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + (int64_t)t * a.H);
    for (int v = lane; v < nv; v += kWave) {
      const f32x4 lo = srow[2 * v], hi = srow[2 * v + 1];
      u32x4 o = {pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                 pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)};
      drow[v] = o;
    }
  } else {
    const u32x4* srow = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + (int64_t)t * a.H);
    for (int v = lane; v < nv; v += kWave) drow[v] = srow[v];
  }
}

template <bool YF32>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int v = blockIdx.y * blockDim.x + threadIdx.x;
  if (v < a.H / 8) combine_vec<YF32>(a, blockIdx.x, v);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.T * a.K + (int64_t)a.n_shared * a.T;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3((n + kRowsPerBlock - 1) / kRowsPerBlock), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.splits > kMaxSplits || a.K > kMaxK) return hipErrorInvalidValue;
  const int nv = a.H / 8;
  const int threads = 64;                  // one wave per 512 features
  const dim3 grid(a.T, (nv + threads - 1) / threads);
  if (a.y_f32) hipLaunchKernelGGL((combine_kernel<true>), grid, dim3(threads), 0, s, a);
  else hipLaunchKernelGGL((combine_kernel<false>), grid, dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
