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
#include "common.hpp"
#include "kernels.hpp"

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

__device__ __forceinline__ void add_bf16x8(float* acc, const u32x4 v, float w) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] += w * __uint_as_float(u[q] << 16);
    acc[2 * q + 1] += w * __uint_as_float(u[q] & 0xffff0000u);
  }
}

// the expert output row `slot` at vector v (8 values), K-split planes summed
__device__ __forceinline__ void load_y(const CombineArgs& a, int64_t slot, int v, float* y8) {
  if (a.y_f32) {
    const float* base = static_cast<const float*>(a.y) + slot * a.H + 8 * v;
#pragma unroll
    for (int q = 0; q < 8; ++q) y8[q] = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const f32x4* p = reinterpret_cast<const f32x4*>(base + s * a.split_stride);
      const f32x4 lo = p[0], hi = p[1];
      y8[0] += lo.x; y8[1] += lo.y; y8[2] += lo.z; y8[3] += lo.w;
      y8[4] += hi.x; y8[5] += hi.y; y8[6] += hi.z; y8[7] += hi.w;
    }
  } else {
    const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.y) + slot * a.H + 8 * v);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y8[2 * q] = __uint_as_float(w[q] << 16);
      y8[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  }
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int nv = a.H / 8;
  const int K = a.K;
  int64_t slots[kMaxK];
  float ws[kMaxK];
  for (int k = 0; k < K; ++k) {
    slots[k] = a.slot_of[(int64_t)t * K + k];
    ws[k] = a.topk_w[(int64_t)t * K + k];
  }
  for (int v = threadIdx.x; v < nv; v += blockDim.x) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int64_t s = slots[k];
      if (s < 0 || s >= a.rows) continue;
      float y8[8];
      load_y(a, s, v, y8);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += ws[k] * y8[q];
    }
    if (a.n_shared) {
      float y8[8];
      load_y(a, a.shared_base + t, v, y8);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += y8[q];
    }
    if (a.out_f32) {
      f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (int64_t)t * a.H + 8 * v);
      o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                 pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + (int64_t)t * a.H + 8 * v) = o;
    }
  }
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.T * a.K + (int64_t)a.n_shared * a.T;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3((n + kRowsPerBlock - 1) / kRowsPerBlock), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nv = a.H / 8;
  const int threads = nv >= 256 ? 256 : ((nv + 63) / 64) * 64;
  hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
