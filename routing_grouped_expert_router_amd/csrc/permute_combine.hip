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

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 u, float* y8) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    y8[2 * q] = __uint_as_float(w[q] << 16);
    y8[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}

constexpr int kMaxSplits = 8;

// out[t] for 8 consecutive features per thread.  All loads of a vector are
// issued before any is summed; the sums run k = 0..K-1 (each k over its K-split
// planes in split order), then the shared row.
template <bool YF32>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int v = blockIdx.y * blockDim.x + threadIdx.x;
  const int nv = a.H / 8;
  if (v >= nv) return;
  const int K = a.K;
  const int nk = K + a.n_shared;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  // Loads use clamped row indices and sit outside divergent branches, so all
  // of them are in flight together; an invalid slot (never expected) is
  // masked to zero after its load.
  if (YF32) {
    for (int k = 0; k < nk; ++k) {
      int64_t slot = k < K ? (int64_t)a.slot_of[(int64_t)t * K + k] : a.shared_base + t;
      const float w = k < K ? a.topk_w[(int64_t)t * K + k] : 1.0f;
      const bool ok = slot >= 0 && slot < a.rows;
      slot = ok ? slot : 0;
      const float* base = static_cast<const float*>(a.y) + slot * a.H + 8 * v;
      f32x4 lo[kMaxSplits], hi[kMaxSplits];
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp) {
        const int spc = sp < a.splits ? sp : 0;
        const f32x4* p = reinterpret_cast<const f32x4*>(base + spc * a.split_stride);
        lo[sp] = p[0]; hi[sp] = p[1];
      }
      float y8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp) {
        if (sp < a.splits) {
          y8[0] += lo[sp].x; y8[1] += lo[sp].y; y8[2] += lo[sp].z; y8[3] += lo[sp].w;
          y8[4] += hi[sp].x; y8[5] += hi[sp].y; y8[6] += hi[sp].z; y8[7] += hi[sp].w;
        }
      }
      if (!ok) continue;
      if (k < K) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += w * y8[q];
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += y8[q];
      }
    }
  } else {
    u32x4 yv[kMaxK + 1];
    float wk[kMaxK + 1];
    bool ok[kMaxK + 1];
#pragma unroll
    for (int k = 0; k < kMaxK + 1; ++k) {
      const int kc = k < nk ? k : 0;
      int64_t slot = kc < K ? (int64_t)a.slot_of[(int64_t)t * K + kc] : a.shared_base + t;
      wk[k] = kc < K ? a.topk_w[(int64_t)t * K + kc] : 1.0f;
      ok[k] = k < nk && slot >= 0 && slot < a.rows;
      slot = (slot >= 0 && slot < a.rows) ? slot : 0;
      yv[k] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.y) + slot * a.H + 8 * v);
    }
#pragma unroll
    for (int k = 0; k < kMaxK + 1; ++k) {
      if (ok[k]) {
        float y8[8];
        bf16x8_to_f32(yv[k], y8);
        if (k < K) {
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += wk[k] * y8[q];
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += y8[q];
        }
      }
    }
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
