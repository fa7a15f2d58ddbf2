// Device function of the combine (one token's 8 output features), shared by
// the combine kernel and the persistent decode kernel.  The method is
// described in permute_combine.hip.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

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
__device__ __forceinline__ void combine_vec(const CombineArgs& a, int t, int v) {
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

}  // namespace moe
