// Device functions of the router-logits kernels, shared with the persistent
// decode kernel.  The method is described in router.hip.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Logits of token t for experts ey*EB .. ey*EB + EB - 1 by one 256-thread
// workgroup.  Each expert's sum runs in the same order for every EB.
// WT: agent-scope stores (written through the XCD's L2) for a reader on
// another XCD later in the same launch.
template <bool WT>
__device__ __forceinline__ void store_logit(float* p, float v) {
  if constexpr (WT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// The same by a group of 256 threads inside a larger workgroup: tid is the
// thread's index in its group, red the group's LDS partials, and a group
// with t < 0 only takes part in the workgroup barrier.
template <bool XF32, int EB, bool WT = false>
__device__ __forceinline__ void router_small_group(const RouterArgs& a, int t, int ey, int tid, float (*red)[EB]) {
  const int eb = ey * EB;                      // first expert of this item
  const int ne = min(EB, a.E - eb);
  const int lane = tid & 63, wave = tid >> 6;
  float part[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) part[e] = 0.f;
  for (int h0 = tid * 8; t >= 0 && h0 < a.H; h0 += 256 * 8) {
    float xv[8];
    if (XF32) {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + (int64_t)t * a.H + h0);
      const f32x4 lo = p[0], hi = p[1];
      xv[0] = lo.x; xv[1] = lo.y; xv[2] = lo.z; xv[3] = lo.w;
      xv[4] = hi.x; xv[5] = hi.y; xv[6] = hi.z; xv[7] = hi.w;
    } else {
      const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + (int64_t)t * a.H + h0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) { xv[2 * q] = __uint_as_float(w[q] << 16); xv[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u); }
    }
    // every W_r load is issued (rows past E re-read the last row, their sums
    // are never stored), so none waits behind a branch
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(a.w + (int64_t)(eb + min(e, ne - 1)) * a.H + h0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      float s = part[e];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s += xv[2 * q] * __uint_as_float(w[q] << 16);
        s += xv[2 * q + 1] * __uint_as_float(w[q] & 0xffff0000u);
      }
      part[e] = s;
    }
  }
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    float v = part[e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    if (lane == 0) red[wave][e] = v;
  }
  __syncthreads();
  if (t >= 0 && tid < ne) {
    const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    store_logit<WT>(a.logits + (int64_t)t * a.E + eb + tid, v + (a.bias ? a.bias[eb + tid] : 0.f));
  }
}

// NI (token, expert) logits by one group of 256 threads, each summed in
// exactly the order router_small_group<XF32, 1> sums it, with the loads of
// all NI items issued together (one memory latency for the NI items rather
// than one each).  Item q is (ts[q], es[q]); ts[q] < 0: no item (es[q]
// must still name a row of W_r).  Each logit is also written to lds_out[q].
// red: this group's LDS partials, 4 * NI floats.
template <bool XF32, int NI>
__device__ __forceinline__ void router_small_group_n(const RouterArgs& a, const int* ts, const int* es, int tid,
                                                     float* red, float* lds_out) {
  const int lane = tid & 63, wave = tid >> 6;
  float part[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) part[q] = 0.f;
  // the 16 bytes of x and of W_r one item takes at h0; the next step's are
  // loaded before this step is summed (past the end: the last step again,
  // never used), so the group waits for memory about once
  u32x4 xr[NI][2], wr[NI];
  auto load = [&](int h0, u32x4 (*xd)[2], u32x4* wd) -> void {
    const int hc = min(h0, a.H - 8);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int t = ts[q] >= 0 ? ts[q] : 0;
      if (XF32) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.x) + (int64_t)t * a.H + hc);
        xd[q][0] = p[0];
        xd[q][1] = p[1];
      } else {
        xd[q][0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + (int64_t)t * a.H + hc);
      }
      wd[q] = *reinterpret_cast<const u32x4*>(a.w + (int64_t)es[q] * a.H + hc);
    }
  };
  load(tid * 8, xr, wr);
  for (int h0 = tid * 8; h0 < a.H; h0 += 256 * 8) {
    u32x4 xc[NI][2], wc[NI];
#pragma unroll
    for (int q = 0; q < NI; ++q) { xc[q][0] = xr[q][0]; xc[q][1] = xr[q][1]; wc[q] = wr[q]; }
    load(h0 + 256 * 8, xr, wr);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      float xv[8];
      if (XF32) {
        xv[0] = __uint_as_float(xc[q][0].x); xv[1] = __uint_as_float(xc[q][0].y);
        xv[2] = __uint_as_float(xc[q][0].z); xv[3] = __uint_as_float(xc[q][0].w);
        xv[4] = __uint_as_float(xc[q][1].x); xv[5] = __uint_as_float(xc[q][1].y);
        xv[6] = __uint_as_float(xc[q][1].z); xv[7] = __uint_as_float(xc[q][1].w);
      } else {
        const uint32_t w[4] = {xc[q][0].x, xc[q][0].y, xc[q][0].z, xc[q][0].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          xv[2 * k] = __uint_as_float(w[k] << 16);
          xv[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
      }
      const uint32_t w[4] = {wc[q].x, wc[q].y, wc[q].z, wc[q].w};
      float s = part[q];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s += xv[2 * k] * __uint_as_float(w[k] << 16);
        s += xv[2 * k + 1] * __uint_as_float(w[k] & 0xffff0000u);
      }
      part[q] = s;
    }
  }
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    float v = part[q];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    if (lane == 0) red[q * 4 + wave] = v;
  }
  __syncthreads();
  if (tid < NI && ts[tid] >= 0) {
    const int q = tid;
    const float v = ((red[q * 4] + red[q * 4 + 1]) + red[q * 4 + 2]) + red[q * 4 + 3];
    const float o = v + (a.bias ? a.bias[es[q]] : 0.f);
    a.logits[(int64_t)ts[q] * a.E + es[q]] = o;
    lds_out[q] = o;
  }
}

template <bool XF32, int EB, bool WT = false>
__device__ __forceinline__ void router_small_item(const RouterArgs& a, int t, int ey) {
  __shared__ float red[4][EB];
  router_small_group<XF32, EB, WT>(a, t, ey, threadIdx.x, red);
}

constexpr int kRouterWaves = 16;   // H slices of the MFMA router (one per wave)
// 64-wide chunks of a slice in flight (register sets of weights and MR
// token tiles, within a 1024-thread workgroup's 128 registers per lane)
template <int MR>
constexpr int router_ahead() { return MR >= 4 ? 2 : 4; }

// Slice `slice` (of kRouterWaves) of H for experts e0 .. e0+15 and tokens
// t0 .. t0 + 16*MR - 1, summed from zero in 64-wide chunks by one wave with
// v_mfma_f32_16x16x32_bf16; lane l returns experts e0 + 4*(l/16) + j of
// token t0 + 16*m + l%16 in acc[m][j].
template <int MR>
__device__ __forceinline__ void router_mfma_slice(const RouterArgs& a, int e0, int t0, int slice, f32x4* acc) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int erow = e0 + lr;
  const bool eok = erow < a.E;
  const uint16_t* wrow = a.w + (int64_t)(eok ? erow : 0) * a.H;
  const uint16_t* xrow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int t = t0 + 16 * m + lr;
    xrow[m] = static_cast<const uint16_t*>(a.x) + (int64_t)(t < a.T ? t : 0) * a.H;
  }
  const int kw = a.H / kRouterWaves;          // multiple of 64 (H % 1024 == 0)
  const int kbeg = slice * kw;
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = f32x4{0, 0, 0, 0};
  auto load = [&](int k0, u32x4* wv, u32x4 (*xv)[2]) -> void {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = k0 + 32 * j + 8 * lg;
      // rows past E or T read row 0; their results are never written
      wv[j] = *reinterpret_cast<const u32x4*>(wrow + k);
#pragma unroll
      for (int m = 0; m < MR; ++m) xv[m][j] = *reinterpret_cast<const u32x4*>(xrow[m] + k);
    }
  };
  // router_ahead<MR>() 64-wide chunks in flight in a ring of register sets (a
  // slice has a few chunks: one at a time left the wave waiting a full
  // memory latency per chunk); the MFMAs run in chunk order.  Slices of up
  // to 8 chunks (H <= 8192) run fully unrolled: with every load at a fixed
  // place the compiler waits for the oldest chunk only, where a loop made it
  // wait for every load in flight once per turn.
  constexpr int D = router_ahead<MR>();
  u32x4 wv[D][2], xv[D][MR][2];
  const int nch = kw / 64;
  auto step = [&](int c, int d) -> void {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < MR; ++m)
        acc[m] = mfma16x16x32(__builtin_bit_cast(bf16x8, wv[d][j]), __builtin_bit_cast(bf16x8, xv[d][m][j]), acc[m]);
  };
  auto unrolled = [&](auto nc) -> void {
    constexpr int NCH = decltype(nc)::value;
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < NCH) load(kbeg + 64 * d, wv[d], xv[d]);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      step(c, c % D);
      if (c + D < NCH) load(kbeg + 64 * (c + D), wv[c % D], xv[c % D]);
    }
  };
  switch (nch) {
    case 1: unrolled(IntC<1>{}); break;
    case 2: unrolled(IntC<2>{}); break;
    case 3: unrolled(IntC<3>{}); break;
    case 4: unrolled(IntC<4>{}); break;
    case 5: unrolled(IntC<5>{}); break;
    case 6: unrolled(IntC<6>{}); break;
    case 7: unrolled(IntC<7>{}); break;
    case 8: unrolled(IntC<8>{}); break;
    default: {
      // every step issues its loads, past the slice's end re-reading its
      // last chunk (never used), so that no load sits under a branch
#pragma unroll
      for (int d = 0; d < D; ++d) load(kbeg + 64 * d, wv[d], xv[d]);
      for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int c = c0 + d;
          if (c < nch) step(c, d);
          load(kbeg + 64 * min(c + D, nch - 1), wv[d], xv[d]);
        }
      }
    }
  }
}

// The kRouterWaves slice sums red[0..15][m][l], added in slice order, stored
// with the bias (threads tid < 64*MR).
template <int MR, bool WT = false>
__device__ __forceinline__ void router_mfma_store(const RouterArgs& a, int e0, int t0, const f32x4 (*red)[MR][64]) {
  const int tid = threadIdx.x;
  if (tid < 64 * MR) {
    const int m = tid >> 6, l = tid & 63;
    f32x4 s = red[0][m][l];
    for (int w = 1; w < kRouterWaves; ++w) s += red[w][m][l];
    const int t = t0 + 16 * m + (l & 15);
    if (t < a.T) {
      const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 4 * (l >> 4) + j;
        if (e < a.E) store_logit<WT>(a.logits + (int64_t)t * a.E + e, v[j] + (a.bias ? a.bias[e] : 0.f));
      }
    }
  }
}

}  // namespace moe
