// Router logits on gfx950: logits[t, e] = sum_h x[t, h] * W_r[e, h] (+ bias[e]),
// fp32 accumulation (vllbc blog, routing section: one logit per expert per
// token; the bias of the synthetic workloads is added before selection).
//
// Two kernels, both with a fixed summation order (bit-reproducible):
//  * router_small (any E, fp32 or bf16 x): one workgroup per token and group of
//    up to 64 experts; thread i takes 8 consecutive h per 2048-wide stride and
//    keeps one partial sum per expert, then a wave butterfly and a fixed-order
//    sum over the four waves.  W_r rows are read from L2 by every workgroup.
//  * router_mfma (E > 64, bf16 x): a workgroup owns 16 experts x 16*MR tokens
//    (MR = 1, 2 or 4 picked so the grid has at least 256 workgroups);
//    its 16 waves split H, each runs v_mfma_f32_16x16x32_bf16 over its slice
//    with operands loaded straight to registers (next slice in flight), and
//    the 16 partial tiles are summed in wave order through LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <bool XF32, int EB>
__global__ __launch_bounds__(256) void router_small_kernel(RouterArgs a) {
  __shared__ float red[4][EB];
  const int t = blockIdx.x;
  const int eb = blockIdx.y * EB;              // first expert of this workgroup
  const int ne = min(EB, a.E - eb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float part[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) part[e] = 0.f;
  for (int h0 = tid * 8; h0 < a.H; h0 += 256 * 8) {
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
  if (tid < ne) {
    const float v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    a.logits[(int64_t)t * a.E + eb + tid] = v + (a.bias ? a.bias[eb + tid] : 0.f);
  }
}

constexpr int kRouterWaves = 16;

template <int MR>
__global__ __launch_bounds__(kRouterWaves * 64) void router_mfma_kernel(RouterArgs a) {
  __shared__ f32x4 red[kRouterWaves][MR][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16 * MR;
  const int erow = e0 + lr;
  const bool eok = erow < a.E;
  const uint16_t* wrow = a.w + (int64_t)(eok ? erow : 0) * a.H;
  const uint16_t* xrow[MR];
  bool xok[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const int t = t0 + 16 * m + lr;
    xok[m] = t < a.T;
    xrow[m] = static_cast<const uint16_t*>(a.x) + (int64_t)(xok[m] ? t : 0) * a.H;
  }
  // this wave's slice of H, in 64-wide chunks (two MFMA K steps)
  const int kw = a.H / kRouterWaves;          // multiple of 64 (H % 1024 == 0)
  const int kbeg = wave * kw;
  f32x4 acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = f32x4{0, 0, 0, 0};
  u32x4 wc[2], xc[MR][2];
  auto load = [&](int k0, u32x4* wv, u32x4 (*xv)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = k0 + 32 * j + 8 * lg;
      // rows past E or T read row 0; their results are never written
      wv[j] = *reinterpret_cast<const u32x4*>(wrow + k);
#pragma unroll
      for (int m = 0; m < MR; ++m) xv[m][j] = *reinterpret_cast<const u32x4*>(xrow[m] + k);
    }
  };
  load(kbeg, wc, xc);
  for (int k0 = kbeg; k0 < kbeg + kw; k0 += 64) {
    u32x4 wn[2], xn[MR][2];
    const bool more = k0 + 64 < kbeg + kw;
    if (more) load(k0 + 64, wn, xn);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int m = 0; m < MR; ++m)
        acc[m] = mfma16x16x32(__builtin_bit_cast(bf16x8, wc[j]), __builtin_bit_cast(bf16x8, xc[m][j]), acc[m]);
    if (more) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        wc[j] = wn[j];
#pragma unroll
        for (int m = 0; m < MR; ++m) xc[m][j] = xn[m][j];
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  if (tid < 64 * MR) {
    const int m = tid >> 6, l = tid & 63;
    f32x4 s = red[0][m][l];
    for (int w = 1; w < kRouterWaves; ++w) s += red[w][m][l];
    // lane l holds experts e0 + 4*(l/16) + j of token t0 + 16*m + l%16
    const int t = t0 + 16 * m + (l & 15);
    if (t < a.T) {
      const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 4 * (l >> 4) + j;
        if (e < a.E) a.logits[(int64_t)t * a.E + e] = v[j] + (a.bias ? a.bias[e] : 0.f);
      }
    }
  }
}

bool router_uses_mfma(int E, int H, int x_f32) { return E > 64 && !x_f32 && H % 1024 == 0; }

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
