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
//  * router_mfma_split (T <= 64, H >= 4096, with a workspace): the same
//    16 slices of a tile spread over 2-16 workgroups, the partials added by
//    the tile's last workgroup in the same order (bit-identical logits).
//  * router_block (the same, when 64-expert x 64-token blocks give at least
//    256 workgroups): 64 experts x 64 tokens per workgroup, 8 H slices.
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

// ---- few tokens: a tile's 16 H slices over S workgroups ---------------------
//
// With T <= 64 the router_mfma grid has E/16 * ceil(T/16) workgroups, a few
// dozen for 256 experts, each reading 16 W_r rows and 16 activation rows
// whole: a few compute units stream everything.  Here the 16 slices of a
// (16-expert, 16-token) tile go to S = 16 / W workgroups of W waves, each
// wave computing its slice exactly as router_mfma_kernel<1>'s wave of the
// same index does.  Every wave writes its partial tile to part; the last
// workgroup of a tile to arrive (an atomic count per tile in `arrive`, left
// at zero again) adds the 16 partials in slice order, as router_mfma_store
// does, so the logits are bit-identical to router_mfma_kernel<1>'s.
// part: [tiles][16][64] f32x4; arrive: [tiles], zero on entry.
//
// The partials cross workgroups, possibly on other XCDs, without an L2
// writeback (an agent-scope release fence writes a whole L2 back and stalls
// it for microseconds, once per workgroup here): they are stored at agent
// scope, which writes them past the XCD's L2, each wave waits until its
// stores have completed before its workgroup arrives, and the last arrival
// reads them with agent-scope loads, which do not stop at its own L2 (the
// same protocol as the grid barrier of the persistent decode kernel).
template <int W>
__global__ __launch_bounds__(W * 64) void router_mfma_split_kernel(RouterArgs a, float* part, uint32_t* arrive) {
  __shared__ int last_s;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  const int slice = blockIdx.z * W + wave;
  float* tp = part + (size_t)tile * kRouterWaves * 64 * 4;
  f32x4 acc[1];
  router_mfma_slice<1>(a, e0, t0, slice, acc);
  {
    float* p = tp + (slice * 64 + lane) * 4;
    __hip_atomic_store(p + 0, acc[0].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, acc[0].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 2, acc[0].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 3, acc[0].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);     // this wave's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    last_s = __hip_atomic_fetch_add(arrive + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             gridDim.z - 1u;
  __syncthreads();
  if (!last_s) return;
  if (threadIdx.x < 64) {
    auto ld = [&](int w) -> f32x4 {
      const float* p = tp + (w * 64 + lane) * 4;
      return f32x4{__hip_atomic_load(p + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                   __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                   __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                   __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
    };
    f32x4 sum = ld(0);
    for (int w = 1; w < kRouterWaves; ++w) sum += ld(w);
    const int t = t0 + (lane & 15);
    if (t < a.T) {
      const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 4 * (lane >> 4) + j;
        if (e < a.E) a.logits[(int64_t)t * a.E + e] = v[j] + (a.bias ? a.bias[e] : 0.f);
      }
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(arrive + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kRouterSplitMaxT = 64;

// Workgroups per tile of the split router for T tokens (0: not used): the
// smallest power of two that brings the grid to 256 workgroups, at most 16.
// Used from 4 chunks per wave (H >= 4096) on: measured on MI355X at E = 256,
// the split router takes 7.4 us against 15 us at H = 7168, but its partial
// round trip makes it slower than the one-workgroup tiles at H <= 2048.
constexpr int kRouterSplitMinH = 4096;
int router_split_count(int E, int H, int x_f32, int T) {
  if (!router_uses_mfma(E, H, x_f32) || H < kRouterSplitMinH || T < 1 || T > kRouterSplitMaxT) return 0;
  const int tiles = ((E + 15) / 16) * ((T + 15) / 16);
  int S = 2;
  while (S < 16 && tiles * S < 256) S *= 2;
  return tiles * 2 <= 256 ? S : 0;
}

// Bytes of the split router's arrival counts and partial tiles for up to
// T_max tokens (0 when the split router is never used).
// The workspace holds the counts, then the partials, of the largest tile
// count any call may have (T = min(T_max, 64)); a call uses the first tiles
// of each, so calls with fewer tokens keep the same layout.
static size_t split_tiles_max(int E, int T_max) {
  const int T = T_max < kRouterSplitMaxT ? T_max : kRouterSplitMaxT;
  return (size_t)((E + 15) / 16) * ((T + 15) / 16);
}

static size_t split_part_offset(size_t tiles_max) { return (tiles_max * sizeof(uint32_t) + 255) / 256 * 256; }

size_t router_split_bytes(int E, int H, int x_f32, int T_max) {
  const int T = T_max < kRouterSplitMaxT ? T_max : kRouterSplitMaxT;
  if (!router_split_count(E, H, x_f32, T)) return 0;
  const size_t tiles = split_tiles_max(E, T_max);
  return split_part_offset(tiles) + tiles * kRouterWaves * 64 * sizeof(f32x4);
}

hipError_t launch_router_split(const RouterArgs& a, void* ws, int T_max, hipStream_t s) {
  const int S = router_split_count(a.E, a.H, a.x_f32, a.T);
  if (!S || a.T > T_max) return hipErrorInvalidValue;
  uint32_t* arrive = static_cast<uint32_t*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + split_part_offset(split_tiles_max(a.E, T_max)));
  const dim3 g((a.E + 15) / 16, (a.T + 15) / 16, S);
  switch (S) {
    case 2: hipLaunchKernelGGL(router_mfma_split_kernel<8>, g, dim3(8 * 64), 0, s, a, part, arrive); break;
    case 4: hipLaunchKernelGGL(router_mfma_split_kernel<4>, g, dim3(4 * 64), 0, s, a, part, arrive); break;
    case 8: hipLaunchKernelGGL(router_mfma_split_kernel<2>, g, dim3(2 * 64), 0, s, a, part, arrive); break;
    default: hipLaunchKernelGGL(router_mfma_split_kernel<1>, g, dim3(64), 0, s, a, part, arrive); break;
  }
  return hipGetLastError();
}

// ---- many tokens: 64 experts x 64 tokens per workgroup ----------------------
//
// A 16-expert block re-reads every activation row once per block (16 times
// for 256 experts); with many tokens that operand traffic, not HBM, bounds
// router_mfma.  Here a workgroup owns 64 experts x 64 tokens, so each
// activation row is read E/64 times and each W_r row T/64 times.  Its 8
// waves split H into 8 slices; wave w sums slice w in 64-wide chunks
// (two v_mfma_f32_16x16x32_bf16 per chunk and tile, the next chunk's
// operands in flight), then the 8 partial tiles are added in wave order
// through LDS.  Summation order is fixed: bit-reproducible.
constexpr int kRouterBlockWaves = 8;

__global__ __launch_bounds__(kRouterBlockWaves * 64) void router_block_kernel(RouterArgs a) {
  __shared__ f32x4 red[kRouterBlockWaves][16][64];   // 128 KiB: [wave][4 expert x 4 token tiles][lane]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int e0 = blockIdx.x * 64, t0 = blockIdx.y * 64;
  // rows past E or T read row 0; their results are never written
  const uint16_t* wrow[4];
  const uint16_t* xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + 16 * i + lr, t = t0 + 16 * i + lr;
    wrow[i] = a.w + (int64_t)(e < a.E ? e : 0) * a.H;
    xrow[i] = static_cast<const uint16_t*>(a.x) + (int64_t)(t < a.T ? t : 0) * a.H;
  }
  const int kw = a.H / kRouterBlockWaves;   // multiple of 64
  const int kbeg = wave * kw;
  f32x4 acc[4][4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[n][m] = f32x4{0, 0, 0, 0};
  u32x4 wc[4][2], xc[4][2];
  auto load = [&](int k0, u32x4 (*wv)[2], u32x4 (*xv)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = k0 + 32 * j + 8 * lg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wv[i][j] = *reinterpret_cast<const u32x4*>(wrow[i] + k);
        xv[i][j] = *reinterpret_cast<const u32x4*>(xrow[i] + k);
      }
    }
  };
  load(kbeg, wc, xc);
  for (int k0 = kbeg; k0 < kbeg + kw; k0 += 64) {
    u32x4 wn[4][2], xn[4][2];
    const bool more = k0 + 64 < kbeg + kw;
    if (more) load(k0 + 64, wn, xn);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[n][m] = mfma16x16x32(__builtin_bit_cast(bf16x8, wc[n][j]), __builtin_bit_cast(bf16x8, xc[m][j]),
                                   acc[n][m]);
    if (more) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) { wc[i][j] = wn[i][j]; xc[i][j] = xn[i][j]; }
    }
  }
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) red[wave][4 * n + m][lane] = acc[n][m];
  __syncthreads();
  // thread tid sums tiles tid / 64 and tid / 64 + 8 (lane tid % 64) over the waves in order;
  // lane l of tile (n, m) holds experts e0 + 16 n + 4 (l / 16) + j of token t0 + 16 m + l % 16
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tile = (tid >> 6) + 8 * h, l = tid & 63;
    f32x4 s = red[0][tile][l];
    for (int w = 1; w < kRouterBlockWaves; ++w) s += red[w][tile][l];
    const int n = tile >> 2, m = tile & 3;
    const int t = t0 + 16 * m + (l & 15);
    if (t < a.T) {
      const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 16 * n + 4 * (l >> 4) + j;
        if (e < a.E) a.logits[(int64_t)t * a.E + e] = v[j] + (a.bias ? a.bias[e] : 0.f);
      }
    }
  }
}

constexpr int kRouterOneExpertMax = 1024;   // T * E up to which each workgroup takes one expert

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t blocks = (int64_t)((a.E + 63) / 64) * ((a.T + 63) / 64);
  if (router_uses_mfma(a.E, a.H, a.x_f32) && blocks >= 256 && !(a.H % (64 * kRouterBlockWaves))) {
    hipLaunchKernelGGL(router_block_kernel, dim3((a.E + 63) / 64, (a.T + 63) / 64), dim3(kRouterBlockWaves * 64),
                       0, s, a);
  } else if (router_uses_mfma(a.E, a.H, a.x_f32)) {
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
