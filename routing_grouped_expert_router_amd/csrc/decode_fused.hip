// The whole decode layer in one persistent launch on gfx950 (CDNA4): router
// logits, routing, the expert gate/up and down projections and the combine.
//
// At decode sizes (T <= 16 tokens) the layer is five launches around about a
// hundred microseconds of weight streaming.  The pages' decode path keeps
// every buffer preallocated so a step can be recorded and replayed as a unit ("推理 INFRA 方法论(5)", DeepEP section: low-latency kernels on
// fixed buffers; vllbc blog, Table 4-2: the decode backend with graph capture
// and the masked layout).  Here the step is one launch of G workgroups, all
// resident at once (G = compute units x workgroups that fit on one), each
// walking the work items of five phases, in item order, separated by grid
// barriers:
//   R  router logits: (token, expert) items, or (16 experts) items on MFMA
//      when E > 64;
//   A  workgroup 0 routes (select, rank, scan, assign) and lists the slots
//      that received tokens; the other workgroups meanwhile run the shared
//      expert's gate/up, which needs no routing;
//   G  routed gate/up: (listed slot, 64-row output block) items, then the
//      shared expert's down projection (its h is complete after A);
//   D  routed down: (output block, listed slot, K split) items;
//   C  combine: (token, 2048 features) items.
// Each item runs the same device code, in the same arithmetic order, as the
// corresponding multi-launch kernel (a single 16-row tile per pass, every
// slot holds at most T <= 16 rows), so the outputs are bit-identical to
// moe_router_logits + moe_route / moe_route_grouped + moe_grouped_ffn_x +
// moe_combine.
//
// Grid barrier (grid_sync below): arrival counters and one release flag per
// workgroup in the caller's fused workspace (zero-filled once; every
// completed launch leaves the counters at zero).  Outputs read by later
// phases (logits, h, y) are stored at agent scope, past the XCD's L2, and
// each XCD's L2 is written back once per barrier, so each phase's global
// writes are visible to the next phase on every XCD.  Every wait is bounded:
// a workgroup whose wait exceeds the spin limit, or that sees the abort word,
// sets the abort word and MOE_STATUS_SYNC_TIMEOUT in the status word and
// leaves; no item of a phase starts before the previous barrier has
// completed, so an abort only leaves outputs unwritten.
//
// Measured on MI355X, this single launch is slower than the five launches
// replayed from a HIP graph (whose launch boundaries cost about nothing):
// a grid barrier costs ~5 us, the L2 writeback it needs stalls an XCD's L2.
#include <cstdlib>

#include "combine_dev.hpp"
#include "route_dev.hpp"
#include "router_dev.hpp"
#include "stream_dev.hpp"

namespace moe {

constexpr int kFusedMaxT = 16;           // one 16-row tile per slot and pass
constexpr int kSpinLimit = 1 << 20;      // polls per wait (about a second)

// The XCD this wave runs on (each XCD has its own L2).
__device__ __forceinline__ int xcd_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & (kFusedGroups - 1));
}

// Per-workgroup barrier state, held by thread 0: its XCD, the workgroups on
// that XCD and the XCDs in use (known after the first barrier).
struct BarState {
  int xcd;
  uint32_t xsize, nx;
};

// Returns false (in every thread of the workgroup) when the grid aborts.
//
// An L2 writeback (the release half of an agent-scope fence) stalls the
// XCD's L2 for several microseconds whatever it holds, so it is done once
// per XCD and barrier, not once per workgroup.  Every wave first waits until
// its own stores have reached its XCD's L2; arrival is then counted per XCD,
// and the XCD's last arrival writes that L2 back for all of them before
// adding the XCD to the top counter.  The first barrier, before the
// workgroups know how many of them share an XCD, counts groups wg % 8 instead
// and each workgroup that wrote anything writes its own L2 back.  The last
// arrival of all resets the counters and releases every workgroup by writing
// the new generation into each one's own flag line, so the waiting
// workgroups poll different memory channels; polls are agent-scope relaxed
// loads (past the L2, without invalidating it), and one acquire fence per
// workgroup follows the wait.
__device__ __forceinline__ bool grid_sync(const FusedArgs& f, BarState& bs, int bar, bool wrote) {
  __shared__ int go_s, last_s;
  __shared__ uint32_t gen_s;
  const int wg = blockIdx.x, G = f.grid;
  uint32_t* const top = f.sync;
  uint32_t* const abort_w = f.sync + kFusedLine;
  uint32_t* const flag = f.sync + kFusedFlagsOff + (size_t)wg * kFusedFlagStride;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* grp;
    uint32_t gsize, ngroups;
    if (bar == 0) {
      const int ng = G < kFusedGroups ? G : kFusedGroups;
      const int gi = wg % ng;
      grp = f.sync + (2 + gi) * kFusedLine;
      gsize = (uint32_t)((G - gi + ng - 1) / ng);
      ngroups = (uint32_t)ng;
      if (wrote) __threadfence();
    } else {
      grp = f.sync + (2 + kFusedGroups + bs.xcd) * kFusedLine;
      gsize = bs.xsize;
      ngroups = bs.nx;
    }
    const uint32_t g0 = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int last = 0;
    if (__hip_atomic_fetch_add(grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == gsize) {
      __hip_atomic_store(grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // every arrival of the group has its stores in this L2 (or, first
      // barrier, already written back): write it back, and order the reset
      __threadfence();
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == ngroups) {
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();   // every group's writes acquired, the reset ordered before the flags
        last = 1;
      }
    }
    last_s = last;
    gen_s = g0 + 1u;
  }
  __syncthreads();
  int go = 1;
  if (last_s) {
    __threadfence();   // release, by every thread that writes a flag
    for (int w = threadIdx.x; w < G; w += kThreads)
      __hip_atomic_store(f.sync + kFusedFlagsOff + (size_t)w * kFusedFlagStride, gen_s, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x == 0) {
    const uint32_t g0 = gen_s - 1u;
    int n = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
      if (++n > f.spin_limit ||
          ((n & 63) == 0 && __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
        go = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  if (threadIdx.x == 0) {
    if (go && __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) go = 0;
    if (!go) {
      __hip_atomic_fetch_or(abort_w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_or(f.route.status, MOE_STATUS_SYNC_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (bar == 0) {
      // every workgroup counted itself on its XCD before arriving
      uint32_t* const members = f.sync + (2 + 2 * kFusedGroups) * kFusedLine;
      bs.xsize = __hip_atomic_load(members + bs.xcd * kFusedLine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bs.nx = 0;
      for (int x = 0; x < kFusedGroups; ++x)
        bs.nx += __hip_atomic_load(members + x * kFusedLine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    }
    go_s = go;
  }
  __syncthreads();
  return go_s != 0;
}

// Router logits of experts e0 .. e0+15 for all T <= 16 tokens: the sixteen
// H slices of the MFMA router kernel, four per wave, summed in slice order.
__device__ __forceinline__ void router_mfma_item4(const RouterArgs& a, int e0) {
  __shared__ f32x4 red[kRouterWaves][1][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int sl = wave; sl < kRouterWaves; sl += kThreads / kWave) {
    f32x4 acc[1];
    router_mfma_slice<1>(a, e0, 0, sl, acc);
    red[sl][0][lane] = acc[0];
  }
  __syncthreads();
  router_mfma_store<1, true>(a, e0, 0, red);
}

// Routing by one workgroup of kThreads, then the list of slots with tokens:
// act[0] = their number, act[1..] = their ids in ascending order.
__device__ __forceinline__ void route_phase(const FusedArgs& f) {
  const RouteArgs& a = f.route;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int nw = kThreads / kWave;
  if (a.T > 0) {
    switch (f.route_variant) {
      case 0: select_tokens<8, 1>(a, 0, a.T, wave, nw); break;
      case 1: select_tokens<16, 1>(a, 0, a.T, wave, nw); break;
      case 2: select_tokens<32, 1>(a, 0, a.T, wave, nw); break;
      case 3: select_tokens<64, 1>(a, 0, a.T, wave, nw); break;
      case 4: select_tokens<64, 2>(a, 0, a.T, wave, nw); break;
      case 5: select_tokens<64, 4>(a, 0, a.T, wave, nw); break;
      case 6: select_tokens<64, 8>(a, 0, a.T, wave, nw); break;
      case 7: select_tokens_grouped<1>(a, 0, a.T, wave, nw); break;
      case 8: select_tokens_grouped<2>(a, 0, a.T, wave, nw); break;
      default: select_tokens_grouped<4>(a, 0, a.T, wave, nw); break;
    }
    __syncthreads();
    rank_block(a, 0);
  }
  __syncthreads();
  scan_all(a);
  __syncthreads();
  const int TK = a.T * a.K;
  for (int i = tid; i < TK; i += kThreads) assign_one(a, i);
  // compaction in slot order: per chunk of kThreads slots, wave counts by
  // ballot, wave bases in wave order
  __shared__ int wcnt[nw];
  int run = 0;
  for (int p0 = 0; p0 < a.E_phys; p0 += kThreads) {
    const int p = p0 + tid;
    const bool has = p < a.E_phys && a.counts[p] > 0;
    const uint64_t m = __ballot(has);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int base = run;
    for (int w = 0; w < wave; ++w) base += wcnt[w];
    if (has) f.act[1 + base + __popcll(m & ((1ull << lane) - 1ull))] = p;
    for (int w = 0; w < nw; ++w) run += wcnt[w];
    __syncthreads();
  }
  if (tid == 0) f.act[0] = run;
}

template <bool FP8>
__device__ __forceinline__ void gate_up_item(const FusedArgs& f, int g, int bx, uint16_t* xs) {
  stream_group<FP8, MODE_GATEUP, 1, true, banks_a<FP8, MODE_GATEUP>(), true, false, true>(f.g1, g, 0, 0, 1, 0, 0, xs, bx);
}

template <bool FP8>
__device__ __forceinline__ void down_item(const FusedArgs& f, int g, int bx, int ks, uint16_t* xs) {
  stream_group<FP8, MODE_DOWN, 1, true, banks_a<FP8, MODE_DOWN>(), true, false, true>(f.g2, g, ks, 0, 1, 0, 0, xs, bx);
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void decode_fused_kernel(FusedArgs f) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[8];   // single-tile passes keep activations in registers
  const int wg = blockIdx.x, G = f.grid;
  const int T = f.route.T;
  const int P = f.route.E_phys;
  uint32_t* const members = f.sync + (2 + 2 * kFusedGroups) * kFusedLine;
  BarState bs{0, 0, 0};
  if (threadIdx.x == 0) {
    bs.xcd = xcd_id();
    __hip_atomic_fetch_add(members + bs.xcd * kFusedLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // R: router logits
  int items = 0;
  if (T > 0 && f.router_mfma) {
    const int nb = (f.router.E + 15) / 16;
    for (int i = wg; i < nb; i += G, ++items) {
      router_mfma_item4(f.router, 16 * i);
      __syncthreads();
    }
  } else if (T > 0) {
    const int ne = f.router.E;
    for (int i = wg; i < T * ne; i += G, ++items) {
      router_small_item<false, 1, true>(f.router, i / ne, i % ne);
      __syncthreads();
    }
  }
  if (!grid_sync(f, bs, 0, items > 0)) return;
  // A: routing (workgroup 0); the shared expert's gate/up (the others)
  const int nbx1 = f.g1.N / kBN, nbx2 = f.g2.N / kBN, ns = f.g2.ksplit;
  const bool shared = f.route.n_shared != 0;
  if (wg == 0) route_phase(f);
  else if (shared)
    for (int i = wg - 1; i < nbx1; i += G - 1) gate_up_item<FP8>(f, P, i, xs);
  if (!grid_sync(f, bs, 1, true)) return;
  // the XCD counts were read after the first barrier and are no longer needed
  if (wg == 0 && threadIdx.x < kFusedGroups)
    __hip_atomic_store(members + threadIdx.x * kFusedLine, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // G: routed gate/up, then the shared expert's down projection
  const int na = f.act[0];
  const int n_gu = na * nbx1;
  const int n_sd = shared ? nbx2 * ns : 0;
  for (int i = wg; i < n_gu + n_sd; i += G) {
    if (i < n_gu) {
      gate_up_item<FP8>(f, f.act[1 + i / nbx1], i % nbx1, xs);
    } else {
      const int j = i - n_gu;
      down_item<FP8>(f, P, j % nbx2, j / nbx2, xs);
    }
  }
  if (!grid_sync(f, bs, 2, true)) return;
  // D: routed down projections
  for (int i = wg; i < na * nbx2 * ns; i += G) {
    const int r = i / nbx2;
    down_item<FP8>(f, f.act[1 + r % na], i % nbx2, r / na, xs);
  }
  if (!grid_sync(f, bs, 3, true)) return;
  // C: combine
  const int nv = f.comb.H / 8;
  const int nvc = (nv + kThreads - 1) / kThreads;
  for (int i = wg; i < T * nvc; i += G) {
    const int v = (i % nvc) * kThreads + threadIdx.x;
    if (v < nv) {
      if (f.comb.y_f32) combine_vec<true>(f.comb, i / nvc, v);
      else combine_vec<false>(f.comb, i / nvc, v);
    }
  }
}

int decode_fused_variant(int E, int grouped) {
  if (grouped) return E <= 64 ? 7 : E <= 128 ? 8 : E <= 256 ? 9 : -1;
  return E <= 8 ? 0 : E <= 16 ? 1 : E <= 32 ? 2 : E <= 64 ? 3 : E <= 128 ? 4 : E <= 256 ? 5 : E <= 512 ? 6 : -1;
}

// Workgroups of the persistent grid on the current device: compute units x
// workgroups that fit on one (registers and LDS), cached per device.
int decode_fused_grid(int fp8) {
  static int cache[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& g = cache[dev][fp8 ? 1 : 0];
  if (g == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const hipError_t e = fp8
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_fused_kernel<true>, kThreads, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_fused_kernel<false>, kThreads, 0);
    if (e != hipSuccess) return 0;
    g = cus * per;
  }
  return g;
}

hipError_t launch_decode_fused(FusedArgs f, int fp8, hipStream_t s) {
  if (f.route.T < 0 || f.route.T > kFusedMaxT || f.route_variant < 0 || f.g2.ksplit > kMaxSplits)
    return hipErrorInvalidValue;
  if (f.g1.nblk != 1 || f.g2.nblk != 1 || f.g1.N % kBN || f.g2.N % kBN) return hipErrorInvalidValue;
  // fewer workgroups than fit are resident all the same
  f.grid = std::min(decode_fused_grid(fp8), kFusedMaxGrid);
  if (f.grid < 2) return hipErrorInvalidConfiguration;
  // MOE_DEBUG_FUSED_NO_WAIT (f.no_wait) bounds every wait at zero polls, so
  // that tests can take the timeout path: a workgroup that must wait aborts
  // the launch instead
  f.spin_limit = f.no_wait ? 0 : kSpinLimit;
  if (fp8) hipLaunchKernelGGL(decode_fused_kernel<true>, dim3(f.grid), dim3(kThreads), 0, s, f);
  else hipLaunchKernelGGL(decode_fused_kernel<false>, dim3(f.grid), dim3(kThreads), 0, s, f);
  return hipGetLastError();
}

}  // namespace moe
