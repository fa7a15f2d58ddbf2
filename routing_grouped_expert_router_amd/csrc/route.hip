// Routing on gfx950: top-K with renormalised softmax weights, per-slot
// counts, prefix-sum offsets, the stable expert-grouped order and the layout
// tables.
//
// Method (vllbc blog "MoE inference and expert parallelism", routing section
// and Table 3-1; vLLM forward path: top-k, then sort token/expert pairs by
// expert; MoonEP online plan: counts -> offsets -> expert-grouped slots):
//   select, grid over tokens: a subgroup of LPT lanes (the power of two >= E,
//     8..64) takes a token; each lane holds NPL = ceil(E / LPT) packed
//     (value, ~id) keys, sorts them once, and each of the K rounds takes the
//     subgroup max of the lanes' heads and pops it from its lane.  Several
//     tokens share a wave when E is small.
//   rank, one workgroup per 64-token block: the block's choices set bits in
//     one 64-bit mask per logical expert, from which each choice's rank among
//     earlier tokens of the block and the block's count per expert follow by
//     popcount.  OR is order-independent, so the result is deterministic.
//   scan, one workgroup: per-expert exclusive scan of the block counts,
//     replica-map validation and the round-robin split into physical counts,
//     then scans for offsets, spill offsets (masked) or padded offsets
//     (contiguous), and the status word.
//   assign, one thread per choice: the choice's rank j among all tokens of
//     its logical expert, its replica l2p[l][j mod R] and rank j / R inside
//     that slot, its row, its buffer slot, and src_of.
//   For T <= 64 (one block) rank, scan and assign run in one workgroup that
//     keeps their tables in LDS (by its first wave alone when experts and
//     slots are at most 64), after the selection in the same workgroup, or,
//     past the tokens it selects in one pass, in a launch of its own.  Up to
//     four blocks: the three phases one after the other in one workgroup,
//     after the selection launch.
#include <type_traits>

#include "route_dev.hpp"
#include "router_dev.hpp"

namespace moe {

template <int NPL>
__global__ __launch_bounds__(kSelectThreads) void route_select_grouped_kernel(RouteArgs a) {
  constexpr int per_wg = kSelectThreads / kWave;   // one token per wave
  select_tokens_grouped<NPL>(a, blockIdx.x * per_wg, per_wg, threadIdx.x / kWave, per_wg);
}

template <int LPT, int NPL>
__global__ __launch_bounds__(kSelectThreads) void route_select_kernel(RouteArgs a) {
  constexpr int per_wg = (kSelectThreads / kWave) * (kWave / LPT);
  select_tokens<LPT, NPL>(a, blockIdx.x * per_wg, per_wg, threadIdx.x / kWave, kSelectThreads / kWave);
}

__global__ __launch_bounds__(kRouteThreads) void route_rank_kernel(RouteArgs a) { rank_block(a, blockIdx.x); }

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(RouteArgs a) { scan_all(a); }

__global__ __launch_bounds__(kRouteThreads) void route_assign_kernel(RouteArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kRouteThreads + threadIdx.x;
  if (i < (int64_t)a.T * a.K) assign_one(a, i);
}

// A few token blocks (at most kTableBlocks) in one workgroup, one launch
// instead of three: every block ranked at once (the tables rank_block makes,
// with one set of expert masks per block in LDS), then scan_all and
// assign_one, the phases handing each other their tables through global
// memory across full barriers.
constexpr int kTableBlocks = 4;

__global__ __launch_bounds__(kScanThreads) void route_blocks_kernel(RouteArgs a) {
  __shared__ unsigned long long mask[kTableBlocks][1024];   // E <= 1024 on the routing paths
  __shared__ int flag_s[kTableBlocks];
  const int E = a.E, K = a.K, T = a.T;
  const int tid = threadIdx.x;
  const int nblk = (T + kBlockTokens - 1) / kBlockTokens;
  const int TK = T * K;
  for (int i = tid; i < nblk * E; i += kScanThreads) mask[i / E][i - (i / E) * E] = 0ull;
  if (tid < kTableBlocks) flag_s[tid] = 0;
  lds_barrier();
  for (int i = tid; i < TK; i += kScanThreads) {
    const int t = i / K;
    atomicOr(&mask[t / kBlockTokens][a.topk_ids[i]], 1ull << (t % kBlockTokens));
  }
  for (int t = tid; t < T; t += kScanThreads)
    if (a.ws.tok_flag[t]) atomicOr(&flag_s[t / kBlockTokens], 1);
  lds_barrier();
  for (int i = tid; i < TK; i += kScanThreads) {
    const int t = i / K, tl = t % kBlockTokens;
    const unsigned long long below = tl ? (mask[t / kBlockTokens][a.topk_ids[i]] & ((1ull << tl) - 1ull)) : 0ull;
    a.ws.local_rank[i] = __popcll(below);
  }
  for (int i = tid; i < nblk * E; i += kScanThreads) a.ws.blk[i] = __popcll(mask[i / E][i - (i / E) * E]);
  if (tid < nblk) a.ws.blk_flags[tid] = flag_s[tid];
  __syncthreads();                           // the block tables are read by every thread below
  scan_all(a);
  __syncthreads();                           // and so are the scan's
  for (int i = tid; i < TK; i += kScanThreads) assign_one(a, i);
}

// T <= 64: the four phases in one workgroup (one launch instead of four).
// The selected ids and the non-finite flag stay in LDS for the other phases
// (route_block_tables), so no phase waits on global memory written by
// another.
template <int LPT, int NPL, bool GROUPED>
__device__ __forceinline__ void route_one_workgroup(const RouteArgs& a, const float* lds_logits = nullptr) {
  __shared__ int ids[kBlockTokens * kMaxK];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  lds_barrier();
  if (a.T > 0) {
    if constexpr (GROUPED) select_tokens_grouped<NPL>(a, 0, a.T, threadIdx.x / kWave, kFusedThreads / kWave, ids, &bad);
    else select_tokens<LPT, NPL>(a, 0, a.T, threadIdx.x / kWave, kFusedThreads / kWave, ids, &bad, lds_logits);
  }
  lds_barrier();
  route_block_tables(a, ids, bad != 0);
}

template <int LPT, int NPL, bool GROUPED>
__global__ __launch_bounds__(kFusedThreads) void route_fused_kernel(RouteArgs a) {
  route_one_workgroup<LPT, NPL, GROUPED>(a);
}

// T <= 64 with more tokens than the fused workgroup selects in one pass:
// the selection runs in its own launch over workgroups of four waves (one
// token per wave for E > 32, on as many compute units: in one workgroup the
// rounds of several tokens per wave queue on four SIMDs), then this
// workgroup reads the ids and the per-token non-finite flags back and
// builds the tables as the fused kernel does.
__global__ __launch_bounds__(kFusedThreads) void route_tables_kernel(RouteArgs a) {
  __shared__ int ids[kBlockTokens * kMaxK];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  lds_barrier();
  const int TK = a.T * a.K;
  for (int i = threadIdx.x; i < TK; i += kFusedThreads) ids[i] = a.topk_ids[i];
  for (int t = threadIdx.x; t < a.T; t += kFusedThreads)
    if (a.ws.tok_flag[t]) atomicOr(&bad, 1);
  lds_barrier();
  route_block_tables(a, ids, bad != 0);
}


// A few tokens and experts (T * E <= kTinyRouterItems, E <= 64): the router
// logits and the routing in one workgroup, one launch instead of two.  Its
// four groups of 256 threads take the (token, expert) items in turn, each
// summed exactly as the router kernel's one-item workgroups sum it, so the
// logits, and with them the tables, are bit-identical to the two launches.
constexpr int kRouterGroups = kFusedThreads / 256;

// Group g takes items g, g + 4, g + 8, g + 12 (item i: token i / E, expert
// i % E), all of them in one pass with their loads issued together; the
// logits also go to LDS, from where the routing reads them.
template <bool XF32, int LPT>
__global__ __launch_bounds__(kFusedThreads) void router_route_kernel(RouterArgs ra, RouteArgs a) {
  constexpr int NI = (kTinyRouterItems + kRouterGroups - 1) / kRouterGroups;
  __shared__ float red[kRouterGroups][4 * NI];
  __shared__ float lg[kRouterGroups * NI];        // logit of item g + 4 q at [g * NI + q]
  __shared__ float lgt[kTinyRouterItems];         // the same in [t, e] order
  const int grp = threadIdx.x >> 8, gtid = threadIdx.x & 255;
  const int items = ra.T * ra.E;
  int ts[NI], es[NI];
#pragma unroll
  for (int q = 0; q < NI; ++q) {
    const int i = grp + kRouterGroups * q;
    ts[q] = i < items ? i / ra.E : -1;
    es[q] = i < items ? i % ra.E : 0;
  }
  const int ni = (items - grp + kRouterGroups - 1) / kRouterGroups;   // this group's items
  // every group runs exactly one of these (each has one workgroup barrier)
  switch (ni) {
    case 0:
    case 1: router_small_group_n<XF32, 1>(ra, ts, es, gtid, red[grp], lg + grp * NI); break;
    case 2: router_small_group_n<XF32, 2>(ra, ts, es, gtid, red[grp], lg + grp * NI); break;
    case 3: router_small_group_n<XF32, 3>(ra, ts, es, gtid, red[grp], lg + grp * NI); break;
    default: router_small_group_n<XF32, NI>(ra, ts, es, gtid, red[grp], lg + grp * NI); break;
  }
  lds_barrier();
  if (threadIdx.x < items) lgt[threadIdx.x] = lg[(threadIdx.x % kRouterGroups) * NI + threadIdx.x / kRouterGroups];
  lds_barrier();
  route_one_workgroup<LPT, 1, false>(a, lgt);
}

bool router_route_fits(const RouterArgs& ra, const RouteArgs& a) {
  return !a.grouped && !a.local_of && a.E <= 64 && ra.E == a.E && ra.T == a.T && a.T >= 1 &&
         a.T * a.E <= kTinyRouterItems && !router_uses_mfma(ra.E, ra.H, ra.x_f32);
}

hipError_t launch_router_route(const RouterArgs& ra, const RouteArgs& a, void* split_ws, int T_max, hipStream_t s) {
  if (!router_route_fits(ra, a)) {
    const hipError_t e = split_ws && router_split_count(ra.E, ra.H, ra.x_f32, ra.T)
                             ? launch_router_split(ra, split_ws, T_max, s)
                             : launch_router(ra, s);
    return e != hipSuccess ? e : launch_route(a, s);
  }
  const dim3 g(1), b(kFusedThreads);
  auto go = [&](auto xf, auto lpt) -> void {
    hipLaunchKernelGGL((router_route_kernel<decltype(xf)::value, decltype(lpt)::value>), g, b, 0, s, ra, a);
  };
  using F = std::false_type;
  using Tr = std::true_type;
  if (a.E <= 8) ra.x_f32 ? go(Tr{}, std::integral_constant<int, 8>{}) : go(F{}, std::integral_constant<int, 8>{});
  else if (a.E <= 16) ra.x_f32 ? go(Tr{}, std::integral_constant<int, 16>{}) : go(F{}, std::integral_constant<int, 16>{});
  else if (a.E <= 32) ra.x_f32 ? go(Tr{}, std::integral_constant<int, 32>{}) : go(F{}, std::integral_constant<int, 32>{});
  else ra.x_f32 ? go(Tr{}, std::integral_constant<int, 64>{}) : go(F{}, std::integral_constant<int, 64>{});
  return hipGetLastError();
}

template <int LPT, int NPL, bool GROUPED = false>
static void launch_shape(const RouteArgs& a, int nblk, hipStream_t s) {
  // one block: a single launch, unless 16 keys per lane would not fit the
  // registers of a 1024-thread workgroup
  constexpr bool kFusedFits = GROUPED ? NPL <= 4 : NPL <= 8;
  const bool one_block = nblk <= 1 && kFusedFits;
  // tokens the fused workgroup selects in one pass (one per LPT lanes)
  constexpr int kFusedPass = (kFusedThreads / kWave) * (GROUPED ? 1 : kWave / LPT);
  if (one_block && a.T <= kFusedPass) {
    hipLaunchKernelGGL((route_fused_kernel<LPT, NPL, GROUPED>), dim3(1), dim3(kFusedThreads), 0, s, a);
    return;
  }
  if (a.T > 0) {
    if constexpr (GROUPED) {
      constexpr int per_wg = kSelectThreads / kWave;
      hipLaunchKernelGGL((route_select_grouped_kernel<NPL>), dim3((a.T + per_wg - 1) / per_wg),
                         dim3(kSelectThreads), 0, s, a);
    } else {
      constexpr int per_wg = (kSelectThreads / kWave) * (kWave / LPT);
      hipLaunchKernelGGL((route_select_kernel<LPT, NPL>), dim3((a.T + per_wg - 1) / per_wg), dim3(kSelectThreads),
                         0, s, a);
    }
  }
  if (one_block) {
    hipLaunchKernelGGL(route_tables_kernel, dim3(1), dim3(kFusedThreads), 0, s, a);
    return;
  }
  if (nblk <= kTableBlocks) {
    hipLaunchKernelGGL(route_blocks_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
    return;
  }
  hipLaunchKernelGGL(route_rank_kernel, dim3(nblk > 0 ? nblk : 1), dim3(kRouteThreads), 0, s, a);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
  const int64_t TK = (int64_t)a.T * a.K;
  if (TK > 0)
    hipLaunchKernelGGL(route_assign_kernel, dim3((TK + kRouteThreads - 1) / kRouteThreads), dim3(kRouteThreads),
                       0, s, a);
}

// Received counts (a dispatch filled rows p*M_max + i, i < counts[p], of the
// masked buffer): the masked tables the expert kernels read, no spill.
__global__ __launch_bounds__(kScanThreads) void route_received_kernel(ReceivedArgs a) {
  __shared__ int cnt[kMaxE + 1];
  __shared__ int aux[kMaxE + 1];
  __shared__ int tmp[kScanThreads / 64 + 1];
  __shared__ int over_s;
  const int tid = threadIdx.x, P = a.E_phys;
  if (tid == 0) over_s = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kScanThreads) {
    const int c = a.counts_in[p];
    if (c < 0 || c > a.M_max) atomicOr(&over_s, 1);
    const int mm = c < 0 ? 0 : (c < a.M_max ? c : a.M_max);
    cnt[p] = mm;
    aux[p] = (mm + kTileRows - 1) / kTileRows;
    a.counts[p] = mm;
    a.masked_m[p] = mm;
    a.spill_off[p] = 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan(cnt, P, tmp);
  const int ttotal = block_exclusive_scan(aux, P, tmp);
  for (int p = tid; p < P; p += kScanThreads) {
    a.offsets[p] = cnt[p];
    a.tile_off[p] = aux[p];
  }
  if (a.claim)
    for (int i = tid; i < MOE_CLAIM_WORDS; i += kScanThreads) a.claim[i] = 0u;
  if (tid == 0) {
    a.offsets[P] = total;
    a.spill_off[P] = 0;
    a.tile_off[P] = ttotal;
    a.tile_off[P + 1] = ttotal + (a.n_shared ? (a.T + kTileRows - 1) / kTileRows : 0);
    a.status[0] = over_s ? MOE_STATUS_RECV_OVERFLOW : 0u;
  }
}

hipError_t launch_route_received(const ReceivedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(route_received_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  // lanes per token: the smallest power of two >= E between 8 and 64; keys
  // per lane: ceil(E / lanes) (E <= 1024)
  const int E = a.E;
  if (a.grouped) {
    // one wave (64 lanes) per token, ceil(E/64) keys per lane
    if (E <= 64) launch_shape<64, 1, true>(a, nblk, s);
    else if (E <= 128) launch_shape<64, 2, true>(a, nblk, s);
    else if (E <= 256) launch_shape<64, 4, true>(a, nblk, s);
    else if (E <= 512) launch_shape<64, 8, true>(a, nblk, s);
    else if (E <= 1024) launch_shape<64, 16, true>(a, nblk, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (E <= 8) launch_shape<8, 1>(a, nblk, s);
  else if (E <= 16) launch_shape<16, 1>(a, nblk, s);
  else if (E <= 32) launch_shape<32, 1>(a, nblk, s);
  else if (E <= 64) launch_shape<64, 1>(a, nblk, s);
  else if (E <= 128) launch_shape<64, 2>(a, nblk, s);
  else if (E <= 256) launch_shape<64, 4>(a, nblk, s);
  else if (E <= 512) launch_shape<64, 8>(a, nblk, s);
  else if (E <= 1024) launch_shape<64, 16>(a, nblk, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe

