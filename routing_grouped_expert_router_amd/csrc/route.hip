// Routing on gfx950: top-K with renormalised softmax weights, per-slot
// counts, prefix-sum offsets, the stable expert-grouped order and the layout
// tables.
//
// Method (vllbc blog "MoE inference and expert parallelism", routing section
// and Table 3-1; vLLM forward path: top-k, then sort token/expert pairs by
// expert; MoonEP online plan: counts -> offsets -> expert-grouped slots):
//   kernel 1, one workgroup per 64-token block: a subgroup of lanes (the
//     power of two >= E, 8..64) takes a token and finds its K largest logits
//     by K rounds of a subgroup max over packed (value, ~id) keys; several
//     tokens share a wave when E is small.  The block's choices set bits in
//     one 64-bit mask per
//     logical expert, from which each choice's rank among earlier tokens of
//     the block and the block's count per expert follow by popcount.  OR is
//     order-independent, so the result is deterministic.
//   kernel 2, one workgroup: per-expert exclusive scan of the block counts,
//     replica-map validation and the round-robin split into physical counts,
//     then scans for offsets, spill offsets (masked) or padded offsets
//     (contiguous), and the status word.
//   kernel 3, one thread per choice: the choice's rank j among all tokens of
//     its logical expert, its replica l2p[l][j mod R] and rank j / R inside
//     that slot, its row, its buffer slot, and src_of.
//   For T <= 64 (one block) the three run back to back in one workgroup.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kTopkThreads = 1024;   // 16 waves per 64-token block

// lanes per token: the smallest power of two >= E, between 8 and 64
inline int topk_lanes(int E) {
  int l = 8;
  while (l < E && l < 64) l <<= 1;
  return l;
}

// one 64-token block b, by a workgroup of kTopkThreads threads
__device__ __forceinline__ void topk_block(const RouteArgs& a, int b) {
  __shared__ unsigned long long mask[1024];
  __shared__ int ids_s[kBlockTokens * kMaxK];
  __shared__ int flag_s;
  const int E = a.E, K = a.K, T = a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kTopkThreads) mask[e] = 0ull;
  if (tid == 0) flag_s = 0;
  __syncthreads();

  // a token is handled by a subgroup of LPT lanes; a wave holds 64/LPT tokens
  const int LPT = a.topk_lanes;
  const int tpw = kWave / LPT;
  const int sub = lane / LPT, sl = lane % LPT, sbase = sub * LPT;
  const int npl = (E + LPT - 1) / LPT;           // logits per lane (<= 16)
  for (int tl0 = wave * tpw; tl0 < kBlockTokens; tl0 += (kTopkThreads / kWave) * tpw) {
    const int tl = tl0 + sub;
    const int t = b * kBlockTokens + tl;
    const bool valid = t < T;
    const float* row = a.logits + (int64_t)(valid ? t : 0) * E;
    uint64_t keys[16];
    bool bad = false;
    // all loads issued unconditionally (clamped column), masked afterwards
    float lv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) lv[j] = row[min(sl + j * LPT, E - 1)];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = sl + j * LPT;
      const bool in = valid && j < npl && e < E;
      bad |= in && !__builtin_isfinite(lv[j]);
      keys[j] = in ? topk_key(lv[j], e) : 0ull;
    }
    if (bad) atomicOr(&flag_s, 1);
    uint64_t prev = ~0ull;
    int my_id = -1;
    for (int k = 0; k < K; ++k) {
      uint64_t best = 0ull;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint64_t c = keys[j] < prev ? keys[j] : 0ull;
        best = c > best ? c : best;
      }
      // max over the LPT lanes of this subgroup
      for (int off = LPT >> 1; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((unsigned)(best & 0xffffffffu), off, kWave);
        const uint32_t hi = __shfl_xor((unsigned)(best >> 32), off, kWave);
        const uint64_t o = (uint64_t(hi) << 32) | lo;
        best = o > best ? o : best;
      }
      prev = best;
      const int id = int(0xffffffffu - uint32_t(best & 0xffffffffu));
      if (sl == k) my_id = id;
    }
    // weights: w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), sum in k order
    const int id0 = __shfl(my_id, sbase, kWave);
    const float l0 = valid ? row[id0] : 0.f;
    float ek = 0.f, sum = 0.f;
    for (int k = 0; k < K; ++k) {
      const int idk = __shfl(my_id, sbase + k, kWave);
      const float e = valid ? expf(row[idk] - l0) : 0.f;
      sum += e;
      if (sl == k) ek = e;
    }
    if (valid && sl < K) {
      // K <= E distinct positive keys always exist, so my_id is in [0, E)
      const int id = (my_id >= 0 && my_id < E) ? my_id : 0;
      a.topk_ids[(int64_t)t * K + sl] = id;
      a.topk_w[(int64_t)t * K + sl] = ek / sum;
      ids_s[tl * K + sl] = id;
      atomicOr(&mask[id], 1ull << tl);
    }
  }
  __syncthreads();
  for (int i = tid; i < kBlockTokens * K; i += kTopkThreads) {
    const int tl = i / K, t = b * kBlockTokens + tl;
    if (t < T) {
      const int e = ids_s[i];
      const unsigned long long below = tl ? (mask[e] & ((1ull << tl) - 1ull)) : 0ull;
      a.ws.local_rank[(int64_t)t * K + (i - tl * K)] = __popcll(below);
    }
  }
  for (int e = tid; e < E; e += kTopkThreads)
    a.ws.blk[(int64_t)b * E + e] = __popcll(mask[e]);
  if (tid == 0) a.ws.blk_flags[b] = flag_s;
}

__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(RouteArgs a) { topk_block(a, blockIdx.x); }

constexpr int kScanThreads = 1024;
static_assert(kScanThreads == kTopkThreads, "the fused route kernel runs both phases in one workgroup");

__device__ __forceinline__ void scan_all(const RouteArgs& a) {
  __shared__ int cnt[kMaxE + 1];
  __shared__ int aux[kMaxE + 1];
  __shared__ int tl_s[1024];
  __shared__ int tmp[kScanThreads / 64 + 1];
  __shared__ int bad_s, nonfinite_s;
  const int tid = threadIdx.x;
  const int E = a.E, P = a.E_phys;
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  if (tid == 0) { bad_s = 0; nonfinite_s = 0; }
  for (int p = tid; p <= P; p += kScanThreads) { cnt[p] = 0; aux[p] = 0; }
  __syncthreads();
  // per logical expert: exclusive prefix over blocks, and total T_l
  for (int l = tid; l < E; l += kScanThreads) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = a.ws.blk[(int64_t)b * E + l];
      a.ws.blk[(int64_t)b * E + l] = run;
      run += c;
    }
    tl_s[l] = run;
  }
  for (int b = tid; b < nblk; b += kScanThreads)
    if (a.ws.blk_flags[b]) atomicOr(&nonfinite_s, 1);
  // replica map validation: counts in [1, max_replicas], slots in range,
  // every slot listed at most once
  const bool has_map = a.l2p != nullptr;
  if (has_map) {
    for (int l = tid; l < E; l += kScanThreads) {
      const int R = a.rcount[l];
      if (R < 1 || R > a.max_replicas) { atomicOr(&bad_s, 1); continue; }
      for (int r = 0; r < R; ++r) {
        const int p = a.l2p[(int64_t)l * a.max_replicas + r];
        if (p < 0 || p >= P) atomicOr(&bad_s, 1);
        else atomicAdd(&aux[p], 1);
      }
    }
  }
  __syncthreads();
  if (has_map)
    for (int p = tid; p < P; p += kScanThreads)
      if (aux[p] > 1) atomicOr(&bad_s, 1);
  __syncthreads();
  const bool valid = has_map && bad_s == 0;
  // physical counts: replica r of l gets the j = r, r+R, ... tokens
  for (int l = tid; l < E; l += kScanThreads) {
    const int Tl = tl_s[l];
    if (valid) {
      const int R = a.rcount[l];
      for (int r = 0; r < R; ++r)
        cnt[a.l2p[(int64_t)l * a.max_replicas + r]] = (Tl - r + R - 1) / R;
    } else {
      cnt[l] = Tl;
    }
  }
  __syncthreads();
  const bool masked = a.layout == MOE_MASKED;
  for (int p = tid; p < P; p += kScanThreads) {
    const int c = cnt[p];
    a.counts[p] = c;
    if (masked) {
      const int mm = c < a.M_max ? c : a.M_max;
      a.masked_m[p] = mm;
      aux[p] = c - mm;
    } else {
      aux[p] = (c + a.BM - 1) / a.BM * a.BM;
    }
  }
  __syncthreads();
  const int total = block_exclusive_scan(cnt, P, tmp);
  const int total2 = block_exclusive_scan(aux, P, tmp);
  for (int p = tid; p < P; p += kScanThreads) {
    a.offsets[p] = cnt[p];
    if (masked) a.spill_off[p] = aux[p];
    else a.pad_off[p] = aux[p];
  }
  __syncthreads();
  // tiles of kTileRows rows per slot for the tiled expert kernel (aux reused;
  // cnt holds the exclusive offsets, so slot p has cnt[p+1] - cnt[p] rows)
  for (int p = tid; p < P; p += kScanThreads) {
    const int rows = (p + 1 < P ? cnt[p + 1] : total) - cnt[p];
    aux[p] = (rows + kTileRows - 1) / kTileRows;
  }
  __syncthreads();
  const int ttotal = block_exclusive_scan(aux, P, tmp);
  for (int p = tid; p < P; p += kScanThreads) a.tile_off[p] = aux[p];
  if (tid == 0) {
    a.tile_off[P] = ttotal;
    a.tile_off[P + 1] = ttotal + (a.n_shared ? (a.T + kTileRows - 1) / kTileRows : 0);
    a.offsets[P] = total;
    if (masked) a.spill_off[P] = total2;
    else a.pad_off[P] = total2;
    uint32_t st = 0;
    if (nonfinite_s) st |= MOE_STATUS_NONFINITE;
    if (masked && total2 > 0) st |= MOE_STATUS_SPILL;
    if (has_map && !valid) st |= MOE_STATUS_BAD_REPLICA;
    a.status[0] = st;
    a.ws.map_valid[0] = valid ? 1 : 0;
  }
}

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(RouteArgs a) { scan_all(a); }

// choice i = t*K + k
__device__ __forceinline__ void assign_one(const RouteArgs& a, int64_t i) {
  const int64_t TK = (int64_t)a.T * a.K;
  const int t = int(i / a.K);
  const int l = a.topk_ids[i];
  const int b = t / kBlockTokens;
  const int j = a.ws.blk[(int64_t)b * a.E + l] + a.ws.local_rank[i];
  int p = l, rank = j;
  if (a.ws.map_valid[0]) {
    const int R = a.rcount[l];
    p = a.l2p[(int64_t)l * a.max_replicas + j % R];
    rank = j / R;
  }
  const int row = a.offsets[p] + rank;
  int64_t slot;
  if (a.layout == MOE_MASKED)
    slot = rank < a.M_max ? (int64_t)p * a.M_max + rank
                          : (int64_t)a.E_phys * a.M_max + a.spill_off[p] + (rank - a.M_max);
  else
    slot = (int64_t)a.pad_off[p] + rank;
  a.topk_phys[i] = p;
  a.row_of[i] = row;
  bool ok = true;
  if (row >= 0 && row < TK) a.src_of[row] = t; else ok = false;
  if (slot < 0 || slot >= a.routed_cap) { slot = -1; ok = false; }
  a.slot_of[i] = int32_t(slot);
  if (!ok) atomicOr(a.status, MOE_STATUS_INTERNAL);
}

__global__ __launch_bounds__(kRouteThreads) void route_assign_kernel(RouteArgs a) {
  const int64_t i = (int64_t)blockIdx.x * kRouteThreads + threadIdx.x;
  if (i < (int64_t)a.T * a.K) assign_one(a, i);
}

// T <= 64: the three phases in one workgroup (one launch instead of three).
// The barrier between phases orders the global-memory tables each phase
// writes before the next one reads them.
__global__ __launch_bounds__(kTopkThreads) void route_fused_kernel(RouteArgs a) {
  if (a.T > 0) topk_block(a, 0);
  __syncthreads();
  scan_all(a);
  __syncthreads();
  const int64_t TK = (int64_t)a.T * a.K;
  for (int64_t i = threadIdx.x; i < TK; i += kTopkThreads) assign_one(a, i);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  RouteArgs b = a;
  b.topk_lanes = topk_lanes(a.E);
  if (nblk <= 1) {
    hipLaunchKernelGGL(route_fused_kernel, dim3(1), dim3(kTopkThreads), 0, s, b);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_topk_kernel, dim3(nblk), dim3(kTopkThreads), 0, s, b);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a);
  const int64_t TK = (int64_t)a.T * a.K;
  if (TK > 0) {
    hipLaunchKernelGGL(route_assign_kernel, dim3((TK + kRouteThreads - 1) / kRouteThreads),
                       dim3(kRouteThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
