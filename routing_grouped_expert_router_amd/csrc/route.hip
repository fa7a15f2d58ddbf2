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
//   For T <= 64 (one block) the four run back to back in one workgroup.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kSelectThreads = 256;
constexpr int kFusedThreads = 1024;   // 16 waves

__device__ __forceinline__ uint64_t max_u64(uint64_t x, uint64_t y) { return x > y ? x : y; }

// Top-K of tokens t0 .. t0+count-1 (clamped to T), by `nwaves` waves of which
// this is `wave`.  Writes topk_ids, topk_w and the per-token non-finite flag.
template <int LPT, int NPL>
__device__ __forceinline__ void select_tokens(const RouteArgs& a, int t0, int count, int wave, int nwaves) {
  constexpr int TPW = kWave / LPT;   // tokens per wave and pass
  const int E = a.E, K = a.K;
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane / LPT, sl = lane % LPT, sbase = sub * LPT;
  for (int base = wave * TPW; base < count; base += nwaves * TPW) {
    const int t = t0 + base + sub;
    const bool valid = base + sub < count && t < a.T;
    const float* row = a.logits + (int64_t)(valid ? t : 0) * E;
    // all loads issued unconditionally (clamped column), masked afterwards
    float lv[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) lv[j] = row[min(sl + j * LPT, E - 1)];
    uint64_t keys[NPL];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = sl + j * LPT;
      const bool in = valid && e < E;
      bad |= in && !__builtin_isfinite(lv[j]);
      keys[j] = in ? topk_key(lv[j], e) : 0ull;
    }
    // descending order inside the lane (keys are distinct unless 0)
#pragma unroll
    for (int i = 1; i < NPL; ++i)
#pragma unroll
      for (int j = i; j > 0; --j) {
        const uint64_t hi = max_u64(keys[j - 1], keys[j]);
        const uint64_t lo = keys[j - 1] ^ keys[j] ^ hi;
        keys[j - 1] = hi;
        keys[j] = lo;
      }
    uint64_t my_key = 0ull;
    for (int k = 0; k < K; ++k) {
      uint64_t best = keys[0];
#pragma unroll
      for (int off = LPT >> 1; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((unsigned)(best & 0xffffffffu), off, kWave);
        const uint32_t hi = __shfl_xor((unsigned)(best >> 32), off, kWave);
        best = max_u64(best, (uint64_t(hi) << 32) | lo);
      }
      if (sl == k) my_key = best;
      // the lane holding the winner pops it (best == 0: nothing left, a no-op)
      const bool win = keys[0] == best;
#pragma unroll
      for (int j = 0; j < NPL - 1; ++j) keys[j] = win ? keys[j + 1] : keys[j];
      keys[NPL - 1] = win ? 0ull : keys[NPL - 1];
    }
    // lane sl < K holds selection sl; its logit comes back out of the key
    const int my_id = int(0xffffffffu - uint32_t(my_key & 0xffffffffu));
    const float my_l = order_key_value(uint32_t(my_key >> 32));
    // weights: w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), sum in k order
    const float l0 = __shfl(my_l, sbase, kWave);
    const float ek = (valid && sl < K) ? expf(my_l - l0) : 0.f;
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += __shfl(ek, sbase + k, kWave);
    const uint64_t badm = __ballot(bad);
    if (valid && sl < K) {
      // K <= E distinct positive keys always exist, so my_id is in [0, E)
      const int id = (my_id >= 0 && my_id < E) ? my_id : 0;
      a.topk_ids[(int64_t)t * K + sl] = id;
      a.topk_w[(int64_t)t * K + sl] = ek / sum;
    }
    if (valid && sl == 0)
      a.ws.tok_flag[t] = ((badm >> sbase) & (LPT == 64 ? ~0ull : ((1ull << LPT) - 1ull))) ? 1 : 0;
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = __shfl_xor((unsigned)(v & 0xffffffffu), off, kWave);
  const uint32_t hi = __shfl_xor((unsigned)(v >> 32), off, kWave);
  return (uint64_t(hi) << 32) | lo;
}

// Grouped sigmoid router (DeepSeek style), one wave per token: lane l holds
// experts l + 64j.  The group size gs = E / n_group divides 64, so the lanes
// of key slot j fall into 64/gs whole groups and a group's reductions are
// xor-shuffles inside gs-lane segments.
//   s_e = fp32(1 / (1 + exp(-l_e))) in fp64; key c_e = fp32(s_e + bias_e)
//   group score = sum of its group_k largest keys, fp32, descending order
//   keep the topk_group best groups (ties to the lower group id), choose the
//   K largest keys among their experts (ties to the lower id)
//   weight = s of the choice (/ sum of the K chosen s) * scale
template <int NPL>
__device__ __forceinline__ void select_tokens_grouped(const RouteArgs& a, int t0, int count, int wave, int nwaves) {
  const int E = a.E, K = a.K, G = a.n_group;
  const int gs = E / G;
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = wave; base < count; base += nwaves) {
    const int t = t0 + base;
    const bool valid = t < a.T;
    const float* row = a.logits + (int64_t)(valid ? t : 0) * E;
    // all loads issued unconditionally (clamped column), masked afterwards
    float lv[NPL], bv[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int ec = min(lane + kWave * j, E - 1);
      lv[j] = row[ec];
      bv[j] = a.score_bias ? a.score_bias[ec] : 0.f;
    }
    float sc[NPL];
    uint64_t key[NPL];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + kWave * j;
      const bool in = valid && e < E;
      bad |= in && !__builtin_isfinite(lv[j]);
      sc[j] = (float)(1.0 / (1.0 + exp(-(double)lv[j])));
      key[j] = in ? topk_key(sc[j] + bv[j], e) : 0ull;
    }
    // ---- group scores: per slot, group_k rounds of a segmented max (the
    // segment's winner pops its key), summed in descending order
    float gsum[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      uint64_t kk = key[j];
      float acc = 0.f;
      for (int r = 0; r < a.group_k; ++r) {
        uint64_t best = kk;
        for (int off = gs >> 1; off >= 1; off >>= 1) {
          const uint64_t o = shfl_xor_u64(best, off);
          best = o > best ? o : best;
        }
        const float v = order_key_value(uint32_t(best >> 32));
        acc = r == 0 ? v : acc + v;
        kk = kk == best ? 0ull : kk;
      }
      gsum[j] = acc;
    }
    // ---- group g's score onto lane g: slot (g*gs)/64, segment lane (g*gs)%64
    float my_g = 0.f;
    const int gj = (lane * gs) >> 6, gl = (lane * gs) & (kWave - 1);
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float v = __shfl(gsum[j], gl, kWave);
      my_g = j == gj ? v : my_g;
    }
    uint64_t gkey = (valid && lane < G) ? topk_key(my_g, lane) : 0ull;
    uint64_t gmask = 0ull;
    for (int r = 0; r < a.topk_group; ++r) {
      const uint64_t best = wave_max_u64(gkey);
      gmask |= 1ull << (int(0xffffffffu - uint32_t(best & 0xffffffffu)) & 63);
      gkey = gkey == best ? 0ull : gkey;
    }
    // ---- experts of the kept groups, sorted inside the lane with their scores
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + kWave * j;
      key[j] = ((gmask >> ((e / gs) & 63)) & 1ull) ? key[j] : 0ull;
    }
#pragma unroll
    for (int i = 1; i < NPL; ++i)
#pragma unroll
      for (int j = i; j > 0; --j) {
        const bool sw = key[j] > key[j - 1];
        const uint64_t k0 = sw ? key[j] : key[j - 1], k1 = sw ? key[j - 1] : key[j];
        const float s0 = sw ? sc[j] : sc[j - 1], s1 = sw ? sc[j - 1] : sc[j];
        key[j - 1] = k0; key[j] = k1; sc[j - 1] = s0; sc[j] = s1;
      }
    uint64_t my_key = 0ull;
    float my_s = 0.f;
    for (int k = 0; k < K; ++k) {
      const uint64_t best = wave_max_u64(key[0]);
      const int id = int(0xffffffffu - uint32_t(best & 0xffffffffu));
      const float sb = __shfl(sc[0], id & (kWave - 1), kWave);   // the winner's lane is id % 64
      if (lane == k) { my_key = best; my_s = sb; }
      const bool win = key[0] == best;
#pragma unroll
      for (int j = 0; j < NPL - 1; ++j) { key[j] = win ? key[j + 1] : key[j]; sc[j] = win ? sc[j + 1] : sc[j]; }
      key[NPL - 1] = win ? 0ull : key[NPL - 1];
    }
    const int my_id = int(0xffffffffu - uint32_t(my_key & 0xffffffffu));
    const float ek = (valid && lane < K) ? my_s : 0.f;
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += __shfl(ek, k, kWave);
    const uint64_t badm = __ballot(bad);
    if (valid && lane < K) {
      const int id = (my_id >= 0 && my_id < E) ? my_id : 0;
      a.topk_ids[(int64_t)t * K + lane] = id;
      a.topk_w[(int64_t)t * K + lane] = (a.renormalize ? ek / sum : ek) * a.scale;
    }
    if (valid && lane == 0) a.ws.tok_flag[t] = badm ? 1 : 0;
  }
}

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

// 64-token block b: masks per logical expert from topk_ids, then each
// choice's rank inside the block, the block's counts and its non-finite flag.
// Any workgroup size.
__device__ __forceinline__ void rank_block(const RouteArgs& a, int b) {
  __shared__ unsigned long long mask[1024];
  __shared__ int flag_s;
  const int E = a.E, K = a.K;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int t0 = b * kBlockTokens;
  const int nt = min(kBlockTokens, a.T - t0);
  for (int e = tid; e < E; e += nth) mask[e] = 0ull;
  if (tid == 0) flag_s = 0;
  __syncthreads();
  for (int i = tid; i < nt * K; i += nth) {
    const int id = a.topk_ids[(int64_t)t0 * K + i];
    atomicOr(&mask[id], 1ull << (i / K));
  }
  for (int tl = tid; tl < nt; tl += nth)
    if (a.ws.tok_flag[t0 + tl]) atomicOr(&flag_s, 1);
  __syncthreads();
  for (int i = tid; i < nt * K; i += nth) {
    const int tl = i / K;
    const int id = a.topk_ids[(int64_t)t0 * K + i];
    const unsigned long long below = tl ? (mask[id] & ((1ull << tl) - 1ull)) : 0ull;
    a.ws.local_rank[(int64_t)t0 * K + i] = __popcll(below);
  }
  for (int e = tid; e < E; e += nth) a.ws.blk[(int64_t)b * E + e] = __popcll(mask[e]);
  if (tid == 0) a.ws.blk_flags[b] = flag_s;
}

__global__ __launch_bounds__(kRouteThreads) void route_rank_kernel(RouteArgs a) { rank_block(a, blockIdx.x); }

constexpr int kScanThreads = 1024;
static_assert(kScanThreads == kFusedThreads, "the fused route kernel runs every phase in one workgroup");

__device__ __forceinline__ void scan_all(const RouteArgs& a) {
  __shared__ int cnt[kMaxE + 1];
  __shared__ int aux[kMaxE + 1];
  __shared__ int tl_s[1024];
  __shared__ int tmp[kScanThreads / 64 + 1];
  __shared__ int bad_s, nonfinite_s;
  __shared__ int bad_ep_s;
  const int tid = threadIdx.x;
  const int E = a.E, P = a.E_phys;
  const bool ep = a.local_of != nullptr;
  const int NG = ep ? a.n_global : P;       // slots the replica map may name
  const int NC = NG > P ? NG : P;
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  if (tid == 0) { bad_s = 0; nonfinite_s = 0; bad_ep_s = 0; }
  for (int p = tid; p <= NC; p += kScanThreads) { cnt[p] = 0; aux[p] = 0; }
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
        if (p < 0 || p >= NG) atomicOr(&bad_s, 1);
        else atomicAdd(&aux[p], 1);
      }
    }
  }
  __syncthreads();
  if (has_map)
    for (int p = tid; p < NG; p += kScanThreads)
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
  bool ep_ok = true;
  if (ep) {
    // local map: entries in [-1, P), each local slot named at most once; the
    // local counts take the counts of their global slots (remote: dropped
    // here, counted by their own rank)
    for (int q = tid; q < NC; q += kScanThreads) aux[q] = 0;
    __syncthreads();
    for (int p = tid; p < NG; p += kScanThreads) {
      const int q = a.local_of[p];
      if (q < -1 || q >= P) atomicOr(&bad_ep_s, 1);
      else if (q >= 0) atomicAdd(&aux[q], 1);
    }
    __syncthreads();
    for (int q = tid; q < P; q += kScanThreads)
      if (aux[q] > 1) atomicOr(&bad_ep_s, 1);
    __syncthreads();
    ep_ok = bad_ep_s == 0;
    for (int q = tid; q < P; q += kScanThreads) aux[q] = 0;
    __syncthreads();
    if (ep_ok)
      for (int p = tid; p < NG; p += kScanThreads) {
        const int q = a.local_of[p];
        if (q >= 0) aux[q] = cnt[p];
      }
    __syncthreads();
    for (int q = tid; q < P; q += kScanThreads) cnt[q] = aux[q];
    __syncthreads();
  }
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
    if (!ep_ok) st |= MOE_STATUS_BAD_EP_MAP;
    a.status[0] = st;
    a.ws.map_valid[0] = (valid ? 1 : 0) | (ep && ep_ok ? 2 : 0);
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
  const int mv = a.ws.map_valid[0];
  if (mv & 1) {
    const int R = a.rcount[l];
    p = a.l2p[(int64_t)l * a.max_replicas + j % R];
    rank = j / R;
  }
  if (a.local_of) {
    // the rank inside a slot counts the tokens of that global slot, all of
    // which are local when the slot is
    p = (mv & 2) ? a.local_of[p] : -1;
    if (p < 0) {                      // another rank's choice: no local row
      a.topk_phys[i] = -1;
      a.row_of[i] = -1;
      a.slot_of[i] = -1;
      return;
    }
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

// T <= 64: the four phases in one workgroup (one launch instead of four).
// The barrier between phases orders the global-memory tables each phase
// writes before the next one reads them.
template <int LPT, int NPL, bool GROUPED>
__global__ __launch_bounds__(kFusedThreads) void route_fused_kernel(RouteArgs a) {
  if (a.T > 0) {
    if constexpr (GROUPED) select_tokens_grouped<NPL>(a, 0, a.T, threadIdx.x / kWave, kFusedThreads / kWave);
    else select_tokens<LPT, NPL>(a, 0, a.T, threadIdx.x / kWave, kFusedThreads / kWave);
    __syncthreads();
    rank_block(a, 0);
  }
  __syncthreads();
  scan_all(a);
  __syncthreads();
  const int64_t TK = (int64_t)a.T * a.K;
  for (int64_t i = threadIdx.x; i < TK; i += kFusedThreads) assign_one(a, i);
}

template <int LPT, int NPL, bool GROUPED = false>
static void launch_shape(const RouteArgs& a, int nblk, hipStream_t s) {
  // one block: a single launch, unless 16 keys per lane would not fit the
  // registers of a 1024-thread workgroup
  constexpr bool kFusedFits = GROUPED ? NPL <= 4 : NPL <= 8;
  if (nblk <= 1 && kFusedFits) {
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
