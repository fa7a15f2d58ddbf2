// Device functions of the routing phases (select, rank, scan, assign),
// shared by the routing kernels and the persistent decode kernel.  The
// method is described in route.hip.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kSelectThreads = 256;
constexpr int kFusedThreads = 1024;   // 16 waves

__device__ __forceinline__ uint64_t max_u64(uint64_t x, uint64_t y) { return x > y ? x : y; }

// Top-K of tokens t0 .. t0+count-1 (clamped to T), by `nwaves` waves of which
// this is `wave`.  Writes topk_ids, topk_w and the per-token non-finite flag.
// lds_ids / lds_flag (single-workgroup routing): the ids also go to LDS at
// (t - t0) * K + k, and a token with a non-finite logit ORs 1 into *lds_flag
// instead of writing its global flag.
// lds_logits: the logits [T, E] in LDS instead of a.logits (they were
// computed by this workgroup).
template <int LPT, int NPL>
__device__ __forceinline__ void select_tokens(const RouteArgs& a, int t0, int count, int wave, int nwaves,
                                              int* lds_ids = nullptr, int* lds_flag = nullptr,
                                              const float* lds_logits = nullptr) {
  constexpr int TPW = kWave / LPT;   // tokens per wave and pass
  const int E = a.E, K = a.K;
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane / LPT, sl = lane % LPT, sbase = sub * LPT;
  // a token's logits; loads issued unconditionally (clamped row and column),
  // masked afterwards.  The next pass's token is loaded while this one is
  // selected, so a wave with several tokens waits for memory once.
  auto load_row = [&](int bse, float* dst) -> void {
    const int tt = t0 + bse + sub;
    const float* row = (lds_logits ? lds_logits : a.logits) + (int64_t)((bse + sub < count && tt < a.T) ? tt : 0) * E;
#pragma unroll
    for (int j = 0; j < NPL; ++j) dst[j] = row[min(sl + j * LPT, E - 1)];
  };
  float nxt[NPL];
  load_row(wave * TPW, nxt);
  for (int base = wave * TPW; base < count; base += nwaves * TPW) {
    const int t = t0 + base + sub;
    const bool valid = base + sub < count && t < a.T;
    float lv[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) lv[j] = nxt[j];
    load_row(base + nwaves * TPW, nxt);
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
      if constexpr (LPT == kWave) {
        best = wave_max_key(best);
      } else {
#pragma unroll
        for (int off = LPT >> 1; off >= 1; off >>= 1) {
          const uint32_t lo = __shfl_xor((unsigned)(best & 0xffffffffu), off, kWave);
          const uint32_t hi = __shfl_xor((unsigned)(best >> 32), off, kWave);
          best = max_u64(best, (uint64_t(hi) << 32) | lo);
        }
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
      if (lds_ids) lds_ids[(t - t0) * K + sl] = id;
    }
    if (valid && sl == 0) {
      const int fl = ((badm >> sbase) & (LPT == 64 ? ~0ull : ((1ull << LPT) - 1ull))) ? 1 : 0;
      if (!lds_flag) a.ws.tok_flag[t] = fl;
      else if (fl) atomicOr(lds_flag, 1);
    }
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
__device__ __forceinline__ void select_tokens_grouped(const RouteArgs& a, int t0, int count, int wave, int nwaves,
                                                      int* lds_ids = nullptr, int* lds_flag = nullptr) {
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
      const uint64_t best = wave_max_key(gkey);
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
      const uint64_t best = wave_max_key(key[0]);
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
      if (lds_ids) lds_ids[(t - t0) * K + lane] = id;
    }
    if (valid && lane == 0) {
      if (!lds_flag) a.ws.tok_flag[t] = badm ? 1 : 0;
      else if (badm) atomicOr(lds_flag, 1);
    }
  }
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
  lds_barrier();
  for (int i = tid; i < nt * K; i += nth) {
    const int id = a.topk_ids[(int64_t)t0 * K + i];
    atomicOr(&mask[id], 1ull << (i / K));
  }
  for (int tl = tid; tl < nt; tl += nth)
    if (a.ws.tok_flag[t0 + tl]) atomicOr(&flag_s, 1);
  lds_barrier();
  for (int i = tid; i < nt * K; i += nth) {
    const int tl = i / K;
    const int id = a.topk_ids[(int64_t)t0 * K + i];
    const unsigned long long below = tl ? (mask[id] & ((1ull << tl) - 1ull)) : 0ull;
    a.ws.local_rank[(int64_t)t0 * K + i] = __popcll(below);
  }
  for (int e = tid; e < E; e += nth) a.ws.blk[(int64_t)b * E + e] = __popcll(mask[e]);
  if (tid == 0) a.ws.blk_flags[b] = flag_s;
}


constexpr int kScanThreads = 1024;
static_assert(kScanThreads == kFusedThreads, "the fused route kernel runs every phase in one workgroup");

// Any workgroup size (the loops stride by blockDim.x); the routing kernels run
// it with kScanThreads.  Its phases hand each other data in LDS only (their
// barriers order LDS alone); its global outputs are read after the caller's
// next full barrier or by the next kernel.
__device__ __forceinline__ void scan_all(const RouteArgs& a) {
  __shared__ int cnt[kMaxE + 1];
  __shared__ int aux[kMaxE + 1];
  __shared__ int tl_s[1024];
  __shared__ int tmp[kScanThreads / 64 + 1];
  __shared__ int bad_s, nonfinite_s;
  __shared__ int bad_ep_s;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int E = a.E, P = a.E_phys;
  const bool ep = a.local_of != nullptr;
  const int NG = ep ? a.n_global : P;       // slots the replica map may name
  const int NC = NG > P ? NG : P;
  const int nblk = (a.T + kBlockTokens - 1) / kBlockTokens;
  if (tid == 0) { bad_s = 0; nonfinite_s = 0; bad_ep_s = 0; }
  for (int p = tid; p <= NC; p += nth) { cnt[p] = 0; aux[p] = 0; }
  lds_barrier();
  // per logical expert: exclusive prefix over blocks, and total T_l (16
  // blocks' counts loaded before any is overwritten, so the loads overlap)
  for (int l = tid; l < E; l += nth) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int c[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = b0 + j < nblk ? a.ws.blk[(int64_t)(b0 + j) * E + l] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < nblk) a.ws.blk[(int64_t)(b0 + j) * E + l] = run;
        run += c[j];
      }
    }
    tl_s[l] = run;
  }
  for (int b = tid; b < nblk; b += nth)
    if (a.ws.blk_flags[b]) atomicOr(&nonfinite_s, 1);
  // replica map validation: counts in [1, max_replicas], slots in range,
  // every slot listed at most once
  const bool has_map = a.l2p != nullptr;
  if (has_map) {
    for (int l = tid; l < E; l += nth) {
      const int R = a.rcount[l];
      if (R < 1 || R > a.max_replicas) { atomicOr(&bad_s, 1); continue; }
      for (int r = 0; r < R; ++r) {
        const int p = a.l2p[(int64_t)l * a.max_replicas + r];
        if (p < 0 || p >= NG) atomicOr(&bad_s, 1);
        else atomicAdd(&aux[p], 1);
      }
    }
  }
  lds_barrier();
  if (has_map)
    for (int p = tid; p < NG; p += nth)
      if (aux[p] > 1) atomicOr(&bad_s, 1);
  lds_barrier();
  const bool valid = has_map && bad_s == 0;
  // physical counts: replica r of l gets the j = r, r+R, ... tokens
  for (int l = tid; l < E; l += nth) {
    const int Tl = tl_s[l];
    if (valid) {
      const int R = a.rcount[l];
      for (int r = 0; r < R; ++r)
        cnt[a.l2p[(int64_t)l * a.max_replicas + r]] = (Tl - r + R - 1) / R;
    } else {
      cnt[l] = Tl;
    }
  }
  lds_barrier();
  bool ep_ok = true;
  if (ep) {
    // local map: entries in [-1, P), each local slot named at most once; the
    // local counts take the counts of their global slots (remote: dropped
    // here, counted by their own rank)
    for (int q = tid; q < NC; q += nth) aux[q] = 0;
    lds_barrier();
    for (int p = tid; p < NG; p += nth) {
      const int q = a.local_of[p];
      if (q < -1 || q >= P) atomicOr(&bad_ep_s, 1);
      else if (q >= 0) atomicAdd(&aux[q], 1);
    }
    lds_barrier();
    for (int q = tid; q < P; q += nth)
      if (aux[q] > 1) atomicOr(&bad_ep_s, 1);
    lds_barrier();
    ep_ok = bad_ep_s == 0;
    for (int q = tid; q < P; q += nth) aux[q] = 0;
    lds_barrier();
    if (ep_ok)
      for (int p = tid; p < NG; p += nth) {
        const int q = a.local_of[p];
        if (q >= 0) aux[q] = cnt[p];
      }
    lds_barrier();
    for (int q = tid; q < P; q += nth) cnt[q] = aux[q];
    lds_barrier();
  }
  const bool masked = a.layout == MOE_MASKED;
  for (int p = tid; p < P; p += nth) {
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
  lds_barrier();
  const int total = block_exclusive_scan(cnt, P, tmp);
  const int total2 = block_exclusive_scan(aux, P, tmp);
  for (int p = tid; p < P; p += nth) {
    a.offsets[p] = cnt[p];
    if (masked) a.spill_off[p] = aux[p];
    else a.pad_off[p] = aux[p];
  }
  lds_barrier();
  // tiles of kTileRows rows per slot for the tiled expert kernel (aux reused;
  // cnt holds the exclusive offsets, so slot p has cnt[p+1] - cnt[p] rows)
  for (int p = tid; p < P; p += nth) {
    const int rows = (p + 1 < P ? cnt[p + 1] : total) - cnt[p];
    aux[p] = (rows + kTileRows - 1) / kTileRows;
  }
  lds_barrier();
  const int ttotal = block_exclusive_scan(aux, P, tmp);
  for (int p = tid; p < P; p += nth) a.tile_off[p] = aux[p];
  if (a.claim)
    for (int i = tid; i < MOE_CLAIM_WORDS; i += nth) a.claim[i] = 0u;
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


// ---- one workgroup, T <= 64 (one token block) ------------------------------
//
// rank, scan and assign of one 64-token block with the tables in LDS: no
// phase waits on global memory written by another, nothing is read back
// from global memory except the maps, and the status word is written once,
// at the end.  The tables are the ones rank_block + scan_all + assign_one
// compute for a single block (a block's exclusive prefix is then 0, so a
// choice's rank among its logical expert's tokens is its rank in the
// block).  With at most 64 experts and slots the workgroup's first wave
// does it alone (route_tables_wave: no workgroup barrier at all, its LDS
// operations complete in order; the other waves return at once); with
// more, the whole workgroup, with LDS-only barriers between phases
// (route_tables_wg).
//   ids: LDS [T * K] selected logical ids (select_tokens' lds_ids), visible
//   to every wave (a workgroup barrier after the select);
//   tok_bad: any selected token had a non-finite logit.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Exclusive scans, in place, of N LDS arrays of n ints by one wave: lane l
// takes elements [l c, l c + c) with c = ceil(n / 64); returns the totals.
template <int N>
__device__ __forceinline__ void wave_exclusive_scan_n(int* const (&arr)[N], int n, int (&total)[N]) {
  const int lane = threadIdx.x & 63;
  const int c = (n + 63) / 64;
  const int lo = lane * c, hi = min(lo + c, n);
#pragma unroll
  for (int q = 0; q < N; ++q) {
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += arr[q][i];
    int x = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    int base = x - sum;
    for (int i = lo; i < hi; ++i) { const int v = arr[q][i]; arr[q][i] = base; base += v; }
    total[q] = __shfl(x, 63, kWave);
  }
}

__device__ __forceinline__ void route_tables_wave(const RouteArgs& a, const int* ids, bool tok_bad,
                                                  unsigned long long* mask, int* cnt, int* aux, int* pad, int* rk) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int E = a.E, P = a.E_phys, K = a.K;
  const int TK = a.T * K;
  const bool ep = a.local_of != nullptr;
  const int NG = ep ? a.n_global : P;
  const int NC = NG > P ? NG : P;
  for (int e = lane; e < E; e += kWave) mask[e] = 0ull;
  for (int p = lane; p <= NC; p += kWave) { cnt[p] = 0; aux[p] = 0; }
  wave_lds_sync();
  // rank: one bit per token in its chosen experts' masks
  for (int i = lane; i < TK; i += kWave) atomicOr(&mask[ids[i]], 1ull << (i / K));
  // replica map validation: counts in [1, max_replicas], slots in range,
  // every slot listed at most once
  const bool has_map = a.l2p != nullptr;
  bool bad = false;
  if (has_map) {
    for (int l = lane; l < E; l += kWave) {
      const int R = a.rcount[l];
      if (R < 1 || R > a.max_replicas) { bad = true; continue; }
      for (int r = 0; r < R; ++r) {
        const int p = a.l2p[(int64_t)l * a.max_replicas + r];
        if (p < 0 || p >= NG) bad = true;
        else atomicAdd(&aux[p], 1);
      }
    }
  }
  wave_lds_sync();
  // rank of choice i among the earlier tokens that chose the same expert
  for (int i = lane; i < TK; i += kWave) {
    const int tl = i / K;
    rk[i] = tl ? __popcll(mask[ids[i]] & ((1ull << tl) - 1ull)) : 0;
  }
  if (has_map)
    for (int p = lane; p < NG; p += kWave)
      if (aux[p] > 1) bad = true;
  const bool valid = has_map && __ballot(bad) == 0ull;
  // physical counts: replica r of l gets the j = r, r+R, ... tokens
  for (int l = lane; l < E; l += kWave) {
    const int Tl = __popcll(mask[l]);
    if (valid) {
      const int R = a.rcount[l];
      for (int r = 0; r < R; ++r)
        cnt[a.l2p[(int64_t)l * a.max_replicas + r]] = (Tl - r + R - 1) / R;
    } else {
      cnt[l] = Tl;
    }
  }
  wave_lds_sync();
  bool ep_ok = true;
  if (ep) {
    // local map: entries in [-1, P), each local slot named at most once; the
    // local counts take the counts of their global slots
    for (int q = lane; q < NC; q += kWave) aux[q] = 0;
    wave_lds_sync();
    bool bad_ep = false;
    for (int p = lane; p < NG; p += kWave) {
      const int q = a.local_of[p];
      if (q < -1 || q >= P) bad_ep = true;
      else if (q >= 0) atomicAdd(&aux[q], 1);
    }
    wave_lds_sync();
    for (int q = lane; q < P; q += kWave)
      if (aux[q] > 1) bad_ep = true;
    ep_ok = __ballot(bad_ep) == 0ull;
    wave_lds_sync();
    for (int q = lane; q < P; q += kWave) aux[q] = 0;
    wave_lds_sync();
    if (ep_ok)
      for (int p = lane; p < NG; p += kWave) {
        const int q = a.local_of[p];
        if (q >= 0) aux[q] = cnt[p];
      }
    wave_lds_sync();
    for (int q = lane; q < P; q += kWave) cnt[q] = aux[q];
    wave_lds_sync();
  }
  const bool masked = a.layout == MOE_MASKED;
  for (int p = lane; p < P; p += kWave) {
    const int c = cnt[p];
    a.counts[p] = c;
    if (masked) {
      const int mm = c < a.M_max ? c : a.M_max;
      a.masked_m[p] = mm;
      pad[p] = c - mm;
    } else {
      pad[p] = (c + a.BM - 1) / a.BM * a.BM;
    }
    aux[p] = (c + kTileRows - 1) / kTileRows;   // row tiles of the tiled expert kernel
  }
  wave_lds_sync();
  // offsets, spill or padded offsets, and tile offsets in one pass
  int* const arrs[3] = {cnt, pad, aux};
  int tots[3];
  wave_exclusive_scan_n<3>(arrs, P, tots);
  wave_lds_sync();
  const int total = tots[0], total2 = tots[1], ttotal = tots[2];
  for (int p = lane; p < P; p += kWave) {
    a.offsets[p] = cnt[p];
    if (masked) a.spill_off[p] = pad[p];
    else a.pad_off[p] = pad[p];
    a.tile_off[p] = aux[p];
  }
  if (a.claim)
    for (int i = lane; i < MOE_CLAIM_WORDS; i += kWave) a.claim[i] = 0u;
  uint32_t st = 0;
  if (tok_bad) st |= MOE_STATUS_NONFINITE;
  if (masked && total2 > 0) st |= MOE_STATUS_SPILL;
  if (has_map && !valid) st |= MOE_STATUS_BAD_REPLICA;
  if (!ep_ok) st |= MOE_STATUS_BAD_EP_MAP;
  if (lane == 0) {
    a.tile_off[P] = ttotal;
    a.tile_off[P + 1] = ttotal + (a.n_shared ? (a.T + kTileRows - 1) / kTileRows : 0);
    a.offsets[P] = total;
    if (masked) a.spill_off[P] = total2;
    else a.pad_off[P] = total2;
  }
  // assign: choice i's replica, row and buffer slot (as assign_one)
  bool internal = false;
  for (int i = lane; i < TK; i += kWave) {
    const int t = i / K;
    const int l = ids[i];
    const int j = rk[i];
    int p = l, rank = j;
    if (valid) {
      const int R = a.rcount[l];
      p = a.l2p[(int64_t)l * a.max_replicas + j % R];
      rank = j / R;
    }
    if (ep) {
      p = ep_ok ? a.local_of[p] : -1;
      if (p < 0) {                    // another rank's choice: no local row
        a.topk_phys[i] = -1;
        a.row_of[i] = -1;
        a.slot_of[i] = -1;
        continue;
      }
    }
    const int row = cnt[p] + rank;
    int64_t slot;
    if (masked)
      slot = rank < a.M_max ? (int64_t)p * a.M_max + rank : (int64_t)P * a.M_max + pad[p] + (rank - a.M_max);
    else
      slot = (int64_t)pad[p] + rank;
    a.topk_phys[i] = p;
    a.row_of[i] = row;
    bool ok = true;
    if (row >= 0 && row < TK) a.src_of[row] = t; else ok = false;
    if (slot < 0 || slot >= a.routed_cap) { slot = -1; ok = false; }
    a.slot_of[i] = int32_t(slot);
    internal |= !ok;
  }
  if (__ballot(internal)) st |= MOE_STATUS_INTERNAL;
  if (lane == 0) a.status[0] = st;
}

__device__ __forceinline__ void route_tables_wg(const RouteArgs& a, const int* ids, bool tok_bad,
                                                unsigned long long* mask, int* cnt, int* aux, int* pad, int* rk) {
  __shared__ int tmp[3 * (kScanThreads / 64 + 1)];
  __shared__ int bad_s, bad_ep_s, st_s;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int E = a.E, P = a.E_phys, K = a.K;
  const int TK = a.T * K;
  const bool ep = a.local_of != nullptr;
  const int NG = ep ? a.n_global : P;
  const int NC = NG > P ? NG : P;
  for (int e = tid; e < E; e += nth) mask[e] = 0ull;
  for (int p = tid; p <= NC; p += nth) { cnt[p] = 0; aux[p] = 0; }
  if (tid == 0) { bad_s = 0; bad_ep_s = 0; st_s = 0; }
  lds_barrier();
  // rank: one bit per token in its chosen experts' masks
  for (int i = tid; i < TK; i += nth) atomicOr(&mask[ids[i]], 1ull << (i / K));
  // replica map validation: counts in [1, max_replicas], slots in range,
  // every slot listed at most once
  const bool has_map = a.l2p != nullptr;
  if (has_map) {
    for (int l = tid; l < E; l += nth) {
      const int R = a.rcount[l];
      if (R < 1 || R > a.max_replicas) { atomicOr(&bad_s, 1); continue; }
      for (int r = 0; r < R; ++r) {
        const int p = a.l2p[(int64_t)l * a.max_replicas + r];
        if (p < 0 || p >= NG) atomicOr(&bad_s, 1);
        else atomicAdd(&aux[p], 1);
      }
    }
  }
  lds_barrier();
  // rank of choice i among the earlier tokens that chose the same expert
  for (int i = tid; i < TK; i += nth) {
    const int tl = i / K;
    rk[i] = tl ? __popcll(mask[ids[i]] & ((1ull << tl) - 1ull)) : 0;
  }
  if (has_map)
    for (int p = tid; p < NG; p += nth)
      if (aux[p] > 1) atomicOr(&bad_s, 1);
  lds_barrier();
  const bool valid = has_map && bad_s == 0;
  // physical counts: replica r of l gets the j = r, r+R, ... tokens
  for (int l = tid; l < E; l += nth) {
    const int Tl = __popcll(mask[l]);
    if (valid) {
      const int R = a.rcount[l];
      for (int r = 0; r < R; ++r)
        cnt[a.l2p[(int64_t)l * a.max_replicas + r]] = (Tl - r + R - 1) / R;
    } else {
      cnt[l] = Tl;
    }
  }
  lds_barrier();
  bool ep_ok = true;
  if (ep) {
    // local map: entries in [-1, P), each local slot named at most once; the
    // local counts take the counts of their global slots
    for (int q = tid; q < NC; q += nth) aux[q] = 0;
    lds_barrier();
    for (int p = tid; p < NG; p += nth) {
      const int q = a.local_of[p];
      if (q < -1 || q >= P) atomicOr(&bad_ep_s, 1);
      else if (q >= 0) atomicAdd(&aux[q], 1);
    }
    lds_barrier();
    for (int q = tid; q < P; q += nth)
      if (aux[q] > 1) atomicOr(&bad_ep_s, 1);
    lds_barrier();
    ep_ok = bad_ep_s == 0;
    for (int q = tid; q < P; q += nth) aux[q] = 0;
    lds_barrier();
    if (ep_ok)
      for (int p = tid; p < NG; p += nth) {
        const int q = a.local_of[p];
        if (q >= 0) aux[q] = cnt[p];
      }
    lds_barrier();
    for (int q = tid; q < P; q += nth) cnt[q] = aux[q];
    lds_barrier();
  }
  const bool masked = a.layout == MOE_MASKED;
  for (int p = tid; p < P; p += nth) {
    const int c = cnt[p];
    a.counts[p] = c;
    if (masked) {
      const int mm = c < a.M_max ? c : a.M_max;
      a.masked_m[p] = mm;
      pad[p] = c - mm;
    } else {
      pad[p] = (c + a.BM - 1) / a.BM * a.BM;
    }
    aux[p] = (c + kTileRows - 1) / kTileRows;   // row tiles of the tiled expert kernel
  }
  lds_barrier();
  // offsets, spill or padded offsets, and tile offsets in one pass
  int* const arrs[3] = {cnt, pad, aux};
  int tots[3];
  block_exclusive_scan_n<3>(arrs, P, tmp, tots);
  const int total = tots[0], total2 = tots[1], ttotal = tots[2];
  for (int p = tid; p < P; p += nth) {
    a.offsets[p] = cnt[p];
    if (masked) a.spill_off[p] = pad[p];
    else a.pad_off[p] = pad[p];
    a.tile_off[p] = aux[p];
  }
  if (a.claim)
    for (int i = tid; i < MOE_CLAIM_WORDS; i += nth) a.claim[i] = 0u;
  if (tid == 0) {
    a.tile_off[P] = ttotal;
    a.tile_off[P + 1] = ttotal + (a.n_shared ? (a.T + kTileRows - 1) / kTileRows : 0);
    a.offsets[P] = total;
    if (masked) a.spill_off[P] = total2;
    else a.pad_off[P] = total2;
    uint32_t st = 0;
    if (tok_bad) st |= MOE_STATUS_NONFINITE;
    if (masked && total2 > 0) st |= MOE_STATUS_SPILL;
    if (has_map && !valid) st |= MOE_STATUS_BAD_REPLICA;
    if (!ep_ok) st |= MOE_STATUS_BAD_EP_MAP;
    atomicOr(&st_s, (int)st);
  }
  // assign: choice i's replica, row and buffer slot (as assign_one)
  for (int i = tid; i < TK; i += nth) {
    const int t = i / K;
    const int l = ids[i];
    const int j = rk[i];
    int p = l, rank = j;
    if (valid) {
      const int R = a.rcount[l];
      p = a.l2p[(int64_t)l * a.max_replicas + j % R];
      rank = j / R;
    }
    if (ep) {
      p = ep_ok ? a.local_of[p] : -1;
      if (p < 0) {                    // another rank's choice: no local row
        a.topk_phys[i] = -1;
        a.row_of[i] = -1;
        a.slot_of[i] = -1;
        continue;
      }
    }
    const int row = cnt[p] + rank;
    int64_t slot;
    if (masked)
      slot = rank < a.M_max ? (int64_t)p * a.M_max + rank : (int64_t)P * a.M_max + pad[p] + (rank - a.M_max);
    else
      slot = (int64_t)pad[p] + rank;
    a.topk_phys[i] = p;
    a.row_of[i] = row;
    bool ok = true;
    if (row >= 0 && row < TK) a.src_of[row] = t; else ok = false;
    if (slot < 0 || slot >= a.routed_cap) { slot = -1; ok = false; }
    a.slot_of[i] = int32_t(slot);
    if (!ok) atomicOr(&st_s, (int)MOE_STATUS_INTERNAL);
  }
  lds_barrier();
  if (tid == 0) a.status[0] = (uint32_t)st_s;
}

__device__ __forceinline__ void route_block_tables(const RouteArgs& a, const int* ids, bool tok_bad) {
  __shared__ unsigned long long mask[1024];      // E <= 1024 on the routing paths
  __shared__ int cnt[kMaxE + 1];
  __shared__ int aux[kMaxE + 1];
  __shared__ int pad[kMaxE + 1];                 // spill (masked) or padded (contiguous) offsets
  __shared__ int rk[kBlockTokens * kMaxK];
  const int ng = a.local_of ? a.n_global : a.E_phys;
  if (a.E <= kWave && a.E_phys <= kWave && ng <= kWave) route_tables_wave(a, ids, tok_bad, mask, cnt, aux, pad, rk);
  else route_tables_wg(a, ids, tok_bad, mask, cnt, aux, pad, rk);
}

}  // namespace moe
