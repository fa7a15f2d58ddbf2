// Work items of the large-group expert kernels and their persistent schedule.
//
// A group (an expert slot, or the shared expert as group E_phys) with R rows
// owns ceil(R / kTileRows) row tiles, counted in the route table's tile_off
// prefix; each row tile pairs with every weight tile of the projection.  The
// bf16 and the W8A8 large-group kernels take such (row tile, weight tile)
// units through claim_units(), which keeps the groups that share weights on
// one XCD ("推理 INFRA 方法论(5)", DeepGEMM section: prefill groups are large,
// so each weight tile is reused over a whole tile of tokens).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// One work item of the tiled kernels: group g, weight-row tile nt, row tile mt
// and the group's row segments (s0, c0 rows, then s1, c1 spill rows).
struct TileWork {
  int g, nt, mt, c0, c1, R;
  int64_t s0, s1;
  bool shared;
};

// The rows of group g (slot g, or the shared expert as group E_phys): the
// segment s0 of c0 rows, then the spill segment s1 of c1 rows.  Args is any
// launch argument struct with the route-table fields (StreamArgs, A8Args).
template <class Args>
__device__ __forceinline__ void group_rows(const Args& a, int g, TileWork& w) {
  w.g = g;
  w.s0 = w.s1 = 0;
  w.c0 = w.c1 = 0;
  w.shared = g == a.E_phys;
  if (w.shared) { w.s0 = a.shared_base; w.c0 = a.T; }
  else if (a.layout == MOE_MASKED) {
    const int mm = a.masked_m[g];
    w.s0 = (int64_t)g * a.M_max; w.c0 = mm;
    w.s1 = (int64_t)a.E_phys * a.M_max + a.spill_off[g]; w.c1 = a.counts[g] - mm;
  } else {
    w.s0 = a.pad_off[g]; w.c0 = a.counts[g];
  }
  w.R = w.c0 + w.c1;
}

// Persistent schedule: one workgroup per compute unit, workgroup b serving
// first the work list of XCD x = b % 8 (the hardware deals linear workgroup
// ids to the XCDs in turn).  List x holds whole groups: first an eighth of the
// shared expert's row tiles, then slots x, x + 8, x + 16, ...  Its units are
// (row tile, weight tile) pairs, group by group, and inside a group weight
// tile major, row tile minor, so the row tiles of one group that read the
// same weights run close together on one XCD and the repeated weight reads
// can hit the memory-side cache, while the weight tiles of one row tile
// follow each other and share its activations in L2.  A workgroup claims its
// next unit with an atomic add on its list's counter, so faster compute units
// take more units; once its list is empty it claims from the other lists in
// turn.  The last workgroup to finish sets the counters back to zero.  Every
// workgroup computes the lists' prefix of row tiles from tile_off, in LDS, at
// start.
constexpr int kClaimLists = 8;
constexpr int kClaimStride = 16;                     // words between list counters (64-byte lines)
constexpr int kClaimDone = kClaimLists * kClaimStride;
static_assert(kClaimDone < MOE_CLAIM_WORDS, "claim counters fit the route table");
constexpr int kPlanGroups = 768;                     // largest E_phys the schedule holds
constexpr int kListChunks = kPlanGroups / kClaimLists + 1;   // groups per list (shared part first)

// Runs item(tw, hook) for every unit of the launch, tw.nt being the weight
// tile (0 .. ntn - 1) and tw.mt the row tile within group tw.g.  The item
// calls hook() once its K loop is done and before its epilogue: thread 0
// claims the next unit there, so the claim's latency overlaps the epilogue's
// arithmetic.  Every thread of the workgroup must call claim_units (it holds
// workgroup barriers); it returns once every list is empty.
template <int NTHREADS, class Args, class Item>
__device__ __forceinline__ void claim_units(const Args& a, const int32_t* tile_off, uint32_t* counters,
                                            int ntn, Item item) {
  // lt[x * L + c]: row tiles of chunk c of list x (chunk 0 the shared
  // expert's part, chunk c > 0 slot x + 8 (c - 1)), then their exclusive
  // prefix over all lists
  __shared__ int lt[kClaimLists * kListChunks + 1];
  __shared__ int scan_tmp[NTHREADS / 64 + 1];
  __shared__ int claim_s;
  const int P = a.E_phys;
  const int L = (P + kClaimLists - 1) / kClaimLists + 1;
  const int ts = tile_off[P + 1] - tile_off[P];                // the shared expert's row tiles
  const int cs = (ts + kClaimLists - 1) / kClaimLists;          // of them per list
  for (int i = threadIdx.x; i < kClaimLists * L; i += NTHREADS) {
    const int x = i / L, c = i - x * L;
    int t;
    if (c == 0) {
      t = ts - x * cs;
      t = t < 0 ? 0 : (t > cs ? cs : t);
    } else {
      const int g = x + kClaimLists * (c - 1);
      t = g < P ? tile_off[g + 1] - tile_off[g] : 0;
    }
    lt[i] = t;
  }
  __syncthreads();
  const int total = block_exclusive_scan(lt, kClaimLists * L, scan_tmp);
  if (threadIdx.x == 0) lt[kClaimLists * L] = total;
  __syncthreads();

  auto claim = [&](int x) -> int {                   // thread 0's claim on list x
    return (int)__hip_atomic_fetch_add(counters + x * kClaimStride, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  };
  auto broadcast = [&](int v) -> int {               // thread 0's value to the workgroup
    if (threadIdx.x == 0) claim_s = v;
    __syncthreads();
    const int r = __builtin_amdgcn_readfirstlane(claim_s);
    __syncthreads();                                 // claim_s is rewritten only after every read
    return r;
  };
  const int home = blockIdx.x % kClaimLists;
  int s = 0, x = home;
  int u = broadcast(threadIdx.x == 0 ? claim(x) : 0);
  for (;;) {
    const int* pl = lt + x * L;                      // list x: chunk prefixes pl[0..L], pl[L] its end
    const int base = pl[0];
    if (u >= (pl[L] - base) * ntn) {                 // list x is empty: the next one
      if (++s == kClaimLists) break;
      x = (home + s) % kClaimLists;
      u = broadcast(threadIdx.x == 0 ? claim(x) : 0);
      continue;
    }
    int lo = 0, hi = L;                              // the chunk holding unit u: largest c with
    while (hi - lo > 1) {                            // (pl[c] - base) * ntn <= u
      const int mid = (lo + hi) >> 1;
      if ((pl[mid] - base) * ntn <= u) lo = mid; else hi = mid;
    }
    const int tc = pl[lo + 1] - pl[lo];              // row tiles of the chunk (> 0: it holds u)
    const int v = u - (pl[lo] - base) * ntn;
    const int nt = v / tc;                           // weight tile major,
    const int t = v - nt * tc;                       // row tile minor
    TileWork tw;
    if (lo == 0) {
      group_rows(a, P, tw);
      tw.mt = x * cs + t;
    } else {
      group_rows(a, x + kClaimLists * (lo - 1), tw);
      tw.mt = t;
    }
    tw.nt = nt;
    int next = 0;
    item(tw, [&]() -> void {
      if (threadIdx.x == 0) next = claim(x);
    });
    u = broadcast(next);
  }
  // every workgroup has made its last claim once the done count reaches the
  // grid; the last one zeroes the counters for the next launch
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(counters + kClaimDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          gridDim.x - 1) {
    for (int xx = 0; xx < kClaimLists; ++xx)
      __hip_atomic_store(counters + xx * kClaimStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(counters + kClaimDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace moe
