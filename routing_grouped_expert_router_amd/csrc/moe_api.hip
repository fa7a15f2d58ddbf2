// Host side of the C ABI declared in include/moe.h: argument validation,
// buffer sizing, and the choice of kernel variants and grids.  Grids depend
// only on (desc, T), never on device-side counts.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>
#include <cstdlib>

#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

// Route workspace of moe_route_noalloc: one copy per GPU the library runs on,
// held until the process ends.  Host code never uses this name as an address
// (here it stands for the symbol only); each device's address comes from
// hipGetSymbolAddress, looked up once per device (scratch_on_device).
constexpr size_t kNoallocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline int64_t nblk_of(int64_t T) { return (T + kBlockTokens - 1) / kBlockTokens; }

struct WsLayout { size_t local_rank, blk, flags, tok_flag, map_valid, total; };

WsLayout ws_layout(const moe_desc_t* d) {
  WsLayout w;
  const int64_t TK = (int64_t)d->T_max * d->K;
  const int64_t nb = nblk_of(d->T_max);
  w.local_rank = 0;
  w.blk = w.local_rank + align_up(sizeof(int32_t) * (size_t)(TK > 0 ? TK : 1));
  w.flags = w.blk + align_up(sizeof(int32_t) * (size_t)((nb > 0 ? nb : 1) * d->E));
  w.tok_flag = w.flags + align_up(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
  w.map_valid = w.tok_flag + align_up(sizeof(int32_t) * (size_t)(d->T_max > 0 ? d->T_max : 1));
  w.total = w.map_valid + kAlign;
  return w;
}

int64_t routed_cap(const moe_desc_t* d) {
  if (d->layout == MOE_MASKED) {
    const int64_t spill = (int64_t)d->K * (d->T_max > d->M_max ? d->T_max - d->M_max : 0);
    return (int64_t)d->E_phys * d->M_max + spill;
  }
  return (int64_t)d->T_max * d->K + (int64_t)d->E_phys * (d->BM - 1);
}

bool route_ptrs_ok(const moe_desc_t* d, const moe_route_t* r) {
  if (!r) return false;
  if (!r->topk_ids || !r->topk_w || !r->topk_phys || !r->row_of || !r->slot_of || !r->src_of ||
      !r->counts || !r->offsets || !r->tile_off || !r->status)
    return false;
  if (d->layout == MOE_MASKED) return r->masked_m && r->spill_off;
  return r->pad_off != nullptr;
}

constexpr int kFusedMaxTokens = 16;

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Row tiles held in registers per pass of the streaming GEMM for the bulk of
// the groups: a slot's expected rows plus two standard deviations (tokens
// choose a slot with probability about K/E_phys), capped by M_max in the
// masked layout.  Larger groups go to the larger size classes below.
int stream_mt(const moe_desc_t* d, int T) {
  const double p = (double)d->K / d->E_phys;
  const double mean = (double)T * p;
  double rows = mean + 2.0 * sqrt(mean * (1.0 - p)) + 1.0;
  if (d->layout == MOE_MASKED && rows > d->M_max) rows = d->M_max;
  if (rows <= 16) return 1;
  if (rows <= 32) return 2;
  return 4;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status_t moe_check_desc(const moe_desc_t* d) {
  if (!d) return MOE_ERR_ARG;
  if (d->T_max < 0 || d->H <= 0 || d->I <= 0 || d->E < 1 || d->K < 1 || d->K > d->E) return MOE_ERR_ARG;
  // E_phys < E only for one rank's expert-parallel share (moe_route_ep)
  if (d->E_phys < 1 || d->n_shared < 0 || d->n_shared > 1 || d->max_replicas < 1) return MOE_ERR_ARG;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_ARG;
  if (d->w_dtype != MOE_BF16 && d->w_dtype != MOE_FP8E4M3_B128) return MOE_ERR_ARG;
  if (d->w_packed != 0 && d->w_packed != 1) return MOE_ERR_ARG;
  if (d->layout == MOE_MASKED) { if (d->M_max < 1) return MOE_ERR_ARG; }
  else if (d->layout == MOE_CONTIG) { if (d->BM < 1) return MOE_ERR_ARG; }
  else return MOE_ERR_ARG;
  if (d->H % 128 || d->I % 128) return MOE_ERR_UNSUPPORTED;
  if (d->E > 1024 || d->E_phys > kMaxE || d->K > kMaxK) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d->T_max * d->K > (int64_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const uint32_t dbg = (uint32_t)d->debug_flags;
  if (dbg & ~(MOE_DEBUG_NBLK_MASK | MOE_DEBUG_TILED_MASK | MOE_DEBUG_FUSED_NO_WAIT)) return MOE_ERR_ARG;
  if ((dbg & MOE_DEBUG_NBLK_MASK) > 8 || ((dbg & MOE_DEBUG_TILED_MASK) >> MOE_DEBUG_TILED_SHIFT) > MOE_DEBUG_A8_STREAM)
    return MOE_ERR_ARG;
  return MOE_OK;
}

size_t moe_route_workspace_bytes(const moe_desc_t* d) {
  if (moe_check_desc(d) != MOE_OK) return 0;
  return ws_layout(d).total;
}

size_t moe_workspace_bytes(const moe_desc_t* d) { return moe_route_workspace_bytes(d); }

size_t moe_router_route_workspace_bytes(const moe_desc_t* d) {
  if (moe_check_desc(d) != MOE_OK) return 0;
  return ws_layout(d).total + router_split_bytes(d->E, d->H, d->act_dtype == MOE_F32, d->T_max);
}

int64_t moe_shared_base(const moe_desc_t* d) {
  if (moe_check_desc(d) != MOE_OK) return -1;
  return routed_cap(d);
}

int64_t moe_buffer_rows(const moe_desc_t* d) {
  if (moe_check_desc(d) != MOE_OK) return -1;
  return routed_cap(d) + (int64_t)d->n_shared * d->T_max;
}

int32_t moe_down_splits(const moe_desc_t* d, int32_t T) {
  if (moe_check_desc(d) != MOE_OK) return 0;
  const int steps = d->I / 128;
  const int64_t groups = ((int64_t)T * d->K < d->E_phys ? (int64_t)T * d->K : d->E_phys) + d->n_shared;
  const int64_t wgs = groups * (d->H / 64);
  // K splits until the launch has about 1024 workgroups, or 512 when the
  // groups hold at most two rows each: measured on the Mixtral-shaped decode
  // (down projection, K = 14336), B = 1 42.7 -> 41.5 us with 4 splits
  // instead of 8 and B = 8 133 -> 127.5 us with 1 instead of 2, while at
  // B = 32 and 64 (8 rows a group) 1 split instead of 2 costs 25-40 us
  const int64_t target = (int64_t)T * d->K <= 2 * groups ? 512 : 1024;
  int s = 1;
  while (wgs * s < target && steps % (2 * s) == 0 && s < 8) s *= 2;
  return s;
}

size_t moe_y_bytes(const moe_desc_t* d, int32_t T) {
  const int32_t s = moe_down_splits(d, T);
  if (s <= 0) return 0;
  const size_t plane = (size_t)moe_buffer_rows(d) * d->H;
  return s == 1 ? plane * 2 : plane * 4 * s;
}

size_t moe_y_bytes_max(const moe_desc_t* d) {
  if (moe_check_desc(d) != MOE_OK) return 0;
  // T enters the split rule only through min(T*K, E_phys), so the token
  // counts up to ceil(E_phys / K) cover every case
  const int32_t tcap = std::min<int64_t>(d->T_max > 0 ? d->T_max : 1, ((int64_t)d->E_phys + d->K - 1) / d->K);
  size_t best = 0;
  int32_t last = -1;
  for (int32_t T = 1; T <= std::max<int32_t>(1, tcap); ++T) {
    const int32_t s = moe_down_splits(d, T);
    if (s == last) continue;           // same split, same size
    last = s;
    best = std::max(best, moe_y_bytes(d, T));
  }
  return best;
}

moe_status_t moe_router_logits(const moe_desc_t* d, const void* x, const void* w_router,
                               const float* bias, int32_t T, float* logits, hipStream_t stream) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (T < 0 || T > d->T_max) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_ARG;
  RouterArgs a = {x, d->act_dtype == MOE_F32, static_cast<const uint16_t*>(w_router), bias,
                  T, d->E, d->H, logits};
  return hip_status(launch_router(a, stream));
}

}  // extern "C"

namespace {

// Checks the routing arguments and fills the kernels' view of them.
moe_status_t route_args(const moe_desc_t* d, const float* logits, int32_t T, const moe_grouped_router_t* g,
                        const moe_ep_map_t* ep, const int32_t* l2p, const int32_t* replica_count,
                        const moe_route_t* r, void* ws, size_t ws_bytes, RouteArgs& a) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (ep) {
    // global slots: the replica map's, or the logical ids without one
    if (!ep->local_of || ep->n_global < 1 || ep->n_global > kMaxE) return MOE_ERR_ARG;
    if (!l2p && ep->n_global < d->E) return MOE_ERR_ARG;
  } else if (d->E_phys < d->E) {
    return MOE_ERR_ARG;                    // every expert needs a local slot
  }
  if (g) {
    const int G = g->n_group;
    if (G < 1 || d->E % G) return MOE_ERR_ARG;
    const int gs = d->E / G;
    if (64 % gs || g->topk_group < 1 || g->topk_group > G || g->group_k < 1 || g->group_k > 8 ||
        g->group_k > gs || (g->renormalize != 0 && g->renormalize != 1) || !std::isfinite(g->scale))
      return MOE_ERR_ARG;
    if (d->K > g->topk_group * gs) return MOE_ERR_UNSUPPORTED;
  }
  if (T < 0 || T > d->T_max || !route_ptrs_ok(d, r)) return MOE_ERR_ARG;
  if (T > 0 && !logits) return MOE_ERR_ARG;
  if ((l2p == nullptr) != (replica_count == nullptr)) return MOE_ERR_ARG;
  const WsLayout wl = ws_layout(d);
  if (!ws || ws_bytes < wl.total) return MOE_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  a = RouteArgs{};
  a.logits = logits; a.T = T; a.E = d->E; a.E_phys = d->E_phys; a.K = d->K;
  a.l2p = l2p; a.rcount = replica_count; a.max_replicas = d->max_replicas;
  if (ep) { a.local_of = ep->local_of; a.n_global = ep->n_global; }
  a.layout = d->layout; a.M_max = d->M_max; a.BM = d->BM; a.routed_cap = routed_cap(d);
  a.topk_ids = r->topk_ids; a.topk_w = r->topk_w; a.topk_phys = r->topk_phys;
  a.row_of = r->row_of; a.slot_of = r->slot_of; a.src_of = r->src_of;
  a.counts = r->counts; a.offsets = r->offsets; a.masked_m = r->masked_m;
  a.spill_off = r->spill_off; a.pad_off = r->pad_off; a.tile_off = r->tile_off;
  a.status = r->status; a.claim = r->claim; a.n_shared = d->n_shared;
  a.ws.local_rank = reinterpret_cast<int32_t*>(base + wl.local_rank);
  a.ws.blk = reinterpret_cast<int32_t*>(base + wl.blk);
  a.ws.blk_flags = reinterpret_cast<int32_t*>(base + wl.flags);
  a.ws.tok_flag = reinterpret_cast<int32_t*>(base + wl.tok_flag);
  a.ws.map_valid = reinterpret_cast<int32_t*>(base + wl.map_valid);
  if (g) {
    a.grouped = 1; a.n_group = g->n_group; a.topk_group = g->topk_group; a.group_k = g->group_k;
    a.renormalize = g->renormalize; a.score_bias = g->score_bias; a.scale = g->scale;
  }
  return MOE_OK;
}

// The current device's copy of `scratch`: its address is looked up on the
// device's first call, with that device current, and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

moe_status_t scratch_on_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

moe_status_t route_impl(const moe_desc_t* d, const float* logits, int32_t T, const moe_grouped_router_t* g,
                        const moe_ep_map_t* ep, const int32_t* l2p, const int32_t* replica_count,
                        const moe_route_t* r, void* ws, size_t ws_bytes, hipStream_t stream) {
  RouteArgs a;
  const moe_status_t st = route_args(d, logits, T, g, ep, l2p, replica_count, r, ws, ws_bytes, a);
  if (st != MOE_OK) return st;
  return hip_status(launch_route(a, stream));
}

}  // namespace

extern "C" {

moe_status_t moe_route(const moe_desc_t* d, const float* logits, int32_t T, const int32_t* l2p,
                       const int32_t* replica_count, const moe_route_t* r, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  return route_impl(d, logits, T, nullptr, nullptr, l2p, replica_count, r, ws, ws_bytes, stream);
}

moe_status_t moe_router_route(const moe_desc_t* d, const void* x, const void* w_router, const float* bias,
                              int32_t T, float* logits, const int32_t* l2p, const int32_t* replica_count,
                              const moe_route_t* r, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (T > 0 && (!x || !w_router)) return MOE_ERR_ARG;
  RouteArgs a;
  st = route_args(d, logits, T, nullptr, nullptr, l2p, replica_count, r, ws, ws_bytes, a);
  if (st != MOE_OK) return st;
  if (T == 0) return hip_status(launch_route(a, stream));   // no logits to compute
  const RouterArgs ra = {x, d->act_dtype == MOE_F32, static_cast<const uint16_t*>(w_router), bias,
                         T, d->E, d->H, logits};
  // the split router's counts and partials follow the route's workspace
  const size_t route_bytes = ws_layout(d).total;
  const size_t split_bytes = router_split_bytes(d->E, d->H, d->act_dtype == MOE_F32, d->T_max);
  void* split_ws = split_bytes && ws_bytes >= route_bytes + split_bytes ? static_cast<char*>(ws) + route_bytes : nullptr;
  return hip_status(launch_router_route(ra, a, split_ws, d->T_max, stream));
}

moe_status_t moe_route_noalloc(const moe_desc_t* d, const float* logits, int32_t T, const int32_t* l2p,
                               const int32_t* replica_count, const moe_route_t* r, hipStream_t stream) {
  const moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  // every word of the workspace is written before it is read, so the array
  // needs no clearing between calls
  if (ws_layout(d).total > kNoallocScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status_t sst = scratch_on_device(&ws);
  if (sst != MOE_OK) return sst;
  return route_impl(d, logits, T, nullptr, nullptr, l2p, replica_count, r, ws, kNoallocScratchBytes, stream);
}

moe_status_t moe_route_grouped(const moe_desc_t* d, const float* logits, int32_t T,
                               const moe_grouped_router_t* g, const int32_t* l2p,
                               const int32_t* replica_count, const moe_route_t* r, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  if (!g) return MOE_ERR_ARG;
  return route_impl(d, logits, T, g, nullptr, l2p, replica_count, r, ws, ws_bytes, stream);
}

moe_status_t moe_route_ep(const moe_desc_t* d, const float* logits, int32_t T,
                          const moe_grouped_router_t* g, const moe_ep_map_t* ep, const int32_t* l2p,
                          const int32_t* replica_count, const moe_route_t* r, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  if (!ep) return MOE_ERR_ARG;
  return route_impl(d, logits, T, g, ep, l2p, replica_count, r, ws, ws_bytes, stream);
}

moe_status_t moe_route_received(const moe_desc_t* d, const int32_t* counts, int32_t T,
                                const moe_route_t* r, hipStream_t stream) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (d->layout != MOE_MASKED) return MOE_ERR_UNSUPPORTED;
  if (!counts || T < 0 || T > d->T_max || !r || !r->counts || !r->masked_m || !r->offsets ||
      !r->spill_off || !r->tile_off || !r->status)
    return MOE_ERR_ARG;
  ReceivedArgs a = {};
  a.counts_in = counts; a.E_phys = d->E_phys; a.M_max = d->M_max; a.T = T; a.n_shared = d->n_shared;
  a.counts = r->counts; a.masked_m = r->masked_m; a.offsets = r->offsets;
  a.spill_off = r->spill_off; a.tile_off = r->tile_off; a.status = r->status; a.claim = r->claim;
  return hip_status(launch_route_received(a, stream));
}

moe_status_t moe_permute(const moe_desc_t* d, const void* x, int32_t T, const moe_route_t* r,
                         void* xg, hipStream_t stream) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (T < 0 || T > d->T_max || !route_ptrs_ok(d, r)) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !xg) return MOE_ERR_ARG;
  PermuteArgs a = {};
  a.x = x; a.act_f32 = d->act_dtype == MOE_F32; a.T = T; a.K = d->K; a.H = d->H;
  a.slot_of = r->slot_of; a.shared_base = routed_cap(d); a.n_shared = d->n_shared;
  a.rows = moe_buffer_rows(d); a.xg = static_cast<uint16_t*>(xg);
  return hip_status(launch_permute(a, stream));
}

}  // extern "C"

namespace {

moe_status_t ffn_common_checks(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                               int32_t T) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (T < 0 || T > d->T_max || !route_ptrs_ok(d, r) || !w) return MOE_ERR_ARG;
  const bool fp8 = d->w_dtype == MOE_FP8E4M3_B128;
  if (d->n_shared && fp8 && (!w->ss1 || !w->ss3 || !w->ss2)) return MOE_ERR_ARG;
  return MOE_OK;
}

// One expert projection, dispatched by each group's row count (read on the
// device; every grid depends on (desc, T) only):
//   class A  rows <= 16*mt         streaming kernel, mt row tiles per pass
//   class B  16*mt < rows <= 64    streaming kernel, 4 row tiles per pass
//   class C  rows > 64             LDS-tiled kernel (when the shape allows it;
//                                  otherwise class B takes these groups too)
// A class is launched only if T allows a group of its size (a routed group
// has at most T rows, the shared group exactly T).
// 64-row output blocks per streaming workgroup.  With fp8 weights and a
// short K range (an fp8 K step is half the bytes of a bf16 one) a workgroup
// would spend a large share of its life waiting for its first loads, so it
// walks several blocks as one pipelined stream, up to 64 K steps, while at
// least 6144 workgroups (about eight rounds of the chip) remain; fewer,
// longer workgroups would leave the chip idle at the end of the launch.
// Measured: it pays for fp8 down projections with K = 2048 and costs time for
// bf16 ones with long K ranges; a bf16 K range of at most 8 steps (a 128 KiB
// stream per block) walks two blocks.  moe_desc_t.debug_flags (MOE_DEBUG_NBLK_MASK)
// overrides the choice.
int debug_nblk(const moe_desc_t* d, int nblocks) {
  const int v = (int)((uint32_t)d->debug_flags & MOE_DEBUG_NBLK_MASK);
  return (v >= 1 && v <= 8 && nblocks % v == 0) ? v : 0;
}

int stream_nblk(const moe_desc_t* d, int32_t T, const StreamArgs& a, bool fp8) {
  const int nblocks = a.N / 64;
  const int steps = a.Kdim / 128 / a.ksplit;
  if (const int v = debug_nblk(d, nblocks)) return v;
  const int64_t TK = (int64_t)T * d->K;
  const int64_t groups = (TK < d->E_phys ? TK : d->E_phys) + d->n_shared;
  if (!fp8)
    return (steps <= 8 && nblocks % 2 == 0 && groups * (nblocks / 2) * a.ksplit >= 6144) ? 2 : 1;
  int nb = 1;
  while (nb < 8 && steps * nb * 2 <= 64 && nblocks % (nb * 2) == 0 &&
         groups * (nblocks / (nb * 2)) * a.ksplit >= 6144)
    nb *= 2;
  return nb;
}

// Which size classes a launch has (see launch_expert_gemm).
struct GemmPlan {
  int mt;          // row tiles per pass of region A
  int a_max;       // rows region A takes
  bool need_b;     // region B (streamed in passes of several tiles)
  bool need_c;     // the tiled kernel for large groups
  bool all_tiled;  // every group in the tiled launch, no streaming launch
};

// The bf16 large-group kernel that debug_flags forces (0: the library's
// choice; the W8A8 switch MOE_DEBUG_A8_STREAM leaves the choice alone).
int tiled_variant(const moe_desc_t* d) {
  const int v = (int)(((uint32_t)d->debug_flags & MOE_DEBUG_TILED_MASK) >> MOE_DEBUG_TILED_SHIFT);
  return v <= kTiledVariants ? v : 0;
}

GemmPlan plan_expert_gemm(const moe_desc_t* d, int32_t T, const StreamArgs& a, bool fp8, int mode) {
  GemmPlan p;
  p.mt = stream_mt(d, T);
  const bool tiled = tiled_supported(mode, fp8, a.N, a.Kdim, a.ksplit);
  p.a_max = 16 * p.mt;
  p.need_b = p.mt < 4 && T > p.a_max;   // a group may outgrow region A
  // The tiled kernel pays only when groups are large on average (T*K/E_phys
  // >= 64 rows, prefill); at decode sizes a few hot groups above 64 rows
  // occupy too few workgroups in a launch of their own (measured on the
  // replica workload: 1036 -> 970 us), so region B streams them, in passes.
  p.need_c = tiled && T > 64 && (int64_t)T * d->K >= (int64_t)64 * d->E_phys;
  // Groups large on average with region A alone streaming (no region B):
  // the few groups of at most a_max rows join the tiled launch, where they
  // overlap the large ones, instead of a streaming launch too small to fill
  // the GPU (DeepSeek-V3-shaped prefill T=8192: about 5 such experts)
  p.all_tiled = p.need_c && !p.need_b;
  return p;
}

moe_status_t launch_expert_gemm(const moe_desc_t* d, const moe_route_t* r, int32_t T, StreamArgs a,
                                bool fp8, int mode, dim3 stream_grid, hipStream_t stream) {
  const GemmPlan pl = plan_expert_gemm(d, T, a, fp8, mode);
  const int mt = pl.mt, a_max = pl.a_max;
  const bool need_b = pl.need_b, need_c = pl.need_c;
  a.nblk = stream_nblk(d, T, a, fp8);
  stream_grid.x = a.N / (64 * a.nblk);
  a.max_rows = (need_b || need_c) ? a_max : 0;
  a.b_rows = 0;
  a.shared_chunks = 1;
  a.b_max_rows = 0;
  a.compact_rows = 0;
  // Few tokens (T*K below the slot count): launch T*K rows for the routed
  // slots instead of one per slot, most of which would find no tokens; each
  // row walks the slots that have tokens (received counts may fill more
  // slots than T*K, and the walk covers them too)
  const int64_t TKc = (int64_t)T * d->K;
  if (!need_b && !need_c && TKc >= 1 && TKc < d->E_phys && stream_compacts(fp8) &&
      stream_grid.y == (unsigned)(d->E_phys + d->n_shared)) {
    a.compact_rows = (int)TKc;
    stream_grid.y = (unsigned)(TKc + d->n_shared);
  }
  dim3 grid = stream_grid;
  if (need_b) {
    a.b_max_rows = need_c ? 64 : 0;
    // the shared expert's T rows, when region B takes them, are split into
    // passes on separate workgroup rows
    const bool shared_in_b = d->n_shared && (a.b_max_rows == 0 || T <= a.b_max_rows);
    const int tb = stream_tiles_b(fp8);
    a.shared_chunks = shared_in_b ? ((T + 15) / 16 + tb - 1) / tb : 1;
    a.b_rows = d->E_phys + d->n_shared * a.shared_chunks;
    grid.y += a.b_rows;
  }
  const bool all_tiled = pl.all_tiled;
  if (!all_tiled) {
    hipError_t e = launch_ffn_stream(a, fp8, d->w_packed, mode, mt, grid, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (!need_c) return MOE_OK;
  TiledArgs ta = {};
  ta.s = a;
  ta.tile_off = r->tile_off;
  ta.claim = r->claim;
  ta.variant = tiled_variant(d);
  ta.min_rows = all_tiled ? 0 : (mt < 4) ? 64 : a_max;
  // X holds the layer input (T rows) when gathering, else the grouped buffer
  ta.x_bytes = (a.gather_src ? (int64_t)T : moe_buffer_rows(d)) * a.ldx * 2;
  // static bound on the live row tiles: a routed layout holds T*K rows in
  // at most E_phys groups; received counts (moe_route_received) fill up to
  // M_max rows of every slot whatever T*K is
  const int64_t TK = (int64_t)T * d->K;
  int64_t routed_tiles = (TK + kTileRows - 1) / kTileRows + d->E_phys;
  if (d->layout == MOE_MASKED)
    routed_tiles = std::max(routed_tiles, (int64_t)d->E_phys * ((d->M_max + kTileRows - 1) / kTileRows));
  const int64_t max_tiles = routed_tiles + (d->n_shared ? (T + kTileRows - 1) / kTileRows : 0);
  return hip_status(launch_ffn_tiled(ta, fp8, d->w_packed, mode, (int)max_tiles, stream));
}

StreamArgs ffn_base_args(const moe_desc_t* d, const moe_route_t* r, int32_t T) {
  StreamArgs a = {};
  a.E_phys = d->E_phys; a.T = T; a.layout = d->layout; a.M_max = d->M_max;
  a.shared_base = routed_cap(d);
  a.counts = r->counts; a.masked_m = r->masked_m; a.spill_off = r->spill_off; a.pad_off = r->pad_off;
  a.ksplit = 1;
  a.nblk = 1;
  return a;
}

StreamArgs gate_up_args(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r, int32_t T,
                        const void* X, bool gather, void* h) {
  StreamArgs g1 = ffn_base_args(d, r, T);
  g1.X = static_cast<const uint16_t*>(X); g1.ldx = d->H; g1.Kdim = d->H; g1.N = d->I;
  if (gather) { g1.gather_src = r->src_of; g1.gather_off = r->offsets; }
  g1.W = w->w1; g1.W3 = w->w3; g1.S = w->s1; g1.S3 = w->s3;
  g1.SW = w->sw1; g1.SW3 = w->sw3; g1.SS = w->ss1; g1.SS3 = w->ss3;
  g1.out = h; g1.ldo = d->I;
  return g1;
}

StreamArgs down_args(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r, int32_t T,
                     const void* h, void* y) {
  const int splits = moe_down_splits(d, T);
  StreamArgs g2 = ffn_base_args(d, r, T);
  g2.X = static_cast<const uint16_t*>(h); g2.ldx = d->I; g2.Kdim = d->I; g2.N = d->H;
  g2.W = w->w2; g2.S = w->s2; g2.SW = w->sw2; g2.SS = w->ss2;
  g2.out = y; g2.ldo = d->H; g2.ksplit = splits; g2.out_f32 = splits > 1;
  g2.split_stride = moe_buffer_rows(d) * d->H;
  return g2;
}

CombineArgs combine_args(const moe_desc_t* d, const moe_route_t* r, int32_t T, const void* y, void* out) {
  const int splits = moe_down_splits(d, T);
  CombineArgs a = {};
  a.y = y; a.y_f32 = splits > 1; a.splits = splits; a.split_stride = moe_buffer_rows(d) * d->H;
  a.T = T; a.K = d->K; a.H = d->H; a.rows = moe_buffer_rows(d);
  a.slot_of = r->slot_of; a.topk_w = r->topk_w;
  a.n_shared = d->n_shared; a.shared_base = routed_cap(d);
  a.out = out; a.out_f32 = d->act_dtype == MOE_F32;
  return a;
}

// gate/up from the grouped buffer (gather = false: X = xg, by slot) or
// straight from the layer input (gather = true: X = x, by token)
moe_status_t gate_up_impl(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                          int32_t T, const void* X, bool gather, void* h, hipStream_t stream) {
  moe_status_t st = ffn_common_checks(d, w, r, T);
  if (st != MOE_OK) return st;
  if (gather && d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const bool fp8 = d->w_dtype == MOE_FP8E4M3_B128;
  if (!X || !h || !w->w1 || !w->w3) return MOE_ERR_ARG;
  if (fp8 && (!w->s1 || !w->s3)) return MOE_ERR_ARG;
  if (d->n_shared && (!w->sw1 || !w->sw3)) return MOE_ERR_ARG;
  const StreamArgs g1 = gate_up_args(d, w, r, T, X, gather, h);
  return launch_expert_gemm(d, r, T, g1, fp8, MODE_GATEUP, dim3(d->I / 64, d->E_phys + d->n_shared, 1),
                            stream);
}

}  // namespace

extern "C" {

moe_status_t moe_expert_gate_up(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                                int32_t T, const void* xg, void* h, hipStream_t stream) {
  return gate_up_impl(d, w, r, T, xg, false, h, stream);
}

moe_status_t moe_expert_gate_up_x(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                                  int32_t T, const void* x, void* h, hipStream_t stream) {
  return gate_up_impl(d, w, r, T, x, true, h, stream);
}

moe_status_t moe_expert_down(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                             int32_t T, const void* h, void* y, hipStream_t stream) {
  moe_status_t st = ffn_common_checks(d, w, r, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const bool fp8 = d->w_dtype == MOE_FP8E4M3_B128;
  if (!h || !y || !w->w2) return MOE_ERR_ARG;
  if (fp8 && !w->s2) return MOE_ERR_ARG;
  if (d->n_shared && !w->sw2) return MOE_ERR_ARG;
  const StreamArgs g2 = down_args(d, w, r, T, h, y);
  return launch_expert_gemm(d, r, T, g2, fp8, MODE_DOWN, dim3(d->H / 64, d->E_phys + d->n_shared, g2.ksplit),
                            stream);
}

moe_status_t moe_grouped_ffn(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                             int32_t T, const void* xg, void* h, void* y, hipStream_t stream) {
  moe_status_t st = moe_expert_gate_up(d, w, r, T, xg, h, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down(d, w, r, T, h, y, stream);
}

moe_status_t moe_grouped_ffn_x(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                               int32_t T, const void* x, void* h, void* y, hipStream_t stream) {
  moe_status_t st = moe_expert_gate_up_x(d, w, r, T, x, h, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down(d, w, r, T, h, y, stream);
}

const char* moe_expert_kernel(const moe_desc_t* d, int32_t T, int32_t which) {
  if (moe_check_desc(d) != MOE_OK || T <= 0 || T > d->T_max || (which != 0 && which != 1)) return "none";
  const bool fp8 = d->w_dtype == MOE_FP8E4M3_B128;
  moe_route_t r = {};                          // table pointers are not read here
  moe_weights_t w = {};
  const bool gather = d->act_dtype == MOE_BF16;
  const StreamArgs a = which == 0 ? gate_up_args(d, &w, &r, T, nullptr, gather, nullptr)
                                  : down_args(d, &w, &r, T, nullptr, nullptr);
  const GemmPlan pl = plan_expert_gemm(d, T, a, fp8, which == 0 ? MODE_GATEUP : MODE_DOWN);
  if (!pl.need_c) return "ffn_stream_kernel";
  TiledArgs ta = {};
  ta.s = a;
  ta.x_bytes = (which == 0 && gather ? (int64_t)T : moe_buffer_rows(d)) * a.ldx * 2;
  ta.variant = tiled_variant(d);
  return tiled_kernel_name(tiled_choice(ta, d->w_packed, which == 0 ? MODE_GATEUP : MODE_DOWN));
}

moe_status_t moe_quantize_1x128(const void* src, int64_t ld, int64_t rows, int32_t C, void* q,
                                float* s, hipStream_t stream) {
  if (rows < 0 || C < 128 || C % 128 || ld < C) return MOE_ERR_ARG;
  if (rows == 0) return MOE_OK;
  if (!src || !q || !s) return MOE_ERR_ARG;
  QuantArgs a;
  a.src = static_cast<const uint16_t*>(src); a.ld = ld; a.rows = rows; a.C = C;
  a.q = static_cast<uint8_t*>(q); a.s = s;
  return hip_status(launch_quant_1x128(a, stream));
}

}  // extern "C"

namespace {

moe_status_t a8_checks(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r, int32_t T) {
  moe_status_t st = ffn_common_checks(d, w, r, T);
  if (st != MOE_OK) return st;
  if (d->w_dtype != MOE_FP8E4M3_B128) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

A8Args a8_base_args(const moe_desc_t* d, const moe_route_t* r, int32_t T) {
  A8Args a = {};
  a.E_phys = d->E_phys; a.T = T; a.layout = d->layout; a.M_max = d->M_max; a.n_shared = d->n_shared;
  a.shared_base = routed_cap(d);
  a.counts = r->counts; a.masked_m = r->masked_m; a.spill_off = r->spill_off; a.pad_off = r->pad_off;
  a.ksplit = 1;
  a.nblk = 1;
  return a;
}

// 64-row output blocks per W8A8 workgroup: as the streaming kernel's fp8 rule
// (stream_nblk), several blocks walked as one pipeline of at most 64 K steps
// while at least 6144 workgroups remain.  MOE_DEBUG_NBLK_MASK overrides it.
int a8_nblk(const moe_desc_t* d, int32_t T, const A8Args& a) {
  const int nblocks = a.N / 64;
  const int steps = a.Kdim / 128 / a.ksplit;
  if (const int v = debug_nblk(d, nblocks)) return v;
  const int64_t TK = (int64_t)T * d->K;
  const int64_t groups = (TK < d->E_phys ? TK : d->E_phys) + d->n_shared;
  int nb = 1;
  while (nb < 8 && steps * nb * 2 <= 64 && nblocks % (nb * 2) == 0 &&
         groups * (nblocks / (nb * 2)) * a.ksplit >= 6144)
    nb *= 2;
  return nb;
}

// The W8A8 kernel for large groups (ffn_a8_tall_kernel) takes a launch when
// groups are large on average (the bf16 rule of plan_expert_gemm: T > 64 and
// T*K >= 64 E_phys), the weights are packed and the route table has its
// claim counters; MOE_DEBUG_A8_STREAM keeps the streaming kernel.
bool a8_tall_wanted(const moe_desc_t* d, const moe_route_t* r, int32_t T) {
  const int v = (int)(((uint32_t)d->debug_flags & MOE_DEBUG_TILED_MASK) >> MOE_DEBUG_TILED_SHIFT);
  return v != MOE_DEBUG_A8_STREAM && d->w_packed && r->claim && r->tile_off && T > 64 &&
         (int64_t)T * d->K >= (int64_t)64 * d->E_phys;
}

// Weight tiles a W8A8 large-group work item walks as one pipeline: doubled
// while the item runs fewer than 48 K stages (each item pays its set-up and
// the pipeline's fill once), at most 8, dividing the tile count.  Measured on
// the DeepSeek-V3-shaped fp8 prefill (one box): down (16 stages a tile)
// 2396 us unwalked, 2282 walking 2, 2219-2272 walking 4; gate/up (56 stages)
// 3766 us unwalked, 3801-3918 walking 2 or 4.  MOE_DEBUG_NBLK_MASK overrides
// it (an override that does not divide the tile count leaves the call on the
// streaming kernel).
int a8_walk(const moe_desc_t* d, int mode, int N, int Kdim) {
  const int tiles = N / (mode == MODE_GATEUP ? 64 : 128);
  if (const int v = (int)((uint32_t)d->debug_flags & MOE_DEBUG_NBLK_MASK)) return v;
  int w = 1;
  while (w < 8 && tiles % (2 * w) == 0 && w * (Kdim / 128) < 48) w *= 2;
  return w;
}

}  // namespace

extern "C" {

moe_status_t moe_expert_gate_up_a8(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                                   int32_t T, const void* xq, const float* xs, void* h,
                                   hipStream_t stream) {
  moe_status_t st = a8_checks(d, w, r, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!xq || !xs || !h || !w->w1 || !w->w3 || !w->s1 || !w->s3) return MOE_ERR_ARG;
  if (d->n_shared && (!w->sw1 || !w->sw3)) return MOE_ERR_ARG;
  A8Args a = a8_base_args(d, r, T);
  a.X = static_cast<const uint8_t*>(xq); a.ldx = d->H; a.XS = xs;
  a.gather_src = r->src_of; a.gather_off = r->offsets;
  a.Kdim = d->H; a.N = d->I;
  a.W = static_cast<const uint8_t*>(w->w1); a.W3 = static_cast<const uint8_t*>(w->w3);
  a.S = w->s1; a.S3 = w->s3;
  a.SW = static_cast<const uint8_t*>(w->sw1); a.SW3 = static_cast<const uint8_t*>(w->sw3);
  a.SS = w->ss1; a.SS3 = w->ss3;
  a.out = h; a.ldo = d->I;
  if (a8_tall_wanted(d, r, T)) {
    const A8TallArgs ta = {a, r->tile_off, r->claim, T, a8_walk(d, MODE_GATEUP, a.N, a.Kdim)};
    if (a8_tall_supported(MODE_GATEUP, ta)) return hip_status(launch_ffn_a8_tall(ta, MODE_GATEUP, stream));
  }
  a.nblk = a8_nblk(d, T, a);
  return hip_status(launch_ffn_a8(a, d->w_packed, MODE_GATEUP, stream));
}

moe_status_t moe_expert_down_a8(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                                int32_t T, const void* hq, const float* hs, void* y,
                                hipStream_t stream) {
  moe_status_t st = a8_checks(d, w, r, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!hq || !hs || !y || !w->w2 || !w->s2) return MOE_ERR_ARG;
  if (d->n_shared && !w->sw2) return MOE_ERR_ARG;
  const int splits = moe_down_splits(d, T);
  A8Args a = a8_base_args(d, r, T);
  a.X = static_cast<const uint8_t*>(hq); a.ldx = d->I; a.XS = hs;
  a.Kdim = d->I; a.N = d->H;
  a.W = static_cast<const uint8_t*>(w->w2); a.S = w->s2;
  a.SW = static_cast<const uint8_t*>(w->sw2); a.SS = w->ss2;
  a.out = y; a.ldo = d->H; a.ksplit = splits; a.out_f32 = splits > 1;
  a.split_stride = moe_buffer_rows(d) * d->H;
  if (a8_tall_wanted(d, r, T)) {
    const A8TallArgs ta = {a, r->tile_off, r->claim, moe_buffer_rows(d), a8_walk(d, MODE_DOWN, a.N, a.Kdim)};
    if (a8_tall_supported(MODE_DOWN, ta)) return hip_status(launch_ffn_a8_tall(ta, MODE_DOWN, stream));
  }
  a.nblk = a8_nblk(d, T, a);
  return hip_status(launch_ffn_a8(a, d->w_packed, MODE_DOWN, stream));
}

moe_status_t moe_grouped_ffn_a8(const moe_desc_t* d, const moe_weights_t* w, const moe_route_t* r,
                                int32_t T, const void* x, void* xq, float* xs, void* h, void* hq,
                                float* hs, void* y, hipStream_t stream) {
  moe_status_t st = a8_checks(d, w, r, T);
  if (st != MOE_OK) return st;
  if (d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  st = moe_quantize_1x128(x, d->H, T, d->H, xq, xs, stream);
  if (st != MOE_OK) return st;
  st = moe_expert_gate_up_a8(d, w, r, T, xq, xs, h, stream);
  if (st != MOE_OK) return st;
  st = moe_quantize_1x128(h, d->I, moe_buffer_rows(d), d->I, hq, hs, stream);
  if (st != MOE_OK) return st;
  return moe_expert_down_a8(d, w, r, T, hq, hs, y, stream);
}

const char* moe_expert_kernel_a8(const moe_desc_t* d, int32_t T, int32_t which) {
  if (moe_check_desc(d) != MOE_OK || T <= 0 || T > d->T_max || (which != 0 && which != 1)) return "none";
  if (d->w_dtype != MOE_FP8E4M3_B128) return "none";
  static int32_t tiles = 0;
  static uint32_t counters = 0;
  moe_route_t r = {};
  r.tile_off = &tiles;                         // only their presence is read here
  r.claim = &counters;
  if (!a8_tall_wanted(d, &r, T)) return "ffn_a8_kernel";
  A8Args a = a8_base_args(d, &r, T);
  if (which == 0) {
    a.ldx = d->H; a.Kdim = d->H; a.N = d->I;
  } else {
    a.ldx = d->I; a.Kdim = d->I; a.N = d->H;
    a.ksplit = moe_down_splits(d, T);
    a.out_f32 = a.ksplit > 1;
  }
  const int mode = which == 0 ? MODE_GATEUP : MODE_DOWN;
  const A8TallArgs ta = {a, r.tile_off, r.claim, which == 0 ? (int64_t)T : (int64_t)moe_buffer_rows(d),
                         a8_walk(d, mode, a.N, a.Kdim)};
  return a8_tall_supported(mode, ta) ? "ffn_a8_tall_kernel" : "ffn_a8_kernel";
}

moe_status_t moe_combine(const moe_desc_t* d, const moe_route_t* r, int32_t T, const void* y,
                         void* out, hipStream_t stream) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (T < 0 || T > d->T_max || !route_ptrs_ok(d, r)) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!y || !out) return MOE_ERR_ARG;
  return hip_status(launch_combine(combine_args(d, r, T, y, out), stream));
}

moe_status_t moe_forward(const moe_desc_t* d, const void* x, const void* w_router,
                         const float* bias, const int32_t* l2p, const int32_t* replica_count,
                         const moe_weights_t* w, int32_t T, float* logits, const moe_route_t* r,
                         void* ws, size_t ws_bytes, void* xg, void* h, void* y, void* out,
                         hipStream_t stream) {
  moe_status_t st = moe_router_route(d, x, w_router, bias, T, logits, l2p, replica_count, r, ws, ws_bytes,
                                     stream);
  if (st != MOE_OK) return st;
  if (d->act_dtype == MOE_BF16) {
    // the expert kernel gathers its rows from x; xg is not used
    st = moe_grouped_ffn_x(d, w, r, T, x, h, y, stream);
  } else {
    st = moe_permute(d, x, T, r, xg, stream);
    if (st != MOE_OK) return st;
    st = moe_grouped_ffn(d, w, r, T, xg, h, y, stream);
  }
  if (st != MOE_OK) return st;
  return moe_combine(d, r, T, y, out, stream);
}

size_t moe_decode_fused_workspace_bytes(const moe_desc_t* d) {
  if (moe_check_desc(d) != MOE_OK) return 0;
  const size_t act = sizeof(int32_t) * (1 + (size_t)d->E_phys);
  return kFusedSyncBytes + (act + 255) / 256 * 256;
}

moe_status_t moe_decode_fused(const moe_desc_t* d, const void* x, const void* w_router, const float* bias,
                              const moe_grouped_router_t* g, const int32_t* l2p,
                              const int32_t* replica_count, const moe_weights_t* w, int32_t T,
                              float* logits, const moe_route_t* r, void* ws, size_t ws_bytes, void* h,
                              void* y, void* out, void* fws, size_t fws_bytes, hipStream_t stream) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if (d->act_dtype != MOE_BF16 || d->w_packed != 1) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || T > d->T_max) return MOE_ERR_ARG;
  if (T > kFusedMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (!x || !w_router || !logits || !h || !y || !out || !fws) return MOE_ERR_ARG;
  RouteArgs ra;
  st = route_args(d, logits, T, g, nullptr, l2p, replica_count, r, ws, ws_bytes, ra);
  if (st != MOE_OK) return st;
  st = ffn_common_checks(d, w, r, T);
  if (st != MOE_OK) return st;
  const bool fp8 = d->w_dtype == MOE_FP8E4M3_B128;
  if (!w->w1 || !w->w3 || !w->w2) return MOE_ERR_ARG;
  if (fp8 && (!w->s1 || !w->s3 || !w->s2)) return MOE_ERR_ARG;
  if (d->n_shared && (!w->sw1 || !w->sw3 || !w->sw2)) return MOE_ERR_ARG;
  const int variant = decode_fused_variant(d->E, g != nullptr);
  if (variant < 0) return MOE_ERR_UNSUPPORTED;
  if (fws_bytes < moe_decode_fused_workspace_bytes(d)) return MOE_ERR_WORKSPACE;
  FusedArgs f = {};
  f.router = RouterArgs{x, 0, static_cast<const uint16_t*>(w_router), bias, T, d->E, d->H, logits};
  f.router_mfma = router_uses_mfma(d->E, d->H, 0);
  f.route = ra;
  f.route_variant = variant;
  f.g1 = gate_up_args(d, w, r, T, x, true, h);
  f.g2 = down_args(d, w, r, T, h, y);
  f.comb = combine_args(d, r, T, y, out);
  f.no_wait = ((uint32_t)d->debug_flags & MOE_DEBUG_FUSED_NO_WAIT) ? 1 : 0;
  f.sync = static_cast<uint32_t*>(fws);
  f.act = reinterpret_cast<int32_t*>(static_cast<char*>(fws) + kFusedSyncBytes);
  return hip_status(launch_decode_fused(f, fp8, stream));
}

moe_status_t moe_pack_weights(const moe_desc_t* d, int32_t which, int32_t G, const void* src,
                              void* dst, hipStream_t stream) {
  moe_status_t st = moe_check_desc(d);
  if (st != MOE_OK) return st;
  if ((which != 0 && which != 1) || G < 0 || (G > 0 && (!src || !dst)) || src == dst) return MOE_ERR_ARG;
  const int N = which == 0 ? d->I : d->H, Kdim = which == 0 ? d->H : d->I;
  return hip_status(launch_pack(src, dst, G, N, Kdim, d->w_dtype == MOE_FP8E4M3_B128, stream));
}

moe_status_t moe_ep_local_map(int32_t n_global, int32_t ep_size, int32_t rank, int32_t layout,
                              int32_t* local_of, int32_t* n_local) {
  if (!local_of || n_global < 1 || ep_size < 1 || rank < 0 || rank >= ep_size) return MOE_ERR_ARG;
  if (layout != MOE_EP_LINEAR && layout != MOE_EP_ROUND_ROBIN) return MOE_ERR_ARG;
  int n = 0;
  if (layout == MOE_EP_LINEAR) {
    // contiguous runs; the first n_global % ep_size ranks take one more slot
    const int base = n_global / ep_size, rem = n_global % ep_size;
    const int first = rank * base + (rank < rem ? rank : rem);
    const int count = base + (rank < rem ? 1 : 0);
    for (int p = 0; p < n_global; ++p) local_of[p] = (p >= first && p < first + count) ? p - first : -1;
    n = count;
  } else {
    for (int p = 0; p < n_global; ++p) local_of[p] = (p % ep_size == rank) ? n++ : -1;
  }
  if (n_local) *n_local = n;
  return MOE_OK;
}

moe_status_t moe_eplb_plan(const double* load, int32_t E, int32_t n_redundant, int32_t ep_size,
                           int32_t* p2l) {
  if (!load || !p2l || E < 1 || n_redundant < 0 || ep_size < 1) return MOE_ERR_ARG;
  const int64_t n = (int64_t)E + n_redundant;
  if (n % ep_size || n > kMaxE) return MOE_ERR_ARG;
  for (int l = 0; l < E; ++l)
    if (!(load[l] >= 0.0) || !std::isfinite(load[l])) return MOE_ERR_ARG;
  // replicas: each redundant slot to the largest load per replica (lowest id on ties)
  std::vector<int> rep(E, 1);
  for (int i = 0; i < n_redundant; ++i) {
    int best = 0;
    double bv = load[0] / rep[0];
    for (int l = 1; l < E; ++l) {
      const double v = load[l] / rep[l];
      if (v > bv) { bv = v; best = l; }
    }
    ++rep[best];
  }
  // longest processing time first: replicas in descending load per replica
  // (lower expert, then replica order, on ties), each to the least loaded
  // rank with a free slot, preferring ranks without a copy of that expert
  struct Item { double w; int l, j; };
  std::vector<Item> items;
  items.reserve(n);
  for (int l = 0; l < E; ++l)
    for (int j = 0; j < rep[l]; ++j) items.push_back({load[l] / rep[l], l, j});
  std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) {
    if (x.w != y.w) return x.w > y.w;
    if (x.l != y.l) return x.l < y.l;
    return x.j < y.j;
  });
  const int S = int(n / ep_size);
  std::vector<std::vector<int>> slots(ep_size);
  std::vector<double> total(ep_size, 0.0);
  for (const Item& it : items) {
    int pick = -1;
    bool pick_fresh = false;
    for (int r = 0; r < ep_size; ++r) {
      if ((int)slots[r].size() >= S) continue;
      const bool fresh = std::find(slots[r].begin(), slots[r].end(), it.l) == slots[r].end();
      if (pick < 0 || (fresh && !pick_fresh) || (fresh == pick_fresh && total[r] < total[pick])) {
        pick = r;
        pick_fresh = fresh;
      }
    }
    slots[pick].push_back(it.l);
    total[pick] += it.w;
  }
  for (int r = 0; r < ep_size; ++r)
    for (int i = 0; i < S; ++i) p2l[(int64_t)r * S + i] = slots[r][i];
  return MOE_OK;
}

moe_status_t moe_replica_map_from_p2l(const int32_t* p2l, int32_t E, int32_t E_phys,
                                      int32_t max_replicas, int32_t* l2p_out, int32_t* count_out) {
  if (!p2l || !l2p_out || !count_out || E < 1 || E_phys < E || max_replicas < 1) return MOE_ERR_ARG;
  for (int64_t i = 0; i < (int64_t)E * max_replicas; ++i) l2p_out[i] = -1;
  for (int l = 0; l < E; ++l) count_out[l] = 0;
  for (int p = 0; p < E_phys; ++p) {
    const int l = p2l[p];
    if (l < 0 || l >= E) return MOE_ERR_ARG;
    if (count_out[l] >= max_replicas) return MOE_ERR_ARG;
    l2p_out[(int64_t)l * max_replicas + count_out[l]] = p;
    count_out[l] += 1;
  }
  for (int l = 0; l < E; ++l)
    if (count_out[l] < 1) return MOE_ERR_ARG;
  return MOE_OK;
}

}  // extern "C"
