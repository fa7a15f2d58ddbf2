// Internal launch interface between the C ABI (moe_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- routing ----------------------------------------------------------------

struct RouteWs {            // views into the caller's route workspace
  int32_t* local_rank;      // [T_max*K] rank of choice i among earlier tokens
                            //           of its 64-token block that chose the
                            //           same logical expert
  int32_t* blk;             // [nblk*E] per-block counts -> exclusive prefixes
  int32_t* blk_flags;       // [nblk] non-finite flag per block
  int32_t* tok_flag;        // [T_max] non-finite flag per token
  int32_t* map_valid;       // [1] bit 0: a replica map is given and valid;
                            //     bit 1: the local map is valid
};

struct RouteArgs {
  const float* logits; int T, E, E_phys, K;
  const int32_t* l2p; const int32_t* rcount; int max_replicas;
  // expert-parallel share: global physical slot -> local slot or -1 (null:
  // every slot local, n_global == E_phys)
  const int32_t* local_of; int n_global;
  int layout, M_max, BM;
  int64_t routed_cap;       // rows of the routed part of the grouped buffer
  // outputs
  int32_t* topk_ids; float* topk_w; int32_t* topk_phys; int32_t* row_of;
  int32_t* slot_of; int32_t* src_of; int32_t* counts; int32_t* offsets;
  int32_t* masked_m; int32_t* spill_off; int32_t* pad_off; int32_t* tile_off; uint32_t* status;
  uint32_t* claim;          // [MOE_CLAIM_WORDS] zeroed here (may be null)
  int n_shared;
  RouteWs ws;
  // grouped sigmoid router (selection phase only); grouped == 0: softmax top-K
  int grouped, n_group, topk_group, group_k, renormalize;
  const float* score_bias; float scale;
};

hipError_t launch_route(const RouteArgs& a, hipStream_t s);

struct ReceivedArgs {
  const int32_t* counts_in; int E_phys, M_max, T, n_shared;
  int32_t* counts; int32_t* masked_m; int32_t* offsets; int32_t* spill_off; int32_t* tile_off;
  uint32_t* status;
  uint32_t* claim;          // [MOE_CLAIM_WORDS] zeroed here (may be null)
};
hipError_t launch_route_received(const ReceivedArgs& a, hipStream_t s);

// ---- permute / combine -------------------------------------------------------

struct PermuteArgs {
  const void* x; int act_f32; int T, K, H;
  const int32_t* slot_of; int64_t shared_base; int n_shared; int64_t rows;
  uint16_t* xg;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);

struct CombineArgs {
  const void* y; int y_f32; int splits; int64_t split_stride;  // elements
  int T, K, H; int64_t rows;
  const int32_t* slot_of; const float* topk_w;
  int n_shared; int64_t shared_base;
  void* out; int out_f32;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// ---- streaming grouped GEMM (decode FFN and router logits) ---------------------

enum { MODE_GATEUP = 0, MODE_DOWN = 1 };

struct StreamArgs {
  const uint16_t* X; int64_t ldx;   // bf16 rows
  // Gather (gate/up only): when gather_src is set, X is the layer input
  // [T, H] and rank r of routed group g reads row gather_src[gather_off[g] + r]
  // (the route tables' src_of and offsets); rank r of the shared expert
  // reads row r.  Otherwise X is the grouped buffer, indexed by slot.
  const int32_t* gather_src; const int32_t* gather_off;
  int Kdim, N;                       // reduction length, output features
  int E_phys, T, layout, M_max; int64_t shared_base;
  const int32_t* counts; const int32_t* masked_m; const int32_t* spill_off;
  const int32_t* pad_off;
  const void* W; const void* W3; const float* S; const float* S3;        // routed
  const void* SW; const void* SW3; const float* SS; const float* SS3;    // shared
  void* out; int64_t ldo; int64_t split_stride; int out_f32;
  int ksplit;         // K splits over grid.z
  int nblk;           // consecutive 64-row output blocks per workgroup (1..8); grid.x = N / (64 * nblk)
  // Two size classes share one launch; grid.y = b_rows + E_phys + n_shared.
  // Region B, the first b_rows rows of grid.y (dispatched first): groups with
  // more than max_rows rows (and at most b_max_rows; 0 = no limit),
  // stream_tiles_b(fp8) row tiles per pass; its first n_shared * shared_chunks
  // rows are the shared expert, whose passes are dealt over shared_chunks
  // workgroup rows.
  // Region A, the rest: groups with at most max_rows rows (0 = no limit).
  int max_rows;
  int b_rows, shared_chunks, b_max_rows;
  // compact_rows > 0 (no region B): region A's first compact_rows workgroup
  // rows take the slots with tokens, in slot order, row y the y-th, the
  // (y + compact_rows)-th, ... (any number of them), and the next n_shared
  // rows the shared expert; 0: row y is slot y
  int compact_rows;
};

// row tiles per pass of region B
inline int stream_tiles_b(int fp8) { return fp8 ? 2 : 4; }
// whether a launch with these arguments keeps its activations in LDS, and
// whether launches of this weight type take compact rows (StreamArgs)
bool stream_uses_xl(int fp8, int mode, int mt, const StreamArgs& a);
bool stream_compacts(int fp8);
// mt: row tiles per pass of region A (1, 2 or 4); grid.x = N / (64 * nblk)
hipError_t launch_ffn_stream(const StreamArgs& a, int fp8, int packed, int mode, int mt, dim3 grid,
                             hipStream_t s);

// ---- LDS-tiled grouped GEMM (large groups) ------------------------------------

constexpr int kTileRows = 256;     // token rows per work item of the large-group kernels

struct TiledArgs {
  StreamArgs s;
  const int32_t* tile_off;   // [E_phys + 2] prefix of ceil(rows / kTileRows) per group
  int min_rows;              // groups with at most this many rows are skipped
  int64_t x_bytes;           // bytes of the activation rows X addresses (rows * ldx * 2)
  int variant;               // 0: the launcher's choice; else a MOE_DEBUG_TILED_* kernel
  uint32_t* claim;           // [MOE_CLAIM_WORDS] work-claim counters, zero on entry and on
                             // exit (null: one workgroup per work item)
};
// largest MOE_DEBUG_TILED_* value
constexpr int kTiledVariants = 5;
bool tiled_supported(int mode, int fp8, int N, int Kdim, int ksplit);
// the MOE_DEBUG_TILED_* kernel a launch with these arguments runs, and its name
int tiled_choice(const TiledArgs& a, int packed, int mode);
const char* tiled_kernel_name(int choice);
hipError_t launch_ffn_tiled(const TiledArgs& a, int fp8, int packed, int mode, int max_tiles,
                            hipStream_t s);

// row-major [G, N, Kdim] weights -> the packed layout the kernels stream
hipError_t launch_pack(const void* src, void* dst, int G, int N, int Kdim, int fp8, hipStream_t s);

// ---- W8A8 (fp8 activations) ----------------------------------------------------

struct QuantArgs {            // rows of bf16 [rows, C] (row stride ld) -> E4M3FN codes
  const uint16_t* src; int64_t ld; int64_t rows; int C;   //   [rows, C] and fp32 scales
  uint8_t* q; float* s;                                     //   [rows, C / 128]
};
hipError_t launch_quant_1x128(const QuantArgs& a, hipStream_t s);

struct A8Args {
  const uint8_t* X; int64_t ldx; const float* XS;   // fp8 rows (natural K order), scales [rows, Kdim/128]
  const int32_t* gather_src; const int32_t* gather_off;   // as StreamArgs (gate/up only)
  int Kdim, N;
  int E_phys, T, layout, M_max, n_shared; int64_t shared_base;
  const int32_t* counts; const int32_t* masked_m; const int32_t* spill_off; const int32_t* pad_off;
  const uint8_t* W; const uint8_t* W3; const float* S; const float* S3;        // routed
  const uint8_t* SW; const uint8_t* SW3; const float* SS; const float* SS3;    // shared
  void* out; int64_t ldo; int64_t split_stride; int out_f32; int ksplit;
  int nblk;           // consecutive 64-row output blocks per workgroup (1..8); grid.x = N / (64 * nblk)
};
hipError_t launch_ffn_a8(const A8Args& a, int packed, int mode, hipStream_t s);

// W8A8 for large groups: one persistent launch over every group's
// (256-row tile, weight tile) units, packed weights, no K split.
struct A8TallArgs {
  A8Args s;
  const int32_t* tile_off;   // [E_phys + 2] prefix of ceil(rows / kTileRows) per group
  uint32_t* claim;           // [MOE_CLAIM_WORDS] work-claim counters, zero on entry and on exit
  int64_t x_rows;            // rows of X and XS the launch may address
  int walk;                  // weight tiles one work item runs as one pipeline (1..8, dividing their count)
};
bool a8_tall_supported(int mode, const A8TallArgs& a);
// compute units of the current device (0 if the query fails)
int device_cus();
hipError_t launch_ffn_a8_tall(const A8TallArgs& a, int mode, hipStream_t s);

// ---- router logits --------------------------------------------------------------

struct RouterArgs {
  const void* x; int x_f32; const uint16_t* w; const float* bias; int T, E, H; float* logits;
};
hipError_t launch_router(const RouterArgs& a, hipStream_t s);
bool router_uses_mfma(int E, int H, int x_f32);

// the router for T <= 64 with each tile's H slices over several workgroups;
// ws: its arrival counts (zero on entry, left zero), then the partial tiles
int router_split_count(int E, int H, int x_f32, int T);
size_t router_split_bytes(int E, int H, int x_f32, int T_max);
hipError_t launch_router_split(const RouterArgs& a, void* ws, int T_max, hipStream_t s);

// router logits, then routing: one launch when T * E <= kTinyRouterItems
// (softmax top-K, E <= 64, no expert-parallel map), else the two launches
constexpr int kTinyRouterItems = 16;
bool router_route_fits(const RouterArgs& ra, const RouteArgs& a);
// split_ws: the split router's workspace (router_split_bytes for T_max), or null
hipError_t launch_router_route(const RouterArgs& ra, const RouteArgs& a, void* split_ws, int T_max, hipStream_t s);

// ---- persistent single-launch decode layer --------------------------------------

// Fused workspace: barrier words, then the slot list.  Lines of 64 words:
// line 0 the top arrival counter, line 1 the abort word, lines 2..9 the
// first barrier's arrival counters (workgroup groups wg % 8), lines 10..17
// the later barriers' counters (one per XCD), lines 18..25 the number of
// workgroups on each XCD, then one 128-byte release flag per workgroup
// (kFusedMaxGrid of them), so that waiting workgroups poll different memory
// channels.
constexpr int kFusedMaxGrid = 2048;
constexpr int kFusedGroups = 8;                // XCDs (and first-barrier groups)
constexpr int kFusedLine = 64;                 // uint32 words per 256-byte line
constexpr int kFusedFlagStride = 32;           // uint32 words per release flag (128 bytes)
constexpr int kFusedFlagsOff = (2 + 3 * kFusedGroups) * kFusedLine;
constexpr size_t kFusedSyncBytes = sizeof(uint32_t) * ((size_t)kFusedFlagsOff + (size_t)kFusedMaxGrid * kFusedFlagStride);

struct FusedArgs {
  RouterArgs router; int router_mfma;   // logits phase (bf16 x)
  RouteArgs route; int route_variant;   // select shape: decode_fused_variant(E, grouped)
  StreamArgs g1, g2;                    // gate/up (gathering from x) and down, nblk = 1
  CombineArgs comb;
  uint32_t* sync;                       // barrier words (kFusedSyncBytes), zero-filled once
  int32_t* act;                         // [1 + E_phys] slots with tokens
  int no_wait;                          // MOE_DEBUG_FUSED_NO_WAIT: waits bounded at zero polls
  int grid, spin_limit;                 // set by the launcher
};
// -1: E (or the grouped router's E) too large for the single-workgroup route
int decode_fused_variant(int E, int grouped);
hipError_t launch_decode_fused(FusedArgs f, int fp8, hipStream_t s);

}  // namespace moe
