/*
 * moe.h -- C ABI of a single-GPU fused MoE layer forward for MI355X (gfx950).
 *
 * The layer, as the pages define it:
 *   router logits -> top-K experts per token with renormalised softmax
 *   weights -> per-expert token counts T_e and prefix-sum offsets ->
 *   tokens permuted into expert-grouped rows -> grouped SwiGLU expert GEMMs
 *   (gate W1 / up W3, SiLU(gate)*up, down W2) -> route-weighted combine back
 *   into token order, plus an always-on shared expert of weight 1.
 * Sources: vllbc blog "MoE inference and expert parallelism" (routing and
 * expert-FFN section, Table 3-1; vLLM forward-path section), "推理 INFRA
 * 方法论(5)" (DeepGEMM section: static [E_loc, M_max, K] buffer with a
 * device-side masked_m), vLLM EPLB explainer section 1.2 (the three replica
 * maps), "MoonEP" (online-plan data flow; zero-copy lifetime).
 *
 * Conventions for every call below:
 *   - Memory: every pointer argument is caller-owned.  Arguments documented
 *     as "device" are device memory on the current HIP device; "host" are
 *     host memory.  The library never allocates, frees or synchronises.
 *   - Launches: calls only enqueue kernels on `stream`.  Grids depend on
 *     (desc, T) only, never on device-side counts, so a call sequence can be
 *     captured in a HIP graph.  No call records a memset.
 *   - Errors: argument errors are detected on the host before anything is
 *     enqueued and returned as MOE_ERR_ARG / MOE_ERR_UNSUPPORTED.  A failed
 *     kernel launch returns MOE_ERR_HIP.  Data-dependent conditions never
 *     trap: moe_route writes a status word (MOE_STATUS_* bits) that the
 *     caller may read after synchronising.
 *   - Validity: outputs stay valid until the next call writing the same
 *     buffers.  Rows of the grouped buffers (xg, h, y) that hold no token --
 *     masked rows past masked_m[p], contiguous pad rows -- are undefined and
 *     are never read into `out` (MoonEP zero-copy section: padding and the
 *     undefined tail are described by the plan).
 *   - Determinism: identical inputs give bit-identical outputs; no result
 *     depends on the order of atomic operations.
 *   - Thread safety: the library keeps no state; concurrent calls on
 *     distinct buffers are safe.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* NULL required pointer, bad size, T > T_max ... */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. H % 128 != 0) */
  MOE_ERR_WORKSPACE = 3,    /* workspace smaller than moe_route_workspace_bytes */
  MOE_ERR_HIP = 4           /* a HIP launch failed */
} moe_status_t;

typedef enum {
  MOE_F32 = 0,              /* IEEE binary32 */
  MOE_BF16 = 1,             /* bfloat16 */
  MOE_FP8E4M3_B128 = 2      /* OCP E4M3FN bytes + one fp32 scale per 128x128
                               block (DeepGEMM section: block-128 fp8) */
} moe_dtype_t;

typedef enum {
  MOE_CONTIG = 0,           /* expert-grouped rows, each segment padded to BM */
  MOE_MASKED = 1            /* static [E_phys, M_max] rows + spill region */
} moe_layout_t;

/* Bits of the device status word written by moe_route. */
#define MOE_STATUS_SPILL       1u  /* some T_p > M_max: rows went to the spill
                                      region (result still exact, no drop) */
#define MOE_STATUS_BAD_REPLICA 2u  /* replica map invalid (count outside
                                      [1, max_replicas], slot outside
                                      [0, E_phys), or a slot listed twice):
                                      the whole map is ignored and expert l
                                      uses slot l */
#define MOE_STATUS_NONFINITE   4u  /* a logit was NaN or +-inf; NaN ranks
                                      below every number, output unspecified */
#define MOE_STATUS_INTERNAL    8u  /* an index fell outside its buffer and the
                                      access was skipped (never expected) */
#define MOE_STATUS_BAD_EP_MAP  16u /* moe_route_ep: local map invalid (an entry
                                      outside [-1, E_phys) or a local slot
                                      named twice): no choice is local */
#define MOE_STATUS_RECV_OVERFLOW 32u /* moe_route_received: a count outside
                                      [0, M_max]; only min(count, M_max) rows
                                      of that slot are computed */
#define MOE_STATUS_SYNC_TIMEOUT 64u /* moe_decode_fused: a grid-barrier wait
                                      exceeded its bound (the grid was not
                                      resident at once); the call's outputs
                                      are incomplete and its fused workspace
                                      must be zero-filled again */

/* Layer description (host struct, copied by value into every call). */
typedef struct {
  int32_t T_max;        /* largest token count any call will pass */
  int32_t H;            /* hidden size; multiple of 128 */
  int32_t I;            /* expert intermediate size; multiple of 128 */
  int32_t E;            /* logical routed experts, 1..1024 */
  int32_t E_phys;       /* physical slots (>= E; == E without replicas); for
                           one rank's expert-parallel share (moe_route_ep) the
                           local slots, >= 1 */
  int32_t K;            /* experts per token, 1..min(E, 16) */
  int32_t n_shared;     /* 0 or 1 always-on shared expert */
  int32_t max_replicas; /* columns of logical_to_physical_map (>= 1) */
  int32_t act_dtype;    /* moe_dtype_t of x and out: MOE_F32 or MOE_BF16 */
  int32_t w_dtype;      /* moe_dtype_t of expert weights: MOE_BF16 or
                           MOE_FP8E4M3_B128 (router weights are always bf16) */
  int32_t layout;       /* moe_layout_t */
  int32_t M_max;        /* masked rows per slot, >= 1 (MOE_MASKED) */
  int32_t BM;           /* segment padding, >= 1 (MOE_CONTIG) */
  int32_t w_packed;     /* 0: expert weights row-major [out, in];
                           1: packed by moe_pack_weights */
  int32_t debug_flags;  /* 0 in normal use.  Test and ablation switches
                           (MOE_DEBUG_*): each selects a kernel variant
                           whose outputs are bit-identical to the default
                           choice, or forces a failure path from the host */
} moe_desc_t;

/* moe_desc_t.debug_flags.  Bits 0-3: 64-row output blocks per streaming or
 * W8A8 streaming workgroup (1..8 and dividing N/64), and weight tiles per work
 * item of the W8A8 large-group kernel (1..8 and dividing their number); 0 =
 * the library's choice.
 * Bits 4-7: the kernel for large groups (MOE_DEBUG_TILED_* for bf16
 * activations, MOE_DEBUG_A8_STREAM for W8A8; 0 = the library's choice).
 * Bit 8: moe_decode_fused bounds every grid-barrier wait at zero polls, so a
 * call aborts with MOE_STATUS_SYNC_TIMEOUT. */
#define MOE_DEBUG_NBLK_MASK        0xFu
#define MOE_DEBUG_TILED_SHIFT      4
#define MOE_DEBUG_TILED_MASK       0xF0u
#define MOE_DEBUG_TILED_NARROW     1  /* 128 x 256 tile, operands via registers */
#define MOE_DEBUG_TILED_WIDE_REGS  2  /* 128 x 512 tile, operands via registers */
#define MOE_DEBUG_TILED_WIDE_LDS   3  /* 128 x 512 tile, both operands by direct-to-LDS loads */
#define MOE_DEBUG_TILED_WIDE_HYB   4  /* 128 x 512 tile, weights to registers, activations via LDS */
#define MOE_DEBUG_TILED_TALL       5  /* 256 x 256 tile, every wave all 256 token rows */
#define MOE_DEBUG_A8_STREAM        6  /* W8A8: the streaming kernel for every group */
#define MOE_DEBUG_FUSED_NO_WAIT    0x100u

/* Routing tables, all device int32/float/uint32 arrays, caller-allocated.
 * Sizes: TK = T_max*K.  Choice i = t*K + k (k-th choice of token t). */
typedef struct {
  int32_t* topk_ids;   /* [TK] logical expert of choice i; per token in
                          descending logit order, ties to the lower id */
  float*   topk_w;     /* [TK] w = exp(l_k - l_0) / sum_j exp(l_j - l_0) */
  int32_t* topk_phys;  /* [TK] physical slot of choice i */
  int32_t* row_of;     /* [TK] row of choice i in the unpadded grouped order */
  int32_t* slot_of;    /* [TK] row of choice i in the layout's buffer */
  int32_t* src_of;     /* [TK] token of each unpadded grouped row */
  int32_t* counts;     /* [E_phys] T_p, tokens per physical slot */
  int32_t* offsets;    /* [E_phys+1] exclusive prefix sum of counts */
  int32_t* masked_m;   /* [E_phys] min(T_p, M_max)   (MOE_MASKED; else NULL ok) */
  int32_t* spill_off;  /* [E_phys+1] prefix sum of T_p - masked_m (MOE_MASKED) */
  int32_t* pad_off;    /* [E_phys+1] prefix sum of ceil(T_p/BM)*BM (MOE_CONTIG) */
  int32_t* tile_off;   /* [E_phys+2] work list of the large-group expert
                          kernels: prefix sum of ceil(T_p/256) over slots,
                          then the shared expert's ceil(T/256) tiles
                          (n_shared = 1) */
  uint32_t* status;    /* [1] MOE_STATUS_* bits of the last moe_route */
  uint32_t* claim;     /* [MOE_CLAIM_WORDS] work-claim counters of the
                          large-group expert kernels (NULL: those kernels
                          run one workgroup per work item instead).
                          moe_route* zero them; every expert call leaves
                          them zero when it ends, so expert calls that
                          share route tables must not overlap */
} moe_route_t;

#define MOE_CLAIM_WORDS 256

/* Expert weights, device memory.  Row-major layout [out, in] (row = output
 * feature), or the packed layout of moe_pack_weights when desc->w_packed:
 *   w1, w3: [E_phys, I, H]   (gate, up)     w2: [E_phys, H, I]   (down)
 *   bf16, or E4M3FN bytes with fp32 scales
 *   s1, s3: [E_phys, I/128, H/128]          s2: [E_phys, H/128, I/128]
 * Slot p holds the weights of logical expert physical_to_logical_map[p].
 * sw1/sw3/sw2 (+ ss*) are the shared expert ([I,H], [I,H], [H,I]), used when
 * n_shared == 1.  Scale pointers are ignored for bf16 weights. */
typedef struct {
  const void* w1; const void* w3; const void* w2;
  const float* s1; const float* s3; const float* s2;
  const void* sw1; const void* sw3; const void* sw2;
  const float* ss1; const float* ss3; const float* ss2;
} moe_weights_t;

/* ---- sizing (host, pure) ------------------------------------------------ */

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status_t s);

/* Validates a description; MOE_OK or the error the calls would return. */
moe_status_t moe_check_desc(const moe_desc_t* d);

/* Bytes of scratch device memory moe_route needs (for T = T_max): per
 * 64-token block, the counts of each expert and the rank of each choice
 * inside its block (the counting pass before the offsets; MoonEP online-plan
 * data flow: counts -> token offsets -> expert-grouped slots). */
size_t moe_route_workspace_bytes(const moe_desc_t* d);

/* The same number under the name the boundary's description uses. */
size_t moe_workspace_bytes(const moe_desc_t* d);

/* Bytes of ws that let moe_router_route split the router of T <= 64
 * tokens over more workgroups: moe_route_workspace_bytes(d), then the split
 * router's per-tile arrival counts and partial tiles (zero-filled by the
 * caller before first use; left zero by every call).  Equals
 * moe_route_workspace_bytes(d) when the split router never applies. */
size_t moe_router_route_workspace_bytes(const moe_desc_t* d);

/* Rows of the grouped buffers xg [rows, H], h [rows, I] and y ("推理 INFRA
 * 方法论(5)", DeepGEMM section: a static [E_loc, M_max, K] buffer whose valid
 * rows per expert masked_m gives at run time; vllbc blog, vLLM forward path:
 * contiguous groups padded to a block size): routed rows
 * (masked: E_phys*M_max + K*max(0, T_max - M_max) spill rows; contiguous:
 * T_max*K + E_phys*(BM-1)), then n_shared*T_max shared-expert rows. */
int64_t moe_buffer_rows(const moe_desc_t* d);

/* Row where the shared expert's rows start (= routed row capacity). */
int64_t moe_shared_base(const moe_desc_t* d);

/* Number of K-splits the down projection uses for T tokens.  With 1 split
 * y is bf16 [rows, H]; with S > 1 it is S fp32 partial sums [S, rows, H],
 * summed in split order by moe_combine.  Fewer tokens touch fewer slots, so
 * the split grows as T shrinks ("推理 INFRA 方法论(5)", C(B) section: the
 * decode batch reads the weights of the slots it touches). */
int32_t moe_down_splits(const moe_desc_t* d, int32_t T);

/* Bytes of y for T tokens.  This is not monotone in T: fewer tokens may use
 * more fp32 split planes.  A y buffer that serves calls with different T must
 * hold moe_y_bytes_max(d). */
size_t moe_y_bytes(const moe_desc_t* d, int32_t T);

/* The largest moe_y_bytes(d, T) over 1 <= T <= T_max (0 for an invalid
 * descriptor): the size of a y buffer allocated once for every call. */
size_t moe_y_bytes_max(const moe_desc_t* d);

/* ---- the hot path -------------------------------------------------------- */

/* a1. logits[t, e] = sum_h x[t, h] * w_router[e, h] (+ bias[e]), fp32
 * accumulation.  x: device [T, H] act_dtype; w_router: device [E, H] bf16;
 * bias: device [E] fp32 or NULL; logits: device [T, E] fp32.
 * (vllbc blog, routing section: one logit per expert per token.) */
moe_status_t moe_router_logits(const moe_desc_t* d, const void* x, const void* w_router,
                               const float* bias, int32_t T, float* logits,
                               hipStream_t stream);

/* a2-a4. From fp32 logits [T, E] (device): top-K ids and weights, per-slot
 * counts and offsets, the stable expert-grouped order (ascending token
 * inside each slot), and the layout tables.  With a replica map
 * (l2p: device [E, max_replicas] logical_to_physical_map, -1 padded;
 * replica_count: device [E] logical_replica_count; both NULL for none) the
 * tokens of logical expert l, in ascending token order, go round-robin over
 * l2p[l][0..count-1] (vLLM EPLB explainer 1.2; MoonEP: ids, weights and
 * combine positions unchanged).  ws: device scratch of at least
 * moe_route_workspace_bytes(d) bytes.  0 <= T <= T_max. */
moe_status_t moe_route(const moe_desc_t* d, const float* logits, int32_t T,
                       const int32_t* l2p, const int32_t* replica_count,
                       const moe_route_t* r, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* a1-a4 in one call: moe_router_logits (writing logits) then moe_route on
 * them, with the arguments, results and errors of the two calls.  With few
 * tokens and experts (T * E <= 16, E <= 64, the router's one-logit-per-
 * workgroup summation) both run in one workgroup of one launch, which saves
 * a launch on the decode path; the logits and every table are bit-identical
 * to the two calls.  (vllbc blog, routing section and Table 3-1.)
 * With ws_bytes >= moe_router_route_workspace_bytes(d), T <= 64 and the
 * MFMA router (E > 64, bf16 x, H % 1024 == 0), the router spreads each
 * 16 x 16 logit tile over several workgroups and adds their partial sums in
 * the single-launch order, so the logits stay bit-identical; the part of ws
 * past moe_route_workspace_bytes(d) bytes must then be zero-filled before
 * the first call, and every call leaves it zero again.  A smaller ws (at
 * least moe_route_workspace_bytes(d)) runs the plain router. */
moe_status_t moe_router_route(const moe_desc_t* d, const void* x, const void* w_router,
                              const float* bias, int32_t T, float* logits,
                              const int32_t* l2p, const int32_t* replica_count,
                              const moe_route_t* r, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* moe_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument.  The route workspace is a static device array of
 * MOE_NOALLOC_WORKSPACE_BYTES in the library, one copy per GPU, held until
 * the process ends; the call allocates and frees nothing.  Same tables,
 * conventions and errors as moe_route, plus MOE_ERR_WORKSPACE when
 * moe_route_workspace_bytes(d) exceeds that size and MOE_ERR_HIP when the
 * array's device address cannot be looked up.  The address is looked up on
 * a device's first call, with that device current: make that first call
 * outside graph capture.  Every call on one GPU shares that GPU's array, so
 * calls that may overlap on one GPU (different streams, graphs replayed
 * concurrently) race and must be serialised by the caller. */
#define MOE_NOALLOC_WORKSPACE_BYTES ((size_t)4 << 20)
moe_status_t moe_route_noalloc(const moe_desc_t* d, const float* logits, int32_t T,
                               const int32_t* l2p, const int32_t* replica_count,
                               const moe_route_t* r, hipStream_t stream);

/* Grouped sigmoid router (DeepSeek style; vllbc blog, routing section and
 * Table 3-1: sigmoid scores, a correction bias used only to choose experts,
 * weights from the unbiased scores, best groups first, then experts inside
 * them).  Per token: s_e = fp32 of the fp64 sigmoid of the fp32 logit;
 * selection key c_e = fp32(s_e + score_bias[e]); the E experts form n_group
 * groups of E/n_group consecutive ids, each scored by the fp32 sum, in
 * descending order, of its group_k largest keys; the topk_group best groups
 * are kept (ties to the lower group id) and the K largest keys among their
 * experts chosen (ties to the lower id), in descending key order; weight k
 * = s of choice k, divided by the sum of the K chosen s when renormalize is
 * set, times scale. */
typedef struct {
  const float* score_bias;   /* [E] device fp32, or NULL for none */
  int32_t n_group;           /* >= 1, divides E; E/n_group divides 64 */
  int32_t topk_group;        /* 1 .. n_group */
  int32_t group_k;           /* 1 .. min(8, E/n_group) */
  int32_t renormalize;       /* 0 or 1 */
  float scale;               /* finite */
} moe_grouped_router_t;

/* moe_route with the grouped sigmoid router in place of the softmax top-K:
 * same tables, conventions and errors; also MOE_ERR_ARG for a NULL g or
 * parameters outside the ranges above, MOE_ERR_UNSUPPORTED for K >
 * topk_group * E/n_group. */
moe_status_t moe_route_grouped(const moe_desc_t* d, const float* logits, int32_t T,
                               const moe_grouped_router_t* g,
                               const int32_t* l2p, const int32_t* replica_count,
                               const moe_route_t* r, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* ---- expert-parallel share of one GPU ------------------------------------
 * (vllbc blog, EP section: an expert map gives each global expert its local
 * slot on this rank, -1 for another rank's; -1 is not a drop: the choice adds
 * nothing here and is computed by the rank that owns it.  "推理 INFRA 方法论(5)",
 * DeepGEMM section: the dispatch's received count per local expert is the
 * masked GEMM's masked_m.) */

typedef struct {
  const int32_t* local_of;   /* [n_global] device: global physical slot ->
                                local slot in [0, E_phys), or -1 */
  int32_t n_global;          /* global physical slots: the slots l2p names,
                                or >= E without a replica map (slot = expert
                                id); <= 4096 */
} moe_ep_map_t;

/* moe_route (g == NULL) or moe_route_grouped (g != NULL) for one rank's share.
 * Top-K over all E experts as usual; each choice takes its global slot
 * (through the replica map if given, whose entries are global slots in
 * [0, n_global)), then its local slot local_of[global].  A choice with local
 * slot -1 gets topk_phys = row_of = slot_of = -1 (moe_permute and
 * moe_combine skip it); counts, offsets and the layout tables cover the local
 * slots only, so offsets[E_phys] <= T*K.  topk_ids and topk_w are those of
 * the full routing.  An invalid local map (an entry outside [-1, E_phys) or a
 * local slot named twice) leaves no choice local and sets
 * MOE_STATUS_BAD_EP_MAP.  Other conventions and errors as moe_route; also
 * MOE_ERR_ARG for a NULL ep or local_of, or n_global outside the range above. */
moe_status_t moe_route_ep(const moe_desc_t* d, const float* logits, int32_t T,
                          const moe_grouped_router_t* g, const moe_ep_map_t* ep,
                          const int32_t* l2p, const int32_t* replica_count,
                          const moe_route_t* r, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Route tables for a masked buffer that a dispatch has filled: rows of local
 * slot p at p*M_max + i, i < counts[p] (counts: [E_phys] device int32, the
 * received count per local expert).  Writes r->counts and r->masked_m
 * (min(max(counts, 0), M_max)), r->offsets (their exclusive prefix), r->
 * spill_off (zeros), r->tile_off (prefix of ceil(rows/256) tiles; the shared
 * expert's ceil(T/256) last when d->n_shared) and r->status
 * (MOE_STATUS_RECV_OVERFLOW if a count is outside [0, M_max]); the other
 * tables are left as they are.  moe_expert_gate_up / moe_expert_down then run
 * on the buffer as after moe_route + moe_permute (shared-expert rows, if any,
 * at moe_buffer_rows' routed capacity + t for t < T).  Masked layout only
 * (else MOE_ERR_UNSUPPORTED); one workgroup, enqueue-only, no host sync. */
moe_status_t moe_route_received(const moe_desc_t* d, const int32_t* counts, int32_t T,
                                const moe_route_t* r, hipStream_t stream);

typedef enum {
  MOE_EP_LINEAR = 0,         /* contiguous runs of slots per rank */
  MOE_EP_ROUND_ROBIN = 1     /* slot p on rank p % ep_size */
} moe_ep_layout_t;

/* Host helper: rank's local map over n_global slots (vllbc blog, EP section:
 * linear cuts contiguous runs and the first n_global % ep_size ranks take one
 * extra slot; round-robin deals the slots out in turn).  Local slots are
 * numbered 0.. in global slot order; local_of [n_global] (host) receives the
 * map, n_local (may be NULL) the number of local slots.  MOE_ERR_ARG for
 * n_global < 1, ep_size < 1, rank outside [0, ep_size) or an unknown layout. */
moe_status_t moe_ep_local_map(int32_t n_global, int32_t ep_size, int32_t rank, int32_t layout,
                              int32_t* local_of, int32_t* n_local);

/* Host helper: EPLB placement (vLLM EPLB explainer, section 1.3: redundant
 * slots replicate the hot experts; "推理 INFRA 方法论(5)", EPLB section:
 * replicate hot experts, then longest-processing-time bin packing).  load [E]
 * (host, finite, >= 0) is each logical expert's load.  Each of the n_redundant
 * extra slots goes to the expert with the largest load per replica (lowest id
 * on ties); then the replicas, each carrying load / replicas, are placed in
 * descending order (lower expert, then replica order, on ties) on the least
 * loaded rank that has a free slot, preferring ranks without a copy of that
 * expert (lowest rank on ties).  p2l [E + n_redundant] (host) receives the
 * physical_to_logical map with rank r owning slots [r*S, (r+1)*S), S =
 * (E + n_redundant) / ep_size, in placement order.  MOE_ERR_ARG for bad sizes,
 * E + n_redundant not divisible by ep_size or above 4096, or a bad load. */
moe_status_t moe_eplb_plan(const double* load, int32_t E, int32_t n_redundant, int32_t ep_size,
                           int32_t* p2l);

/* a5. Gathers token rows into the grouped buffer: xg[slot_of[t*K+k]] = x[t]
 * (cast to bf16 if x is fp32) and, with a shared expert,
 * xg[moe_shared_base + t] = x[t].  x: device [T, H] act_dtype;
 * xg: device [moe_buffer_rows, H] bf16.
 * (vllbc blog, vLLM forward-path section: after top-K the token rows are
 * sorted by expert and block-aligned before the first expert GEMM; MoonEP,
 * online-plan section: each token row is written to its slot of the
 * expert-grouped buffer at the offset the counts give.) */
moe_status_t moe_permute(const moe_desc_t* d, const void* x, int32_t T,
                         const moe_route_t* r, void* xg, hipStream_t stream);

/* a6 (+a8). Gate/up projection with the SwiGLU activation for every slot
 * with tokens, and for the shared expert over all T tokens:
 * h[row] = SiLU(xg[row] W1^T) * (xg[row] W3^T), fp32 accumulation, stored
 * bf16.  Slots with no token, and row tiles holding no valid row, issue no
 * MFMA and read no weights ("推理 INFRA 方法论(5)", DeepGEMM section: a tile
 * with m_blk*BM >= masked_m[e] is skipped).  fp8 weights are promoted with
 * their block scale every 128 K (the same section's two-level
 * accumulation).  xg: device [moe_buffer_rows, H] bf16;
 * h: device [moe_buffer_rows, I] bf16. */
moe_status_t moe_expert_gate_up(const moe_desc_t* d, const moe_weights_t* w,
                                const moe_route_t* r, int32_t T, const void* xg,
                                void* h, hipStream_t stream);

/* a5 + a6 (+a8) in one call, for bf16 activations: as moe_expert_gate_up,
 * but each group's rows are read straight from the layer input instead of a
 * grouped buffer -- rank r of slot p is token src_of[offsets[p] + r], rank
 * r of the shared expert token r -- so moe_permute and its buffer are not
 * needed (the gather of vllbc blog's forward path, fused into the expert
 * kernel).  x: device [T, H] bf16.  h as for moe_expert_gate_up (same
 * values).  MOE_ERR_UNSUPPORTED unless act_dtype is MOE_BF16. */
moe_status_t moe_expert_gate_up_x(const moe_desc_t* d, const moe_weights_t* w,
                                  const moe_route_t* r, int32_t T, const void* x,
                                  void* h, hipStream_t stream);

/* a7 (+a8). Down projection y[row] = h[row] W2^T for the same rows.
 * y: device, moe_y_bytes(d, T) bytes: bf16 [moe_buffer_rows, H] when
 * moe_down_splits(d, T) == 1, else that many fp32 partial planes (a buffer
 * reused across calls with different T: moe_y_bytes_max(d) bytes). */
moe_status_t moe_expert_down(const moe_desc_t* d, const moe_weights_t* w,
                             const moe_route_t* r, int32_t T, const void* h, void* y,
                             hipStream_t stream);

/* a6-a8 in one call: moe_expert_gate_up then moe_expert_down (vllbc blog,
 * vLLM forward-path section: GEMM1, activation, GEMM2 over the
 * expert-grouped rows; "推理 INFRA 方法论(5)", DeepGEMM section: one grouped
 * launch serves every expert, empty experts skipped). */
moe_status_t moe_grouped_ffn(const moe_desc_t* d, const moe_weights_t* w,
                             const moe_route_t* r, int32_t T, const void* xg,
                             void* h, void* y, hipStream_t stream);

/* a5-a8 in one call: moe_expert_gate_up_x then moe_expert_down (the same
 * passages as moe_grouped_ffn, with the gather of moe_permute inside). */
moe_status_t moe_grouped_ffn_x(const moe_desc_t* d, const moe_weights_t* w,
                               const moe_route_t* r, int32_t T, const void* x,
                               void* h, void* y, hipStream_t stream);

/* Name of the kernel that moe_expert_gate_up_x / moe_expert_gate_up (which
 * = 0) or moe_expert_down (which = 1) runs for the largest groups of a
 * T-token call: "ffn_stream_kernel" (decode-sized groups, weights streamed
 * once per group) or one of the large-group kernels ("ffn_whyb_kernel" ...).
 * A static string; "none" for an invalid descriptor, T outside [1, T_max]
 * or another `which`.  Host only, pure: profiles and benchmarks use it to
 * name the kernel they time. */
const char* moe_expert_kernel(const moe_desc_t* d, int32_t T, int32_t which);

/* The same for moe_expert_gate_up_a8 (which = 0) and moe_expert_down_a8
 * (which = 1) with route tables that hold claim counters:
 * "ffn_a8_tall_kernel" or "ffn_a8_kernel"; "none" as above and for weights
 * that are not fp8. */
const char* moe_expert_kernel_a8(const moe_desc_t* d, int32_t T, int32_t which);

/* ---- W8A8: fp8 activations on fp8 MFMA ------------------------------------
 * ("推理 INFRA 方法论(5)", DeepGEMM section: FP8 operands with per-128 scales
 * and two-level accumulation -- each 128-wide K block summed by the matrix
 * unit, promoted to fp32, scaled and accumulated.)  For fp8 weights
 * (MOE_FP8E4M3_B128; else MOE_ERR_UNSUPPORTED).  The W8A8 layer differs from
 * the W8A16 one (moe_grouped_ffn_x) by the activation quantization: a few
 * percent of the largest output on DeepSeek-V3 shapes, more than the 3e-2
 * bound of the fp8 path, so it is a separate, opt-in path. */

/* Each row's 128-wide blocks of a bf16 matrix [rows, C] (row stride ld
 * elements, C a multiple of 128): s = amax / 448 (1 for an all-zero block),
 * codes = E4M3FN of x / s (IEEE fp32 division, round to nearest even, clamped
 * to +-448).  q: device [rows, C] bytes (row stride C), natural K order; s:
 * device fp32 [rows, C/128].  Non-finite inputs give unspecified codes. */
moe_status_t moe_quantize_1x128(const void* src, int64_t ld, int64_t rows, int32_t C, void* q,
                                float* s, hipStream_t stream);

/* a6 with fp8 activations: xq / xs = moe_quantize_1x128 of the layer input x
 * [T, H]; rows are gathered by token (src_of) as moe_expert_gate_up_x does.
 * h as moe_expert_gate_up.  Decode-sized groups: a group's rows run in passes
 * of 16 (at most 16 rows) or 64, each pass streaming the group's weights.
 * Groups large on average (T > 64 and T*K >= 64 E_phys, the prefill case),
 * with packed weights, route tables holding claim counters, H a multiple of
 * 1024 (at most 16384) and I of 128: one persistent launch over 256-row tiles
 * of every group, each weight tile read once per 256 rows (the DeepGEMM
 * section's contiguous layout with large tiles).  Both kernels give the same
 * bits. */
moe_status_t moe_expert_gate_up_a8(const moe_desc_t* d, const moe_weights_t* w,
                                   const moe_route_t* r, int32_t T, const void* xq,
                                   const float* xs, void* h, hipStream_t stream);

/* a7 with fp8 activations: hq / hs = moe_quantize_1x128 of h over its
 * moe_buffer_rows(d) rows (C = I).  y as moe_expert_down (same K split).
 * The large-group kernel as for gate/up, where the call has no K split, I
 * is a multiple of 1024 (at most 16384) and H of 128. */
moe_status_t moe_expert_down_a8(const moe_desc_t* d, const moe_weights_t* w,
                                const moe_route_t* r, int32_t T, const void* hq,
                                const float* hs, void* y, hipStream_t stream);

/* a6-a8 with fp8 activations: quantize x, gate/up, quantize h, down.
 * Caller-owned scratch: xq [T_max, H] bytes, xs [T_max, H/128] fp32, hq
 * [moe_buffer_rows, I] bytes, hs [moe_buffer_rows, I/128] fp32; bf16
 * activations only (else MOE_ERR_UNSUPPORTED). */
moe_status_t moe_grouped_ffn_a8(const moe_desc_t* d, const moe_weights_t* w,
                                const moe_route_t* r, int32_t T, const void* x, void* xq,
                                float* xs, void* h, void* hq, float* hs, void* y,
                                hipStream_t stream);

/* a9. out[t] = sum_k topk_w[t,k] * y[slot_of[t*K+k]] (+ y[shared_base + t]),
 * in fp32 with k ascending, then rounded to act_dtype (RNE).
 * (vllbc blog, combine: weight by g_i, then sum the K results.)
 * y: device as produced by moe_grouped_ffn; out: device [T, H] act_dtype. */
moe_status_t moe_combine(const moe_desc_t* d, const moe_route_t* r, int32_t T,
                         const void* y, void* out, hipStream_t stream);

/* All five steps in order on one stream (same arguments as above): the
 * MoE layer forward of vllbc blog's routing / expert-FFN section (router,
 * top-K with renormalised softmax, SwiGLU experts, weighted sum) along the
 * vLLM forward path of the same page (topk -> align/sort -> GEMM1 -> act ->
 * GEMM2 -> moe_sum).  With bf16 activations the permute is fused into the
 * expert kernel (moe_grouped_ffn_x) and xg is not used (may be NULL).  y
 * must hold moe_y_bytes(d, T) bytes (moe_y_bytes_max(d) if T varies). */
moe_status_t moe_forward(const moe_desc_t* d, const void* x, const void* w_router,
                         const float* bias, const int32_t* l2p, const int32_t* replica_count,
                         const moe_weights_t* w, int32_t T, float* logits,
                         const moe_route_t* r, void* ws, size_t ws_bytes,
                         void* xg, void* h, void* y, void* out, hipStream_t stream);

/* Bytes of the fused workspace moe_decode_fused needs: grid-barrier words and
 * the list of slots with tokens (0 if the descriptor is invalid). */
size_t moe_decode_fused_workspace_bytes(const moe_desc_t* d);

/* The whole decode layer (router logits, routing, gate/up, down, combine) in
 * ONE persistent launch, for T <= 16 tokens: every buffer is the caller's and
 * preallocated, so the call can be recorded into a graph and replayed (the
 * low-latency decode path on fixed buffers: "推理 INFRA 方法论(5)", DeepEP
 * section; vllbc blog, Table 4-2).  Outputs -- logits, the route tables, h, y
 * and out -- are bit-identical to moe_router_logits, moe_route (g NULL) or
 * moe_route_grouped (g given), moe_grouped_ffn_x and moe_combine called with
 * the same arguments.
 *   x [T, H] bf16, w_router [E, H] bf16, bias [E] fp32 or NULL, g, l2p and
 *   replica_count as moe_route_grouped, w as moe_grouped_ffn, logits
 *   [T_max, E] fp32, r / ws / ws_bytes as moe_route, h [moe_buffer_rows, I]
 *   bf16, y moe_y_bytes(d, T), out [T, H] bf16: all device memory.
 *   fws: device, fws_bytes >= moe_decode_fused_workspace_bytes(d); zero-filled
 *   by the caller before the first call (and after a call whose status word
 *   has MOE_STATUS_SYNC_TIMEOUT), then left alone: each call leaves it ready
 *   for the next.  Calls that may overlap need workspaces of their own.
 * Requires bf16 activations and packed weights (w_packed = 1), and E <= 512
 * (softmax) or E <= 256 (grouped router); else MOE_ERR_UNSUPPORTED, as for
 * T > 16.  The launch holds every compute unit of the device until it ends;
 * its workgroups wait for one another, with each wait bounded (about a
 * second; MOE_DEBUG_FUSED_NO_WAIT in desc->debug_flags sets the bound to zero
 * polls), so work on other streams can only delay it.  Its grid barriers
 * write each XCD's L2 back once per barrier, from the XCD's last arrival,
 * relying on that writeback covering the stores of every workgroup on that
 * XCD (a property of gfx950's cache operations rather than of the HIP memory
 * model); the multi-launch chain relies on no such property and stays the
 * default path. */
moe_status_t moe_decode_fused(const moe_desc_t* d, const void* x, const void* w_router,
                              const float* bias, const moe_grouped_router_t* g,
                              const int32_t* l2p, const int32_t* replica_count,
                              const moe_weights_t* w, int32_t T, float* logits,
                              const moe_route_t* r, void* ws, size_t ws_bytes, void* h,
                              void* y, void* out, void* fws, size_t fws_bytes,
                              hipStream_t stream);

/* ---- weight layout ------------------------------------------------------ */

/* Repacks G expert matrices from row-major [G, N, Kdim] (row = output
 * feature) into the layout the expert kernels stream: for every 128-wide K
 * block (outer) and 16-row panel (inner), the 16-byte pieces each lane loads,
 * in lane order, so every load instruction of a wave reads 1 KiB of
 * contiguous memory.  The 16-byte piece of element (n, k) is
 *   ((g*(Kdim/128) + k/128)*(N/16) + n/16)*NI*64 + (kk/c)*64 + 16*((kk%c)/e) + n%16
 * with kk = k%128, c = 32 (bf16) or 64 (fp8), e = 8 or 16 elements per piece,
 * NI = 128/c, and the element sits at position kk%e inside the piece.
 * Same size as the input.  which = 0 for W1 or W3 (N = I, Kdim = H), 1 for
 * W2 (N = H, Kdim = I); element type from desc->w_dtype (fp8 scales are not
 * repacked).  src, dst: device, distinct; a one-time step, not on the hot
 * path.  Weights are an input the pages treat as given; packing changes
 * only their order in memory. */
moe_status_t moe_pack_weights(const moe_desc_t* d, int32_t which, int32_t G, const void* src,
                              void* dst, hipStream_t stream);

/* ---- replica maps (host, pure) ------------------------------------------- */

/* physical_to_logical_map p2l [E_phys] (host) -> logical_to_physical_map
 * l2p_out [E, max_replicas] (host, -1 padded, replicas in ascending slot) and
 * logical_replica_count count_out [E] (host).  MOE_ERR_ARG if an entry is
 * outside [0, E), a logical expert has no slot, or has more than
 * max_replicas.  (vLLM EPLB explainer, section 1.2.) */
moe_status_t moe_replica_map_from_p2l(const int32_t* p2l, int32_t E, int32_t E_phys,
                                      int32_t max_replicas, int32_t* l2p_out,
                                      int32_t* count_out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
