"""CPU reference (oracle) for one MoE layer forward: router -> top-K with
renormalised softmax -> per-expert counts and offsets -> expert-grouped rows
-> SwiGLU experts -> route-weighted combine.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU path
and imports nothing from it.

Written from the definitions on the pages, in plain numpy:
  * float64 for every floating-point value it computes, except the router
    logits, which are rounded to fp32 because the routing decision is defined
    on fp32 logits (the GPU takes the same decision in fp32);
  * no blocking, fusion or reordering beyond what the definition states.

Pages cited (titles and sections):
  [vllbc]  vllbc blog, "MoE inference and expert parallelism" -- routing /
           expert-FFN / "fused MoE" section with Table 3-1, and the vLLM
           forward-path section (topk -> align/sort -> GEMM1 -> act -> GEMM2
           -> moe_sum).
  [infra5] "推理 INFRA 方法论(5)" -- C(B), DeepGEMM (masked layout,
           masked_m, pad waste) sections.
  [eplb]   vLLM EPLB explainer -- section 1.2 (basic concepts: the three maps).
  [moonep] "MoonEP: dynamic redundant experts" -- the routing-count identity
           (sum_e T_e = RSK), the redundant-expert semantics (ids, weights and
           combine positions unchanged), the online-plan data flow (counts ->
           token offsets -> expert-grouped slots) and the zero-copy section.

Readings taken where the pages leave a step open (each is listed in the
design notes with its reason):
  R1 ties in top-K go to the lower expert id; -0.0 equals +0.0; a NaN logit
     ranks below every number (including -inf).
  R2 slot order inside a token's K choices is descending logit.
  R3 rows inside an expert group are in ascending token order (a stable
     counting sort by expert).
  R4 the shared expert has weight 1 and is added outside the top-K.
  R5 SwiGLU = SiLU(x W1^T) * (x W3^T), then W2^T; weights are stored
     [out, in] (W1, W3: [I, H]; W2: [H, I]).
  R6 masked overflow is never dropped: rows past M_max go to a spill region.
  R7 a replicated expert's tokens, in ascending token order, go round-robin
     over its replicas in logical_to_physical order.
  R8 an invalid replica map (a count outside [1, max_replicas], a slot
     outside [0, E_phys), or one slot listed twice) is ignored as a whole:
     every expert uses slot = its logical id, and status bit 1 is set.
  R13 grouped sigmoid router ([vllbc] routing section and Table 3-1: sigmoid
     scores, the correction bias only for choosing experts, weights from the
     unbiased scores; grouped top-k: first the best groups, then experts
     inside them): a score is the fp64 sigmoid of the fp32 logit rounded to
     fp32; the selection key is the fp32 sum score + bias.
  R14 groups are n_group runs of E/n_group consecutive expert ids; a group's
     score is the fp32 sum, in descending order, of its group_k largest
     selection keys (DeepSeek-V3's node-limited rule sums the K/M largest
     affinities of a node); the topk_group best groups are kept (ties to
     the lower group id), then the K best keys among their experts (ties to
     the lower expert id), in descending key order.
  R15 the weights are the chosen unbiased scores, divided by their sum when
     renormalising, times a scale factor (the routed scaling factor).
  R16 expert-parallel share of one GPU ([vllbc] EP section: expert_map, -1 =
     "not this rank's", zero local contribution, not a drop): a local map
     over the global physical slots gives each slot's local slot or -1; a
     choice whose slot is remote gets no row (row_of = slot_of = -1) and adds
     nothing to this GPU's output.  Replicas (R7) are taken over the global
     slots first.  An invalid local map (an entry outside [-1, E_phys) or a
     local slot listed twice) leaves no choice local and sets status bit 4.
  R17 EPLB replication ([eplb] section 1.3; [infra5] EPLB): each redundant
     slot goes, one at a time, to the logical expert with the largest load
     per replica (ties to the lower id).
  R18 EPLB packing ([infra5] EPLB: longest-processing-time bin packing): the
     replicas, each carrying load / replicas of its expert, are placed in
     descending load (ties: lower expert, then replica order) on the rank
     with the least load among those with a free slot and no replica of the
     same expert yet (if every rank with a free slot holds one, any rank with
     a free slot); ties to the lower rank.  Rank r owns global slots
     [r*S, (r+1)*S), S = (E + redundant) / ranks, filled in placement order.
  R20 W8A8 activations ([infra5] DeepGEMM section: FP8 operands with
     per-128 scales and two-level accumulation): each row's 128-wide K block
     is scaled by s = fp32(amax / 448) (1 for an all-zero block) and coded as
     E4M3FN of fp32(x / s), round to nearest even; the amax element codes to
     exactly +-448.
  R21 W8A8 product: y[t, n] = sum over K blocks b of sa[t, b] * sw[n/128, b]
     * (sum over k in b of dec(qa[t, k]) * dec(qw[n, k])) -- the per-block
     sum promoted to fp32 and scaled, then accumulated (two-level
     accumulation); the reference takes it exactly.
  R22 W8A8 layer: x is quantized per token (R20), gate/up use R21, h is
     rounded to bf16 (the layer's intermediate format) and quantized per row
     the same way for the down projection.
  R19 received counts ([infra5] DeepGEMM section: the dispatch's received
     count per local expert is masked_m): rows of local slot p sit at
     p*M_max + i, i < count; counts outside [0, M_max] are an error (status
     bit 5) and only min(count, M_max) rows are computed.

Parity pins: see tests/test_oracle_pins.py (brute force, a third-party
Mixtral MoE block, textbook sorts, page worked examples, closed forms).
"""
from __future__ import annotations

import numpy as np

STATUS_SPILL = 1        # bit 0: masked overflow went to the spill region
STATUS_BAD_REPLICA = 2  # bit 1: replica map entry invalid, home slot used
STATUS_NONFINITE = 4    # bit 2: a logit was NaN or infinite
STATUS_BAD_EP_MAP = 16  # bit 4: local map invalid, no choice is local (bit 3
                        # is the library's internal-index bit)
STATUS_RECV_OVERFLOW = 32  # bit 5: a received count above M_max


# --------------------------------------------------------------------------
# Number formats (decoders written from the format definitions)
# --------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  A bf16 value is the upper
    16 bits of the IEEE binary32 value with the same bits."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(q: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN bytes -> float64: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
    there is no infinity."""
    q = np.asarray(q).astype(np.int64)
    sign = np.where(q & 0x80, -1.0, 1.0)
    e = (q >> 3) & 0xF
    m = (q & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((q & 7) == 7), np.nan, val)
    return sign * val


# the value of each of the 256 codes by the definition above; decoding a
# matrix looks its codes up here instead of re-evaluating the definition
# per element (same values, a fraction of the time on large weights)
_E4M3_VALUES = _e4m3fn_value(np.arange(256))


def decode_e4m3fn(q: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN bytes (0..255) -> float64, per _e4m3fn_value."""
    return _E4M3_VALUES[np.asarray(q).astype(np.int64) & 0xFF]


def dequant_block128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """value[i, j] = e4m3(q[i, j]) * s[i // 128, j // 128], exact in float64
    (a 4-bit by 24-bit significand product).  [infra5] DeepGEMM section:
    128-wide blocks, each with one fp32 scale."""
    v = decode_e4m3fn(q)
    sf = np.asarray(s, dtype=np.float64)
    return v * np.repeat(np.repeat(sf, 128, axis=0), 128, axis=1)


# --------------------------------------------------------------------------
# W8A8: activation quantization and the two-level product  (R20 - R22)
# --------------------------------------------------------------------------

_E4M3_POS = None


def encode_e4m3fn(v: np.ndarray) -> np.ndarray:
    """Finite values -> OCP E4M3FN bytes: the nearest of the 127 non-negative
    finite codes (ties to the even code, i.e. even mantissa), magnitudes
    above 448 saturate to 448, the sign bit copied (-0 -> 0x80)."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = decode_e4m3fn(np.arange(127))          # ascending: 0 .. 448
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    code = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def quant_1x128(x: np.ndarray):
    """R20: rows of fp32-exact values [R, C] (C a multiple of 128) -> (codes
    uint8 [R, C], scales fp32 [R, C/128])."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    blk = x.reshape(R, C // 128, 128)
    amax = np.abs(blk).max(axis=2)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    v = (blk / s[:, :, None]).astype(np.float32)
    return encode_e4m3fn(v).reshape(R, C), s


def w8a8_matmul(qa: np.ndarray, sa: np.ndarray, qw: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """R21: qa [T, K] codes with sa [T, K/128]; qw [N, K] codes with sw
    [N/128, K/128].  Per-block sums, each scaled by sa * sw, then summed."""
    T, K = qa.shape
    N = qw.shape[0]
    A = decode_e4m3fn(qa).reshape(T, K // 128, 128).transpose(1, 0, 2)     # [b, T, 128]
    W = decode_e4m3fn(qw).reshape(N, K // 128, 128).transpose(1, 2, 0)     # [b, 128, N]
    part = np.matmul(A, W)                                                  # [b, T, N] block sums
    scale = (np.asarray(sa, np.float64).T[:, :, None] *
             np.repeat(np.asarray(sw, np.float64), 128, axis=0).T[:, None, :])
    return (part * scale).sum(axis=0)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Values -> nearest bf16 (ties to even), as float64, via fp32."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def swiglu_expert_w8a8(X: np.ndarray, codes) -> np.ndarray:
    """R22: codes = (q1, s1, q3, s3, q2, s2) of one expert (E4M3FN bytes and
    128x128 block scales)."""
    q1, s1, q3, s3, q2, s2 = codes
    qx, sx = quant_1x128(X)
    G = w8a8_matmul(qx, sx, q1, s1)
    U = w8a8_matmul(qx, sx, q3, s3)
    Hh = round_bf16(silu(G) * U)
    qh, sh = quant_1x128(Hh)
    return w8a8_matmul(qh, sh, q2, s2)


# --------------------------------------------------------------------------
# Router
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[e, h] (+ bias[e]), returned as fp32.
    [vllbc] routing section: the router gives one logit per expert per token.
    The bias is added before selection and weighting (workload reading)."""
    lg = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, np.float64)[None, :]
    return lg.astype(np.float32)


def topk_route(logits: np.ndarray, K: int):
    """Per token: the K largest fp32 logits (R1, R2) and their renormalised
    softmax weights  w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0)  over the K
    chosen logits (l_0 the largest).  This equals the softmax over all experts
    renormalised over the K chosen ([vllbc] routing section and Table 3-1:
    top-2 then softmax for Mixtral; softmax then renormalize in vLLM).

    Returns ids [T, K] int32, weights [T, K] float64, status bits."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    assert 1 <= K <= E
    v = lg.astype(np.float64) + 0.0            # -0.0 + 0.0 == +0.0
    nan = np.isnan(v)
    v = np.where(nan, 0.0, v)
    eid = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary -> not-NaN first, then value descending,
    # then id ascending
    order = np.lexsort((eid, -v, nan.astype(np.int8)), axis=-1)
    ids = order[:, :K].astype(np.int32)
    sel = np.take_along_axis(v, order[:, :K], axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    status = STATUS_NONFINITE if (~np.isfinite(lg)).any() else 0
    return ids, w, status


def sigmoid_scores_fp32(logits: np.ndarray) -> np.ndarray:
    """R13: s = 1 / (1 + exp(-l)) evaluated in fp64 on the fp32 logit, then
    rounded to fp32 (both sides of a routing comparison use these values)."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-l))).astype(np.float32)


def _desc_order(v: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Indices of v sorted by value descending (NaN last, -0 == +0), ties to
    the lower id: R1's order."""
    v64 = np.asarray(v, np.float64) + 0.0
    nan = np.isnan(v64)
    v64 = np.where(nan, 0.0, v64)
    return np.lexsort((ids, -v64, nan.astype(np.int8)))


def grouped_topk_route(logits: np.ndarray, K: int, n_group: int, topk_group: int, group_k: int,
                       score_bias: np.ndarray | None = None, renormalize: bool = True,
                       scale: float = 1.0):
    """Grouped sigmoid routing per token (R13-R15): scores, selection keys
    with the correction bias, group scores, the kept groups, the K chosen
    experts and their weights from the unbiased scores.

    Returns ids [T, K] int32, weights [T, K] float64, status bits."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    assert E % n_group == 0 and 1 <= topk_group <= n_group
    gsize = E // n_group
    assert 1 <= group_k <= gsize and 1 <= K <= topk_group * gsize
    s = sigmoid_scores_fp32(lg)
    b = np.zeros(E, np.float32) if score_bias is None else np.asarray(score_bias, np.float32)
    key = (s + b[None, :]).astype(np.float32)          # fp32 addition
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    for t in range(T):
        # group scores: the group_k largest keys of each group, summed in fp32
        # in descending order
        gscore = np.empty(n_group, np.float32)
        for g in range(n_group):
            vals = key[t, g * gsize:(g + 1) * gsize]
            top = vals[_desc_order(vals, np.arange(gsize))[:group_k]]
            acc = np.float32(top[0])
            for v in top[1:]:
                acc = np.float32(acc + v)
            gscore[g] = acc
        kept = _desc_order(gscore, np.arange(n_group))[:topk_group]
        cand = np.concatenate([np.arange(g * gsize, (g + 1) * gsize) for g in sorted(kept)])
        chosen = cand[_desc_order(key[t, cand], cand)[:K]]
        ids[t] = chosen
        sw = s[t, chosen].astype(np.float64)
        wt = sw / sw.sum() if renormalize else sw
        w[t] = wt * scale
    status = STATUS_NONFINITE if (~np.isfinite(lg)).any() else 0
    return ids, w, status


# --------------------------------------------------------------------------
# Replica maps  ([eplb] section 1.2; [moonep] redundant-expert semantics)
# --------------------------------------------------------------------------

def replica_tables(p2l: np.ndarray, E: int, max_replicas: int | None = None):
    """physical_to_logical_map [E_phys] -> (logical_to_physical_map
    [E, max_replicas] padded with -1, logical_replica_count [E]).  The
    replicas of a logical expert are listed in ascending physical slot."""
    p2l = np.asarray(p2l, dtype=np.int64)
    count = np.zeros(E, dtype=np.int32)
    for l in p2l:
        count[l] += 1
    R = int(count.max()) if max_replicas is None else max_replicas
    l2p = np.full((E, R), -1, dtype=np.int32)
    fill = np.zeros(E, dtype=np.int64)
    for p, l in enumerate(p2l):
        l2p[l, fill[l]] = p
        fill[l] += 1
    return l2p, count


def replica_map_valid(l2p: np.ndarray, count: np.ndarray, E_phys: int) -> bool:
    """R8: counts in [1, max_replicas], slots in [0, E_phys), no slot twice."""
    l2p = np.asarray(l2p)
    seen = set()
    for l in range(l2p.shape[0]):
        R = int(count[l])
        if R < 1 or R > l2p.shape[1]:
            return False
        for r in range(R):
            p = int(l2p[l, r])
            if not (0 <= p < E_phys) or p in seen:
                return False
            seen.add(p)
    return True


def assign_physical(ids: np.ndarray, E_phys: int, l2p: np.ndarray | None = None,
                    count: np.ndarray | None = None):
    # (E_phys: the slots the map may name -- the global slots under R16)
    """Physical slot of every (token, k) choice.  Without a map the slot is
    the logical id.  With a map (R7): the tokens that chose logical expert l,
    taken in ascending token order, are numbered j = 0, 1, ...; choice j goes
    to l2p[l][j mod R_l].  An invalid map follows R8."""
    ids = np.asarray(ids)
    T, K = ids.shape
    if l2p is None:
        return ids.astype(np.int32).copy(), 0
    if not replica_map_valid(l2p, count, E_phys):
        return ids.astype(np.int32).copy(), STATUS_BAD_REPLICA
    phys = np.empty_like(ids, dtype=np.int32)
    seen: dict[int, int] = {}
    for t in range(T):
        for k in range(K):
            l = int(ids[t, k])
            j = seen.get(l, 0)
            seen[l] = j + 1
            phys[t, k] = l2p[l, j % int(count[l])]
    return phys, 0


# --------------------------------------------------------------------------
# Expert-parallel share of one GPU and the EPLB plan  (R16 - R18)
# --------------------------------------------------------------------------

def ep_local_map(n_global: int, ep_size: int, rank: int, layout: str = "linear") -> np.ndarray:
    """[vllbc] EP section: the expert map of one rank over n_global slots --
    local slots numbered 0.. in slot order, -1 elsewhere.  "linear" cuts
    contiguous runs and the first n_global % ep_size ranks take one extra;
    "round_robin" deals slot p to rank p % ep_size."""
    local = np.full(n_global, -1, dtype=np.int32)
    if layout == "linear":
        base, rem = divmod(n_global, ep_size)
        start = rank * base + min(rank, rem)
        n = base + (1 if rank < rem else 0)
        local[start:start + n] = np.arange(n, dtype=np.int32)
    elif layout == "round_robin":
        mine = np.arange(rank, n_global, ep_size)
        local[mine] = np.arange(len(mine), dtype=np.int32)
    else:
        raise ValueError(layout)
    return local


def ep_map_valid(local_of: np.ndarray, E_phys: int) -> bool:
    """R16: entries in [-1, E_phys), no local slot named twice."""
    v = np.asarray(local_of, dtype=np.int64)
    if ((v < -1) | (v >= E_phys)).any():
        return False
    used = v[v >= 0]
    return len(np.unique(used)) == len(used)


def localize(phys_global: np.ndarray, local_of: np.ndarray, E_phys: int):
    """R16: each choice's local slot (-1 = another rank's)."""
    if not ep_map_valid(local_of, E_phys):
        return np.full_like(phys_global, -1, dtype=np.int32), STATUS_BAD_EP_MAP
    return np.asarray(local_of, dtype=np.int32)[phys_global], 0


def eplb_replicas(load: np.ndarray, n_redundant: int) -> np.ndarray:
    """R17: replica count per logical expert after handing out the redundant
    slots one at a time to the largest load per replica."""
    load = np.asarray(load, dtype=np.float64)
    rep = np.ones(len(load), dtype=np.int64)
    for _ in range(n_redundant):
        per = load / rep
        rep[int(np.argmax(per))] += 1        # argmax: first (lowest id) of the ties
    return rep


def eplb_plan(load: np.ndarray, n_redundant: int, ep_size: int) -> np.ndarray:
    """R17 + R18: physical_to_logical map over E + n_redundant global slots,
    rank r owning slots [r*S, (r+1)*S)."""
    load = np.asarray(load, dtype=np.float64)
    E = len(load)
    n = E + n_redundant
    if n % ep_size:
        raise ValueError("E + redundant must divide by the number of ranks")
    S = n // ep_size
    rep = eplb_replicas(load, n_redundant)
    items = [(load[l] / rep[l], l, j) for l in range(E) for j in range(rep[l])]
    items.sort(key=lambda it: (-it[0], it[1], it[2]))
    slots = [[] for _ in range(ep_size)]
    total = [0.0] * ep_size
    for wgt, l, _ in items:
        free = [r for r in range(ep_size) if len(slots[r]) < S]
        fresh = [r for r in free if l not in slots[r]]
        pool = fresh if fresh else free
        r = min(pool, key=lambda q: (total[q], q))
        slots[r].append(l)
        total[r] += wgt
    return np.array([l for r in range(ep_size) for l in slots[r]], dtype=np.int32)


def received_tables(counts: np.ndarray, M_max: int, tile_rows: int = 128):
    """R19: the masked tables of a buffer a dispatch filled -- masked_m =
    counts (an error above M_max), offsets = exclusive prefix of masked_m,
    no spill, and the prefix of ceil(rows / tile_rows) tiles."""
    counts = np.asarray(counts, dtype=np.int64)
    status = STATUS_RECV_OVERFLOW if ((counts > M_max) | (counts < 0)).any() else 0
    mm = np.clip(counts, 0, M_max)
    offsets = np.zeros(len(mm) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(mm)
    tiles = np.zeros(len(mm) + 1, dtype=np.int64)
    tiles[1:] = np.cumsum((mm + tile_rows - 1) // tile_rows)
    return dict(masked_m=mm.astype(np.int32), offsets=offsets.astype(np.int32),
                tile_off=tiles.astype(np.int32), status=status)


# --------------------------------------------------------------------------
# Counts, offsets and the expert-grouped order
# --------------------------------------------------------------------------

def group_rows(phys: np.ndarray, E_phys: int):
    """counts T_p = #{(t, k): phys = p}; offsets = exclusive prefix sum
    (E_phys + 1 entries, the cu_seqlens of [moonep] online plan);
    src_of[row] = token of each row of the expert-grouped order, a stable sort
    by slot (R3); row_of[t, k] = the row of choice (t, k).  [vllbc] vLLM
    forward path: sort token/expert pairs by expert.  Remote choices
    (phys = -1, R16) have no row: row_of = -1, and src_of holds the local
    rows only."""
    T, K = phys.shape
    flat = phys.reshape(-1).astype(np.int64)
    local = flat >= 0
    counts = np.bincount(flat[local], minlength=E_phys).astype(np.int32)
    offsets = np.zeros(E_phys + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    idx = np.nonzero(local)[0]
    order = idx[np.argsort(flat[idx], kind="stable")]
    src_of = (order // K).astype(np.int32)
    row_of = np.full(T * K, -1, dtype=np.int32)
    row_of[order] = np.arange(len(order), dtype=np.int32)
    return counts, offsets.astype(np.int32), row_of.reshape(T, K), src_of


def layout_masked(counts, offsets, row_of, phys, M_max: int, E_phys: int):
    """Static [E_phys, M_max] buffer with device-side valid counts masked_m
    ([infra5] DeepGEMM section) and, under R6, a spill region after it.
    rank = row_of - offsets[p]; slot = p*M_max + rank if rank < M_max, else
    E_phys*M_max + spill_off[p] + rank - M_max."""
    counts = np.asarray(counts, np.int64)
    masked_m = np.minimum(counts, M_max)
    spill_m = counts - masked_m
    spill_off = np.zeros(E_phys + 1, dtype=np.int64)
    spill_off[1:] = np.cumsum(spill_m)
    pl = np.maximum(phys, 0)                  # remote choices (R16): slot -1 below
    rank = row_of - offsets[pl]
    slot = np.where(rank < M_max, pl.astype(np.int64) * M_max + rank,
                    E_phys * M_max + spill_off[pl] + rank - M_max)
    slot = np.where(phys >= 0, slot, -1)
    status = STATUS_SPILL if spill_m.sum() > 0 else 0
    return (masked_m.astype(np.int32), spill_off.astype(np.int32),
            slot.astype(np.int32), status)


def layout_contig(counts, offsets, row_of, phys, BM: int):
    """Expert-grouped rows with each slot's segment padded to a multiple of BM
    ([vllbc] forward path: block-aligned and padded).  pad_off = exclusive
    prefix sum of ceil(T_p / BM) * BM; slot = pad_off[p] + rank."""
    counts = np.asarray(counts, np.int64)
    padded = (counts + BM - 1) // BM * BM
    pad_off = np.zeros(len(counts) + 1, dtype=np.int64)
    pad_off[1:] = np.cumsum(padded)
    pl = np.maximum(phys, 0)
    rank = row_of - offsets[pl]
    slot = np.where(phys >= 0, pad_off[pl] + rank, -1)
    return pad_off.astype(np.int32), slot.astype(np.int32)


# --------------------------------------------------------------------------
# Experts and combine
# --------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu_expert(X: np.ndarray, W1: np.ndarray, W3: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """(SiLU(X W1^T) * (X W3^T)) W2^T in float64 (R5; [vllbc] expert FFN:
    W1/W3 are gate/up, W2 is down)."""
    G = X @ W1.T
    U = X @ W3.T
    return (silu(G) * U) @ W2.T


def moe_forward(x, w_router, bias, K, E_phys, expert_weights, shared_weights=None,
                p2l=None, layout="contig", M_max=0, BM=16, logits=None,
                tokens=None, grouped=None, local_of=None, expert_codes=None, shared_codes=None):
    """The layer forward as defined: returns a dict with every intermediate.

    x [T, H] (values exactly as the layer receives them); w_router [E, H];
    expert_weights(p) -> (W1 [I,H], W3 [I,H], W2 [H,I]) float64 for physical
    slot p; shared_weights the same triple or None.  ``logits`` (fp32), if
    given, replaces the router step (routing parity is defined on the same
    fp32 logits).  ``tokens`` restricts the FFN and combine to a sample of
    token ids (routing still covers every token, as it must).  ``grouped``,
    a dict of grouped_topk_route's keyword arguments (n_group, topk_group,
    group_k, score_bias, renormalize, scale), selects the grouped sigmoid
    router instead of the softmax top-K.  ``local_of`` (R16), a local map
    over the global physical slots (the p2l slots, or the logical ids without
    one), makes this the output of one GPU's expert-parallel share: E_phys is
    then the number of local slots.  ``expert_codes(p)`` (and ``shared_codes``),
    the fp8 codes and block scales of slot p, select the W8A8 experts (R22)
    instead of the fp64 products of the dequantized weights.

    out[t] = S[t] + sum_k w[t, k] * Y[row_of[t, k]]   ([vllbc] combine:
    weight by g_i then sum the K results; R4 for S)."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = np.asarray(w_router).shape[0]
    if logits is None:
        logits = router_logits(x, w_router, bias)
    if grouped is None:
        ids, w, status = topk_route(logits, K)
    else:
        ids, w, status = grouped_topk_route(logits, K, **grouped)
    l2p = count = None
    if p2l is not None:
        l2p, count = replica_tables(p2l, E)
    n_slots = E_phys if local_of is None else len(local_of)
    phys, st = assign_physical(ids, n_slots, l2p, count)
    status |= st
    if local_of is not None:
        phys, st = localize(phys, local_of, E_phys)
        status |= st
    counts, offsets, row_of, src_of = group_rows(phys, E_phys)
    res = dict(logits=logits, ids=ids, w=w, phys=phys, counts=counts,
               offsets=offsets, row_of=row_of, src_of=src_of)
    if layout == "masked":
        masked_m, spill_off, slot_of, st = layout_masked(counts, offsets, row_of, phys, M_max, E_phys)
        status |= st
        res.update(masked_m=masked_m, spill_off=spill_off, slot_of=slot_of)
    else:
        pad_off, slot_of = layout_contig(counts, offsets, row_of, phys, BM)
        res.update(pad_off=pad_off, slot_of=slot_of)
    res["status"] = status

    want = np.arange(T) if tokens is None else np.asarray(tokens)
    need = np.zeros(T, dtype=bool)
    need[want] = True
    Y = np.zeros((T * K, H), dtype=np.float64)
    for p in range(E_phys):
        lo, hi = int(offsets[p]), int(offsets[p + 1])
        if hi == lo:
            continue
        rows = np.arange(lo, hi)
        rows = rows[need[src_of[lo:hi]]]
        if rows.size == 0:
            continue
        if expert_codes is not None:
            Y[rows] = swiglu_expert_w8a8(x[src_of[rows]], expert_codes(p))
        else:
            W1, W3, W2 = expert_weights(p)
            Y[rows] = swiglu_expert(x[src_of[rows]], W1, W3, W2)
    out = np.zeros((len(want), H), dtype=np.float64)
    if shared_codes is not None:
        out += swiglu_expert_w8a8(x[want], shared_codes)
    elif shared_weights is not None:
        out += swiglu_expert(x[want], *shared_weights)
    for k in range(K):
        r = row_of[want, k]
        out += np.where((r >= 0)[:, None], w[want, k][:, None] * Y[np.maximum(r, 0)], 0.0)
    res["out"] = out
    res["tokens"] = want
    return res


def bruteforce_forward(x, w_router, bias, K, expert_weights_logical, shared_weights=None,
                       logits=None):
    """Dense evaluation: every logical expert on every token, then a mask of
    route weights (m[t, e] = w[t, k] where ids[t, k] = e, else 0):
    out = S + sum_e m[:, e] * F_e(x).  Replicas do not appear: by the
    redundant-expert semantics ([moonep]) they leave the function unchanged."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = np.asarray(w_router).shape[0]
    if logits is None:
        logits = router_logits(x, w_router, bias)
    ids, w, _ = topk_route(logits, K)
    m = np.zeros((T, E))
    for t in range(T):
        for k in range(K):
            m[t, ids[t, k]] = w[t, k]
    out = np.zeros((T, H))
    if shared_weights is not None:
        out += swiglu_expert(x, *shared_weights)
    for e in range(E):
        out += m[:, e:e + 1] * swiglu_expert(x, *expert_weights_logical(e))
    return out


# --------------------------------------------------------------------------
# Accounting ([infra5] C(B) and DeepGEMM sections)
# --------------------------------------------------------------------------

def coverage(B: int, K: int, E: int) -> float:
    """C(B) = 1 - (1 - k/E)^B: expected fraction of experts a batch of B
    tokens touches when each token picks k of E uniformly."""
    return 1.0 - (1.0 - K / E) ** B


def pad_waste(M_e: int, BM: int) -> float:
    """FLOP waste of a tile-granular skip: ceil(M_e / BM) * BM / M_e."""
    return -(-M_e // BM) * BM / M_e


def expert_bytes(H: int, I: int, w_dtype: str) -> int:
    """Bytes of one SwiGLU expert (3 matrices of H*I) with block-128 scales
    for fp8."""
    if w_dtype == "bf16":
        return 3 * H * I * 2
    return 3 * H * I + 3 * (H // 128) * (I // 128) * 4
