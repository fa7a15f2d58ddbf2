"""GPU parity: the HIP path through the C ABI against the CPU reference.

Routing tables must be bit-exact when both sides start from the same fp32
logits; layer outputs must satisfy max|d| / max|ref| <= 1e-2 (bf16 weights)
or 3e-2 (fp8 block-128 weights).  Small shapes span several tiles and a
ragged tail and are compared on every token; the full workload shapes are
compared on sampled tokens, in the launch configuration the benchmark uses.
"""
import zlib

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from routing_grouped_expert_router_amd import binding as B
from workloads import configs, generate
from gpu_util import (Built, TOL, rel_err, out_np, route_np, say, tile_off_expected, weight_tol, DEV,
                      covering_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_hygiene(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# small shapes: several 64-row weight blocks, several 16-row tiles, ragged tails
def small_configs():
    base = configs.tiny()
    return [
        base,
        base.with_(name="mixtral_small_masked", T=37, H=512, I=768, act_dtype="bf16", M_max=37),
        base.with_(name="mixtral_small_spill", T=37, H=512, I=768, act_dtype="bf16", M_max=5),
        base.with_(name="dsv3_small_fp8", T=45, H=1024, I=256, E=64, E_phys=64, K=8, n_shared=1,
                   act_dtype="bf16", w_dtype="fp8", M_max=45 * 8 // 64 * 4),
        base.with_(name="dsv3_small_fp8_contig", T=45, H=1024, I=256, E=64, E_phys=64, K=8,
                   n_shared=1, act_dtype="bf16", w_dtype="fp8", layout="contig", BM=16),
        base.with_(name="prefill_small", T=200, H=512, I=256, E=16, E_phys=16, K=4, n_shared=1,
                   act_dtype="bf16", layout="contig", BM=128, bias="normal0.5"),
        base.with_(name="replica_small", T=70, H=256, I=128, E=32, E_phys=40, K=4,
                   act_dtype="bf16", layout="contig", BM=16, bias="zipf1.1"),
        # groups of ~150 rows (masked: the masked/spill boundary falls inside
        # a tile of the tiled kernel)
        base.with_(name="tiled_masked_spill", T=300, H=256, I=256, E=4, E_phys=4, K=2,
                   act_dtype="bf16", M_max=100),
        base.with_(name="tiled_contig_shared", T=300, H=512, I=384, E=4, E_phys=4, K=2, n_shared=1,
                   act_dtype="bf16", layout="contig", BM=128, bias="normal0.5"),
        # fp8 with skewed groups: single-tile groups, hot groups of several
        # tiles (the large-group class) and a shared expert split over chunks
        base.with_(name="fp8_skewed_classes", T=100, H=512, I=256, E=32, E_phys=32, K=2, n_shared=1,
                   act_dtype="bf16", w_dtype="fp8", M_max=64, bias="zipf1.1"),
        # groups of ~300 rows with shapes the wide tiled kernel takes for both
        # projections (gate/up and down), masked with spill, shared expert
        base.with_(name="tiled_wide", T=600, H=512, I=512, E=4, E_phys=4, K=2, n_shared=1,
                   act_dtype="bf16", M_max=200),
        # groups large on average (T*K = 64*E) but skewed: rows per expert
        # 253, 6, 0, 165, 4, 58, 24, 2 and a 256-row shared expert, every
        # group (the empty one aside) in the tiled launch, tiny ones included
        base.with_(name="tiled_skewed_small_groups", T=256, H=512, I=512, E=8, E_phys=8, K=2, n_shared=1,
                   act_dtype="bf16", layout="contig", BM=128, bias="zipf1.1"),
    ]


SMALL = small_configs()
# every workload at its full size
FULL = [configs.mixtral_decode(1), configs.mixtral_decode(8), configs.mixtral_decode(32),
        configs.mixtral_decode(64), configs.dsv3_decode(32), configs.dsv3_decode(128),
        configs.dsv3_decode(256), configs.dsv3_prefill(), configs.replica_decode()]

TILED_VARIANTS = (B.MOE_DEBUG_TILED_NARROW, B.MOE_DEBUG_TILED_WIDE_REGS, B.MOE_DEBUG_TILED_WIDE_LDS,
                  B.MOE_DEBUG_TILED_WIDE_HYB, B.MOE_DEBUG_TILED_TALL)

ROUTE_KEYS = ["ids", "phys", "row_of", "slot_of", "src_of", "counts", "offsets"]


def check_route(b: Built, res: dict, wscale: float = 1.0):
    T, K = b.T, b.cfg.K
    g = route_np(b.layer.rt, T, K)
    for k in ROUTE_KEYS:
        assert np.array_equal(g[k], np.asarray(res[k]).reshape(g[k].shape)), k
    if b.cfg.layout == "masked":
        assert np.array_equal(g["masked_m"], res["masked_m"])
        assert np.array_equal(g["spill_off"], res["spill_off"])
    else:
        assert np.array_equal(g["pad_off"], res["pad_off"])
    assert np.array_equal(g["tile_off"], tile_off_expected(np.asarray(res["counts"]), T, b.cfg.n_shared))
    assert np.abs(g["w"] - res["w"]).max() <= weight_tol(K) * max(1.0, wscale)
    assert g["status"] == res["status"], (g["status"], res["status"])
    return g


def test_mfma_operand_layout_probe():
    """The one-expert, one-token layer is a dense SwiGLU of one row; exercising
    it at H = I = 128 checks the MFMA lane layout end to end on the smallest
    case (a wrong D layout scrambles columns; a wrong K pairing scrambles sums)."""
    cfg = configs.tiny().with_(name="probe", T=1, H=128, I=128, E=1, E_phys=1, K=1, act_dtype="bf16")
    b = Built(cfg)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    ref = b.oracle(lg)["out"]
    assert rel_err(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_route_and_layer_small(cfg, packed):
    b = Built(cfg, packed=packed)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    res = b.oracle(lg)
    check_route(b, res)
    e = rel_err(out, res["out"])
    say(f"  {cfg.name}: rel err {e:.3e}  status {res['status']}")
    assert e <= TOL[cfg.w_dtype]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_router_logits(cfg):
    b = Built(cfg)
    ref = b.oracle_logits().astype(np.float64)
    B.moe_router_logits(b.d, b.x, b.wr, b.bias, b.T, b.layer.logits)
    got = b.layer.logits[: b.T].cpu().numpy().astype(np.float64)
    from oracle_adapt import to_f64
    absdot = np.abs(to_f64(b.inp.x)) @ np.abs(to_f64(b.inp.w_router)).T
    bound = cfg.H * 2.0 ** -24 * absdot + 2.0 ** -24 * np.abs(ref) + 1e-30
    assert (np.abs(got - ref) <= bound).all(), float((np.abs(got - ref) / bound).max())


# few tokens and experts: moe_router_route runs the router and the routing
# in one launch while T * E <= 16 (the last case takes the two launches)
ROUTER_ROUTE = [
    configs.tiny().with_(name="rr_e8_t1_masked", T=1, H=4096, I=128, E=8, E_phys=8, K=2, act_dtype="bf16",
                         M_max=1, bias="normal0.5"),
    configs.tiny().with_(name="rr_e8_t2_f32_contig", T=2, H=1024, I=128, E=8, E_phys=8, K=2, act_dtype="f32",
                         layout="contig", BM=16),
    configs.tiny().with_(name="rr_e16_t1_replicas", T=1, H=512, I=128, E=16, E_phys=20, K=4, act_dtype="bf16",
                         layout="contig", BM=16, bias="zipf1.1"),
    configs.tiny().with_(name="rr_e8_t16_two_launches", T=16, H=512, I=128, E=8, E_phys=8, K=2,
                         act_dtype="bf16", M_max=16, bias="normal0.5"),
    # 12 and 4 items: router groups of three items and of one
    configs.tiny().with_(name="rr_e12_t1_three_items", T=1, H=2560, I=128, E=12, E_phys=12, K=3,
                         act_dtype="f32", layout="contig", BM=16, bias="normal0.5"),
    configs.tiny().with_(name="rr_e4_t1_one_item", T=1, H=768, I=128, E=4, E_phys=4, K=2,
                         act_dtype="bf16", M_max=1),
]
RR_KEYS = ("ids", "w", "phys", "row_of", "slot_of", "src_of", "counts", "offsets", "masked_m", "spill_off",
           "pad_off", "tile_off", "status")


@pytest.mark.parametrize("cfg", ROUTER_ROUTE, ids=lambda c: c.name)
def test_router_route_matches_two_calls(cfg):
    """moe_router_route equals moe_router_logits + moe_route bit for bit:
    the logits and every routing table, at T and at T = 0; its claim
    counters end zero."""
    b = Built(cfg)
    d, L = b.d, b.layer
    for T in (b.T, 0):
        B.moe_router_logits(d, b.x, b.wr, b.bias, T, L.logits)
        B.moe_route(d, L.logits, T, L.rt, L.ws, b.l2p, b.rcount)
        rt2 = B.RouteTables(d, DEV)
        rt2.claim.fill_(7)
        lg2 = torch.full_like(L.logits, float("nan"))
        ws2 = torch.empty_like(L.ws)
        B.moe_router_route(d, b.x, b.wr, b.bias, T, lg2, rt2, ws2, b.l2p, b.rcount)
        torch.cuda.synchronize()
        assert torch.equal(L.logits[:T], lg2[:T]), (cfg.name, T)
        ref, got = route_np(L.rt, T, cfg.K), route_np(rt2, T, cfg.K)
        for k in RR_KEYS:
            assert np.array_equal(np.asarray(ref[k]), np.asarray(got[k])), (cfg.name, T, k)
        assert not rt2.claim.any()
        say(f"  {cfg.name} T={T}: logits and tables bit-identical, status {got['status']}")


# up to 64 tokens and more than 64 experts: with the larger workspace the
# router spreads each 16 x 16 logit tile over 2..16 workgroups
ROUTER_SPLIT = [
    configs.tiny().with_(name="split_e256_t32_masked", T=32, H=7168, I=128, E=256, E_phys=256, K=8,
                         act_dtype="bf16", M_max=4, bias="normal0.5"),
    configs.tiny().with_(name="split_e256_t5_h4096", T=5, H=4096, I=128, E=256, E_phys=256, K=8,
                         act_dtype="bf16", M_max=4),
    configs.tiny().with_(name="split_e200_t37_contig", T=37, H=5120, I=128, E=200, E_phys=200, K=6,
                         act_dtype="bf16", layout="contig", BM=16, bias="zipf1.1"),
    configs.tiny().with_(name="split_e512_t64_contig", T=64, H=4096, I=128, E=512, E_phys=512, K=10,
                         act_dtype="bf16", layout="contig", BM=16),
]


@pytest.mark.parametrize("cfg", ROUTER_SPLIT, ids=lambda c: c.name)
def test_split_router_matches_two_calls(cfg):
    """moe_router_route with moe_router_route_workspace_bytes of zeroed ws
    (the split router) equals moe_router_logits + moe_route bit for bit, at
    T, at a smaller T right after, at T again (the arrival counts were left
    zero, the layout does not depend on T) and at T = 0."""
    b = Built(cfg)
    d, L = b.d, b.layer
    rbytes = B.route_workspace_bytes(d)
    assert B.router_route_workspace_bytes(d) > rbytes, cfg.name      # the split router applies
    ws_plain = torch.zeros(rbytes, dtype=torch.uint8, device=DEV)
    ws_split = torch.zeros(B.router_route_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    rt2 = B.RouteTables(d, DEV)
    for T in (b.T, max(1, b.T // 3), b.T, 0):
        lg1 = torch.full_like(L.logits, float("nan"))
        B.moe_router_logits(d, b.x, b.wr, b.bias, T, lg1)
        B.moe_route(d, lg1, T, L.rt, ws_plain, b.l2p, b.rcount)
        lg2 = torch.full_like(L.logits, float("nan"))
        B.moe_router_route(d, b.x, b.wr, b.bias, T, lg2, rt2, ws_split, b.l2p, b.rcount)
        torch.cuda.synchronize()
        assert torch.equal(lg1[:T], lg2[:T]), (cfg.name, T)
        ref, got = route_np(L.rt, T, cfg.K), route_np(rt2, T, cfg.K)
        for k in RR_KEYS:
            assert np.array_equal(np.asarray(ref[k]), np.asarray(got[k])), (cfg.name, T, k)
        ncount = 4 * ((cfg.E + 15) // 16) * ((min(b.T, 64) + 15) // 16)
        assert not ws_split[rbytes:rbytes + ncount].any(), (cfg.name, T)   # arrival counts back at zero
        say(f"  {cfg.name} T={T}: split router logits and tables bit-identical")


# many tokens and more than 64 experts: the 64-expert x 64-token block
# router (ragged token and expert counts: partial blocks on both axes)
ROUTER_BLOCK = [
    configs.tiny().with_(name="router_block_e256_t4100", T=4100, H=1024, I=128, E=256, E_phys=256, K=8,
                         act_dtype="bf16", layout="contig", BM=128, bias="normal0.5"),
    configs.tiny().with_(name="router_block_e200_t5000", T=5000, H=2048, I=128, E=200, E_phys=200, K=8,
                         act_dtype="bf16", layout="contig", BM=128, bias="normal0.5"),
]


@pytest.mark.parametrize("cfg", ROUTER_BLOCK, ids=lambda c: c.name)
def test_router_block_logits(cfg):
    """Same bound as test_router_logits: |got - exact| within H ulps of the
    sum of |x||w| (fp32 accumulation) plus one of the result."""
    b = Built(cfg)
    ref = b.oracle_logits().astype(np.float64)
    b.layer.logits.fill_(float("nan"))
    B.moe_router_logits(b.d, b.x, b.wr, b.bias, b.T, b.layer.logits)
    got = b.layer.logits[: b.T].cpu().numpy().astype(np.float64)
    from oracle_adapt import to_f64
    absdot = np.abs(to_f64(b.inp.x)) @ np.abs(to_f64(b.inp.w_router)).T
    bound = cfg.H * 2.0 ** -24 * absdot + 2.0 ** -24 * np.abs(ref) + 1e-30
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= bound).all(), float((np.abs(got - ref) / bound).max())
    # deterministic: a second call gives the same bits
    first = b.layer.logits[: b.T].clone()
    B.moe_router_logits(b.d, b.x, b.wr, b.bias, b.T, b.layer.logits)
    assert torch.equal(first, b.layer.logits[: b.T])


def test_permute_copies_rows_exactly():
    cfg = SMALL[3]   # fp8 + shared + masked
    b = Built(cfg)
    lg = b.oracle_logits()
    b.run(lg, fused_gather=False)             # the chain with moe_permute
    g = route_np(b.layer.rt, b.T, cfg.K)
    xg = b.layer.xg.cpu()
    xb = b.inp.x.to(torch.bfloat16)
    for t in range(b.T):
        for k in range(cfg.K):
            assert torch.equal(xg[g["slot_of"][t, k]], xb[t])
    base = B.shared_base(b.d)
    assert torch.equal(xg[base: base + b.T], xb)


def test_f32_activations_cast_to_bf16_in_permute():
    b = Built(configs.tiny())
    b.run(b.oracle_logits())
    g = route_np(b.layer.rt, b.T, 2)
    xg = b.layer.xg.cpu()
    assert torch.equal(xg[g["slot_of"][:, 0]], b.inp.x.to(torch.bfloat16))


# ---------------------------------------------------------------- routing edge cases

def _route_only(b: Built, lg: np.ndarray, l2p=None, cnt=None):
    t = torch.from_numpy(np.ascontiguousarray(lg.astype(np.float32))).to(DEV)
    B.moe_route(b.d, t, lg.shape[0], b.layer.rt, b.layer.ws, l2p, cnt)
    torch.cuda.synchronize()
    return route_np(b.layer.rt, lg.shape[0], b.cfg.K)


def _ref_route(cfg, lg, p2l=None):
    ids, w, st = O.topk_route(lg, cfg.K)
    l2p = cnt = None
    if p2l is not None:
        l2p, cnt = O.replica_tables(p2l, cfg.E)
    phys, st2 = O.assign_physical(ids, cfg.E_phys, l2p, cnt)
    counts, offsets, row_of, src_of = O.group_rows(phys, cfg.E_phys)
    res = dict(ids=ids, w=w, phys=phys, counts=counts, offsets=offsets, row_of=row_of, src_of=src_of,
               status=st | st2)
    if cfg.layout == "masked":
        mm, so, slot, st3 = O.layout_masked(counts, offsets, row_of, phys, cfg.M_max, cfg.E_phys)
        res.update(masked_m=mm, spill_off=so, slot_of=slot)
        res["status"] |= st3
    else:
        po, slot = O.layout_contig(counts, offsets, row_of, phys, cfg.BM)
        res.update(pad_off=po, slot_of=slot)
    return res


@pytest.mark.parametrize("case", ["ties", "all_equal", "signed_zero", "nan_inf", "K_eq_E", "T1",
                                  "T65", "spill_all"])
def test_route_edge_cases(case):
    cfg = configs.tiny().with_(T=130, M_max=40)
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    T = cfg.T
    if case == "ties":
        lg = rng.integers(-2, 3, size=(T, cfg.E)).astype(np.float32)
    elif case == "all_equal":
        lg = np.full((T, cfg.E), 0.5, np.float32)
    elif case == "signed_zero":
        lg = np.where(rng.random((T, cfg.E)) < 0.5, -0.0, 0.0).astype(np.float32)
        lg[:, 5] = -1.0
    elif case == "nan_inf":
        lg = rng.standard_normal((T, cfg.E)).astype(np.float32)
        lg[3, 2] = np.nan
        lg[7, :] = np.nan
        lg[9, 4] = np.inf
        lg[11, 6] = -np.inf
    elif case == "K_eq_E":
        cfg = cfg.with_(K=8)
        lg = rng.standard_normal((T, cfg.E)).astype(np.float32)
    elif case == "T1":
        lg = rng.standard_normal((1, cfg.E)).astype(np.float32)
    elif case == "T65":
        lg = rng.standard_normal((65, cfg.E)).astype(np.float32)
    elif case == "spill_all":
        cfg = cfg.with_(M_max=1)
        lg = np.tile(np.arange(cfg.E, dtype=np.float32)[::-1], (T, 1))   # every token picks 0, 1
    b = Built(cfg)
    g = _route_only(b, lg)
    ref = _ref_route(cfg, lg)
    for k in ROUTE_KEYS:
        assert np.array_equal(g[k], np.asarray(ref[k]).reshape(g[k].shape)), k
    if cfg.layout == "masked":
        assert np.array_equal(g["masked_m"], ref["masked_m"]) and np.array_equal(g["spill_off"], ref["spill_off"])
    assert g["status"] == ref["status"]
    fin = np.isfinite(lg).all(axis=1)        # weights of non-finite rows are unspecified
    assert np.abs(g["w"][fin] - ref["w"][fin]).max(initial=0) <= weight_tol(cfg.K)


def test_route_zero_tokens():
    b = Built(configs.tiny())
    lg = np.zeros((0, 8), np.float32)
    B.moe_route(b.d, b.layer.logits, 0, b.layer.rt, b.layer.ws)
    torch.cuda.synchronize()
    g = route_np(b.layer.rt, 0, 2)
    assert (g["counts"] == 0).all() and (g["offsets"] == 0).all() and g["status"] == 0
    out = b.layer.forward(b.x[:0], 0)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


@pytest.mark.parametrize("kind", ["out_of_range", "zero_count", "duplicate", "too_many"])
def test_invalid_replica_map_is_ignored(kind):
    cfg = configs.tiny().with_(E_phys=10, layout="contig")
    b = Built(cfg, p2l=np.array([0, 1, 2, 3, 4, 5, 6, 7, 0, 1], np.int32))
    l2p, cnt = O.replica_tables(b.inp.p2l, cfg.E)
    if kind == "out_of_range":
        l2p[0, 1] = 12
    elif kind == "zero_count":
        cnt[3] = 0
    elif kind == "duplicate":
        l2p[1, 1] = 8
    else:
        cnt[0] = 3
    lg = b.oracle_logits()
    g = _route_only(b, lg, torch.from_numpy(l2p).to(DEV), torch.from_numpy(cnt).to(DEV))
    ids, _, _ = O.topk_route(lg, cfg.K)
    phys, st = O.assign_physical(ids, cfg.E_phys, l2p, cnt)
    assert st & O.STATUS_BAD_REPLICA and g["status"] & B.MOE_STATUS_BAD_REPLICA
    assert np.array_equal(g["phys"], phys) and np.array_equal(g["phys"], ids)


# ---------------------------------------------------------------- layer-level properties

def test_layouts_give_identical_outputs():
    cfg = SMALL[1]
    a = Built(cfg, layout="masked", M_max=3)     # heavy spill
    c = Built(cfg, layout="contig")
    lg = a.oracle_logits()
    oa, oc = a.run(lg).clone(), c.run(lg).clone()
    assert int(a.layer.rt.status.item()) & B.MOE_STATUS_SPILL
    assert torch.equal(oa, oc)


def test_replica_map_leaves_output_unchanged():
    cfg = SMALL[6]
    with_map = Built(cfg)
    no_map = Built(cfg.with_(E_phys=cfg.E))
    lg = with_map.oracle_logits()
    a, b = with_map.run(lg).clone(), no_map.run(lg).clone()
    g = route_np(with_map.layer.rt, cfg.T, cfg.K)
    assert (g["phys"] >= cfg.E).any()            # replicas really used
    assert torch.equal(a, b)


def test_packed_weights_give_identical_outputs():
    """Packing only reorders weight bytes: every row's reduction runs in the
    same order, so outputs must match the row-major run bit for bit."""
    for cfg in (SMALL[1], SMALL[3], SMALL[6]):
        a = Built(cfg)
        p = Built(cfg, packed=True)
        lg = a.oracle_logits()
        assert torch.equal(a.run(lg).clone(), p.run(lg).clone()), cfg.name


def test_fused_gather_gives_identical_outputs():
    """moe_grouped_ffn_x reads each group's rows straight from x (token
    src_of[offsets[p] + rank]) instead of a permuted buffer; the expert
    arithmetic is unchanged, so outputs match moe_permute + moe_grouped_ffn
    bit for bit -- masked with spill, contiguous, shared expert, both size
    classes of the streaming kernel and the tiled kernel."""
    for cfg in SMALL[1:]:
        assert cfg.act_dtype == "bf16", cfg.name
        b = Built(cfg, packed=True)
        lg = b.oracle_logits()
        ref = b.run(lg, fused_gather=False).clone()
        out = b.run(lg).clone()
        assert torch.equal(ref, out), cfg.name
    b = Built(SMALL[6])                      # row-major weights, replica map
    lg = b.oracle_logits()
    assert torch.equal(b.run(lg, fused_gather=False).clone(), b.run(lg).clone())


@pytest.mark.parametrize("nblk", [2, 4])
def test_block_walk_gives_identical_outputs(nblk):
    """A streaming workgroup that walks several 64-row output blocks as one
    pipelined stream (MOE_DEBUG_NBLK_MASK forces the count) reduces every
    output over the same K steps in the same order: bit-identical outputs."""
    for cfg in (SMALL[1], SMALL[3], SMALL[9]):
        for packed in (False, True):
            b = Built(cfg, packed=packed)
            lg = b.oracle_logits()
            ref = b.run(lg).clone()
            b.d.debug_flags = nblk
            try:
                out = b.run(lg).clone()
            finally:
                b.d.debug_flags = 0
            assert torch.equal(ref, out), (cfg.name, packed, nblk)


@pytest.mark.parametrize("name", ["tiled_masked_spill", "tiled_contig_shared", "tiled_wide",
                                  "tiled_skewed_small_groups"])
def test_wide_tiled_kernel_matches_narrow(name):
    """Every kernel for large groups reduces each output over the same
    32-wide K steps in the same order with the same MFMA: bit-identical
    outputs, row-major and packed weights, gathered or permuted rows.
    MOE_DEBUG_TILED_* in the descriptor forces each one: the narrow tile
    (64 weight rows per wave), the wide tile with operands staged through
    registers, with both operands by direct-to-LDS loads, with weights to
    registers and activations through LDS, and the tall 256-row tile (where
    a kernel does not apply to a shape the launch takes the next one)."""
    cfg = next(c for c in SMALL if c.name == name)
    for packed in (False, True):
        b = Built(cfg, packed=packed)
        lg = b.oracle_logits()
        for fused in (True, False):
            ref = b.run(lg, fused_gather=fused).clone()
            for var in TILED_VARIANTS:
                b.d.debug_flags = var << B.MOE_DEBUG_TILED_SHIFT
                try:
                    out = b.run(lg, fused_gather=fused).clone()
                finally:
                    b.d.debug_flags = 0
                assert torch.equal(ref, out), (name, packed, fused, var)


@pytest.mark.parametrize("name", ["tiled_contig_shared", "tiled_wide", "tiled_skewed_small_groups"])
def test_claim_counters(name):
    """The large-group kernels' persistent schedule claims work through the
    route table's counters.  Routing zeroes them (here over a poisoned
    table), every expert call leaves them zero, and the outputs equal those
    of the one-workgroup-per-item schedule (no counter table) bit for bit."""
    cfg = next(c for c in SMALL if c.name == name)
    b = Built(cfg, packed=True)
    lg = b.oracle_logits()
    rt = b.layer.rt
    rt.claim.fill_(12345)
    ref = b.run(lg).clone()
    assert not rt.claim.any(), name
    ref2 = b.run(lg, fused_gather=False).clone()
    assert not rt.claim.any(), name
    assert torch.equal(ref, ref2)
    rt.c.claim = None
    try:
        out = b.run(lg).clone()
    finally:
        rt.c.claim = rt.claim.data_ptr()
    assert torch.equal(ref, out), name


def test_pack_layout_matches_definition():
    """moe_pack_weights places element (n, k) where the layout definition
    says: K block k/128, panel n/16 (step-major), then the lane piece of
    kk = k % 128."""
    for w_dtype, dt in (("bf16", torch.bfloat16), ("fp8", torch.uint8)):
        cfg = configs.tiny().with_(H=256, I=384, w_dtype=w_dtype)
        d = B.Desc.from_config(cfg)
        G, N, Kd = 2, cfg.I, cfg.H
        src = torch.arange(G * N * Kd, dtype=torch.int64) % 251
        src = src.to(torch.int16).view(torch.bfloat16) if dt == torch.bfloat16 else src.to(torch.uint8)
        src = src.reshape(G, N, Kd).to(DEV)
        dst = torch.empty_like(src)
        B.moe_pack_weights(d, 0, src, dst)
        s_ = src.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.uint8).numpy()
        d_ = dst.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.uint8).numpy().reshape(-1)
        esz = 2 if dt == torch.bfloat16 else 1
        per_piece = 16 // esz
        NI = 4 if esz == 2 else 2
        rng = np.random.default_rng(0)
        for _ in range(2000):
            g, n, k = int(rng.integers(G)), int(rng.integers(N)), int(rng.integers(Kd))
            kk = k % 128
            instr = kk // (32 if esz == 2 else 64)
            within = kk % (32 if esz == 2 else 64)
            lane = 16 * (within // per_piece) + n % 16
            e = within % per_piece
            piece = ((((g * (Kd // 128) + k // 128) * (N // 16) + n // 16) * NI + instr) * 64 + lane)
            assert d_[piece * per_piece + e] == s_[g, n, k]


def test_determinism_bit_identical():
    cfg = SMALL[3]
    b = Built(cfg)
    o1 = b.run(None).clone()
    t1 = {k: v.copy() for k, v in route_np(b.layer.rt, b.T, cfg.K).items() if isinstance(v, np.ndarray)}
    o2 = b.run(None).clone()
    t2 = route_np(b.layer.rt, b.T, cfg.K)
    assert torch.equal(o1, o2)
    for k, v in t1.items():
        assert np.array_equal(v, t2[k]), k


def test_fewer_tokens_than_T_max():
    cfg = SMALL[1]
    b = Built(cfg, T=9)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    res = b.oracle(lg)
    check_route(b, res)
    assert rel_err(out, res["out"]) <= TOL["bf16"]


def test_forward_chain_with_gpu_router():
    """GPU router -> route -> ... compared with the reference on its own
    logits.  Where the two fp32 logit vectors order a near-tie differently
    the token is skipped, and such tokens must be rare and genuine ties."""
    for cfg in (SMALL[0], SMALL[3], SMALL[5]):
        b = Built(cfg)
        out = out_np(b.run(None))
        res = b.oracle()
        g = route_np(b.layer.rt, b.T, cfg.K)
        same = (np.sort(g["ids"], 1) == np.sort(res["ids"], 1)).all(1)
        lg = res["logits"].astype(np.float64)
        for t in np.nonzero(~same)[0]:
            srt = np.sort(lg[t])[::-1]
            assert srt[cfg.K - 1] - srt[cfg.K] <= 1e-5 * max(1.0, abs(srt[0])), t
        assert same.mean() >= 0.95
        assert rel_err(out[same], res["out"][same]) <= TOL[cfg.w_dtype]


class _Guarded:
    """Device buffers with guard bands before and after; writes outside the
    documented extent change the guard bytes."""
    G = 4096

    def __init__(self):
        self.bufs = []

    def make(self, n, dtype):
        esz = torch.tensor([], dtype=dtype).element_size()
        g = self.G // esz
        full = torch.full((n + 2 * g,), 0, dtype=dtype, device=DEV)
        full.view(torch.uint8)[:] = 0xA5
        self.bufs.append((full, g, n))
        return full[g: g + n]

    def intact(self):
        for full, g, n in self.bufs:
            u = full.view(torch.uint8)
            esz = full.element_size()
            if not (bool((u[: g * esz] == 0xA5).all()) and bool((u[(g + n) * esz:] == 0xA5).all())):
                return False
        return True


def test_canaries_around_every_buffer():
    for cfg in (SMALL[2], SMALL[4], SMALL[6], SMALL[7], SMALL[8]):
        b = Built(cfg)
        d, T, K = b.d, b.T, cfg.K
        gd = _Guarded()
        rt = B.RouteTables(d, DEV)
        TK = T * K
        for name, n, dt in [("topk_ids", TK, torch.int32), ("topk_w", TK, torch.float32),
                            ("topk_phys", TK, torch.int32), ("row_of", TK, torch.int32),
                            ("slot_of", TK, torch.int32), ("src_of", TK, torch.int32),
                            ("counts", d.E_phys, torch.int32), ("offsets", d.E_phys + 1, torch.int32),
                            ("masked_m", d.E_phys, torch.int32), ("spill_off", d.E_phys + 1, torch.int32),
                            ("pad_off", d.E_phys + 1, torch.int32), ("tile_off", d.E_phys + 2, torch.int32),
                            ("status", 1, torch.int32)]:
            setattr(rt, name, gd.make(n, dt))
        rt.c = B.moe_route_t(*[B._ptr(getattr(rt, f)) for f, _ in B.moe_route_t._fields_])
        rows = B.buffer_rows(d)
        ws = gd.make(B.route_workspace_bytes(d), torch.uint8)
        xg = gd.make(rows * d.H, torch.bfloat16)
        h = gd.make(rows * d.I, torch.bfloat16)
        y = gd.make(B.y_bytes(d, T), torch.uint8)
        out = gd.make(T * d.H, torch.bfloat16)
        logits = gd.make(T * d.E, torch.float32)
        L = b.layer
        B.moe_router_logits(d, b.x, b.wr, b.bias, T, logits)
        B.moe_route(d, logits, T, rt, ws, b.l2p, b.rcount)
        B.moe_permute(d, b.x, T, rt, xg)
        B.moe_grouped_ffn(d, L.weights, rt, T, xg, h, y)
        B.moe_combine(d, rt, T, y, out)
        torch.cuda.synchronize()
        assert gd.intact(), cfg.name
        ref = L.forward(b.x, T)
        torch.cuda.synchronize()
        assert torch.equal(out.view(T, d.H), ref)


# ---------------------------------------------------------------- full workload shapes

def _sample(T, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=min(n, T), replace=False)]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", FULL, ids=lambda c: c.name)
def test_full_size(cfg):
    """Each workload at full size in the launch configuration the benchmark
    times (packed weights, fused gather).  Routing tables bit-exact on the
    whole batch.  Outputs: every token of a decode batch (every touched slot
    and every masked/spill boundary included); for the prefill batch, the
    tokens on the first and last row of every group and on both sides of
    every 128- and 256-row tile boundary of every group and of the shared
    expert, so that each expert, each K loop and each partial last tile is
    compared against the reference."""
    b = Built(cfg, packed=True)          # the layout the benchmark times
    say(f"  built {cfg.name}")
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    assert not b.layer.rt.claim.any()    # the large-group kernels leave their counters zero
    g = route_np(b.layer.rt, b.T, cfg.K)
    if b.T <= 256:
        toks = np.arange(b.T)
    else:
        toks = covering_tokens(g["counts"], g["offsets"], g["src_of"], b.T, cfg.n_shared)
    slots = sorted({int(p) for p in g["phys"][toks].ravel() if p >= 0})
    res = b.oracle(lg, tokens=toks, slots=slots)
    check_route(b, res)
    e = rel_err(out[toks], res["out"])
    say(f"  {cfg.name}: {len(toks)} tokens over {len(slots)} slots, rel err {e:.3e} status {res['status']}")
    assert e <= TOL[cfg.w_dtype]


@pytest.mark.parametrize("name", ["tiny_t16", "dsv3_small_fp8", "replica_small", "tiled_contig_shared"])
def test_c_forward_chain(name):
    """moe_forward, the C ABI's one-call chain (router logits, route,
    permute or fused gather, grouped FFN, combine): its output matches the
    reference on every token and equals the step-by-step calls bit for bit
    (fp32 activations take the permute; bf16 ones the fused gather)."""
    cfg = next(c for c in SMALL if c.name == name)
    b = Built(cfg, packed=cfg.act_dtype == "bf16")
    L = b.layer
    out = torch.zeros_like(L.out)
    B.moe_forward(b.d, b.x, b.wr, b.bias, L.weights, b.T, L.logits, L.rt, L.ws, L.xg, L.h, L.y, out,
                  b.l2p, b.rcount)
    torch.cuda.synchronize()
    got = out_np(out[: b.T])
    res = b.oracle(L.logits[: b.T].cpu().numpy())
    check_route(b, res)
    e = rel_err(got, res["out"])
    say(f"  {name}: rel err {e:.3e}")
    assert e <= TOL[cfg.w_dtype]
    steps = L.forward(b.x, b.T).clone()
    torch.cuda.synchronize()
    assert torch.equal(steps, out[: b.T])


def test_graph_replays_match_eager():
    """The five calls captured in a HIP graph, replayed several times with
    eager work and synchronisations in between; every replay must equal the
    eager result bit for bit (no call records a memset)."""
    for cfg in (SMALL[2], SMALL[3], SMALL[6], SMALL[8]):
        b = Built(cfg)
        other = Built(SMALL[0])
        eager = b.run(None).clone()
        g = torch.cuda.CUDAGraph()
        b.layer.out.zero_()
        with torch.cuda.graph(g):
            b.layer.forward(b.x, b.T)
        for i in range(3):
            b.layer.out.zero_()
            b.layer.xg.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(b.layer.out[: b.T], eager), (cfg.name, i)
            other.run(None)                       # eager work between replays
            torch.cuda.synchronize()
        del g


# ------------------------------------------------- grouped sigmoid router

def _gparams(E, n_group, topk_group, group_k, bias_scale, renorm, scale, seed=11):
    rng = np.random.default_rng(seed)
    sb = None if bias_scale == 0 else rng.normal(scale=bias_scale, size=E).astype(np.float32)
    return dict(n_group=n_group, topk_group=topk_group, group_k=group_k, score_bias=sb,
                renormalize=renorm, scale=scale)


# (config, grouped-router parameters): group sizes 8, 32 and 64 lanes, 1 to
# 4 keys per lane, with and without bias / renormalisation, T inside one
# 64-token block (one fused launch) and across several
_G_BASE = configs.tiny()
GROUPED = [
    (_G_BASE.with_(name="g_e64_k8", T=45, H=256, I=128, E=64, E_phys=64, K=8, act_dtype="bf16",
                   w_dtype="fp8", n_shared=1, M_max=45 * 8 // 64 * 4),
     _gparams(64, 8, 4, 2, 0.3, True, 2.5)),
    (_G_BASE.with_(name="g_e32_k4_nobias", T=70, H=256, I=128, E=32, E_phys=32, K=4, act_dtype="bf16",
                   layout="contig", BM=16),
     _gparams(32, 4, 2, 1, 0.0, False, 1.0)),
    (_G_BASE.with_(name="g_e128_k6", T=1, H=256, I=128, E=128, E_phys=128, K=6, act_dtype="bf16",
                   M_max=4),
     _gparams(128, 16, 4, 3, 0.2, True, 1.0)),
    (_G_BASE.with_(name="g_e256_k8_multiblock", T=300, H=256, I=128, E=256, E_phys=256, K=8,
                   act_dtype="bf16", layout="contig", BM=16, n_shared=1),
     _gparams(256, 8, 4, 2, 0.1, True, 2.5)),
    (_G_BASE.with_(name="g_e64_one_group", T=64, H=256, I=128, E=64, E_phys=64, K=8, act_dtype="bf16",
                   M_max=32),
     _gparams(64, 1, 1, 2, 0.3, True, 1.0)),
]


@pytest.mark.parametrize("cfg,gp", GROUPED, ids=[c.name for c, _ in GROUPED])
def test_grouped_router_route_and_layer(cfg, gp):
    """moe_route_grouped: ids, slots and every table bit-exact against the
    reference's grouped router on the same fp32 logits; weights within the
    fp32 bound (times the scale); the layer output within tolerance."""
    b = Built(cfg, grouped=gp, packed=True)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    res = b.oracle(lg)
    check_route(b, res, wscale=gp["scale"])
    e = rel_err(out, res["out"])
    say(f"  {cfg.name}: rel err {e:.3e}")
    assert e <= TOL[cfg.w_dtype]


def test_grouped_router_full_size_sampled():
    """The DeepSeek-V3-shaped decode layer (256 experts, K=8, fp8, B=256)
    with its router shape: 8 groups of 32, 4 kept, group score = the two
    largest biased scores, weights renormalised and scaled by 2.5."""
    cfg = configs.dsv3_decode(256)
    gp = _gparams(cfg.E, 8, 4, 2, 0.05, True, 2.5)
    b = Built(cfg, grouped=gp, packed=True)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    toks = _sample(b.T, 6)
    res = b.oracle(lg, tokens=toks)
    check_route(b, res, wscale=gp["scale"])
    e = rel_err(out[toks], res["out"])
    say(f"  sampled tokens {list(toks)} rel err {e:.3e}")
    assert e <= TOL[cfg.w_dtype]
