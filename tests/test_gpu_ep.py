"""GPU parity for one GPU's expert-parallel share (moe_route_ep) and for
the received-counts entry point (moe_route_received), through the C ABI,
against the CPU reference (readings R16, R19)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from routing_grouped_expert_router_amd import binding as B
from workloads import configs, generate
from oracle_adapt import oracle_forward, to_f64
from gpu_util import DEV, TOL, Built, out_np, rel_err, route_np, say, tile_off_expected, weight_tol

pytestmark = pytest.mark.gpu

_BASE = configs.tiny()
# (config, ranks, layout, replica slots): masked with spill, contiguous, a
# replica map planned by EPLB, fp8 with a shared expert, groups large enough
# for the tiled kernel, and more ranks than slots (a rank with none)
EP_CASES = [
    (_BASE.with_(name="ep_masked", T=70, H=256, I=128, E=12, E_phys=12, K=3, act_dtype="bf16",
                 M_max=12), 3, "linear", 0),
    (_BASE.with_(name="ep_contig_rr", T=70, H=256, I=128, E=12, E_phys=12, K=3, act_dtype="bf16",
                 layout="contig", BM=16), 4, "round_robin", 0),
    (_BASE.with_(name="ep_eplb", T=90, H=256, I=128, E=12, E_phys=16, K=4, act_dtype="bf16",
                 layout="contig", BM=16, bias="zipf1.1"), 4, "linear", 4),
    (_BASE.with_(name="ep_fp8_shared", T=45, H=1024, I=256, E=64, E_phys=64, K=8, n_shared=1,
                 act_dtype="bf16", w_dtype="fp8", M_max=24), 4, "linear", 0),
    (_BASE.with_(name="ep_tiled", T=600, H=512, I=512, E=4, E_phys=4, K=2, act_dtype="bf16",
                 M_max=200), 2, "round_robin", 0),
    (_BASE.with_(name="ep_more_ranks", T=20, H=256, I=128, E=4, E_phys=4, K=2, act_dtype="bf16",
                 M_max=20), 5, "linear", 0),
]


def _setup(cfg, n_red):
    inp = generate.make_inputs(cfg, wdevice=DEV)
    if n_red:
        # EPLB placement of the expected loads: replicas of the hot experts
        load = generate.zipf_probs(cfg) if cfg.bias == "zipf1.1" else np.ones(cfg.E)
        inp.p2l = O.eplb_plan(load, cfg.E_phys - cfg.E, 4)
    weights = generate.upload_weights(inp, DEV)
    l2p = rc = None
    max_rep = 1
    if inp.p2l is not None:
        l2p_np, rc_np = O.replica_tables(inp.p2l, cfg.E)
        max_rep = l2p_np.shape[1]
        l2p, rc = torch.from_numpy(l2p_np).to(DEV), torch.from_numpy(rc_np).to(DEV)
    return inp, weights, l2p, rc, max_rep


def _rank_layer(cfg, inp, weights, l2p, rc, max_rep, local_of, with_shared):
    """The layer of one rank: its local slots' weights in local order."""
    glob = [p for p in np.argsort(local_of) if local_of[p] >= 0]
    n_local = len(glob)
    E_local = max(1, n_local)
    n_shared = cfg.n_shared if with_shared else 0
    lcfg = cfg.with_(E_phys=E_local, n_shared=n_shared)
    d = B.Desc.from_config(lcfg, max_replicas=max_rep)
    idx = glob + [glob[0] if glob else 0] * (E_local - n_local)
    local = {k: v[torch.tensor(idx, device=DEV)].contiguous() for k, v in weights.items()}
    if n_shared:
        G = cfg.E_phys
        local = {k: torch.cat([local[k], v[G:G + 1]], 0) for k, v in weights.items()}
    ep = B.EPMap(torch.from_numpy(np.ascontiguousarray(local_of)).to(DEV))
    layer = B.MoELayer(d, local, inp.w_router.to(DEV), None if inp.bias is None else inp.bias.to(DEV),
                       l2p, rc, DEV, ep=ep)
    return layer, E_local, n_shared


@pytest.mark.parametrize("case", EP_CASES, ids=lambda c: c[0].name)
def test_ep_share_route_tables_and_output(case):
    cfg, ranks, layout, n_red = case
    say(f"  {cfg.name}: {ranks} ranks, {layout}, {n_red} redundant")
    inp, weights, l2p, rc, max_rep = _setup(cfg, n_red)
    x = inp.x.to(DEV)
    lg_np = O.router_logits(to_f64(inp.x), to_f64(inp.w_router),
                            None if inp.bias is None else inp.bias.numpy())
    lg = torch.from_numpy(lg_np).to(DEV)
    full_layer = B.MoELayer(B.Desc.from_config(cfg, max_replicas=max_rep), weights,
                            inp.w_router.to(DEV), None if inp.bias is None else inp.bias.to(DEV),
                            l2p, rc, DEV)
    full = out_np(full_layer.forward(x, cfg.T, logits=lg).clone())
    total = np.zeros_like(full)
    rows = 0
    for r in range(ranks):
        local_of = O.ep_local_map(cfg.E_phys, ranks, r, layout)
        layer, E_local, n_shared = _rank_layer(cfg, inp, weights, l2p, rc, max_rep, local_of, r == 0)
        out = out_np(layer.forward(x, cfg.T, logits=lg).clone())
        torch.cuda.synchronize()
        got = route_np(layer.rt, cfg.T, cfg.K)
        ref_inp = inp if n_shared else _without_shared(inp)
        res = oracle_forward(ref_inp, logits=lg_np, local_of=local_of, E_local=E_local)
        assert got["status"] == res["status"], (r, got["status"], res["status"])
        for key in ("ids", "phys", "row_of", "slot_of", "counts", "offsets"):
            assert np.array_equal(got[key], res[key]), (cfg.name, r, key)
        n = int(res["offsets"][-1])
        assert np.array_equal(got["src_of"][:n], res["src_of"]), (cfg.name, r)
        if cfg.layout == "masked":
            assert np.array_equal(got["masked_m"], res["masked_m"])
            assert np.array_equal(got["spill_off"], res["spill_off"])
        else:
            assert np.array_equal(got["pad_off"], res["pad_off"])
        assert np.array_equal(got["tile_off"], tile_off_expected(res["counts"], cfg.T, n_shared))
        assert np.abs(got["w"] - res["w"]).max() <= weight_tol(cfg.K)
        e = rel_err(out, res["out"]) if np.abs(res["out"]).max() > 0 else float(np.abs(out).max())
        say(f"    rank {r}: {E_local} local slots, {n} rows, rel err {e:.3e}")
        assert e <= TOL[cfg.w_dtype]
        total += out
        rows += n
    assert rows == cfg.T * cfg.K
    e = rel_err(total, full)
    say(f"    sum over ranks vs the full layer: rel err {e:.3e}")
    assert e <= TOL[cfg.w_dtype]


def _without_shared(inp):
    import copy
    out = copy.copy(inp)
    out.cfg = inp.cfg.with_(n_shared=0)
    return out


def test_ep_invalid_local_map_leaves_nothing_local():
    cfg = EP_CASES[0][0]
    inp, weights, l2p, rc, max_rep = _setup(cfg, 0)
    local_of = O.ep_local_map(cfg.E_phys, 3, 0, "linear")
    local_of[5] = 0                            # local slot 0 named twice
    layer, E_local, _ = _rank_layer(cfg, inp, weights, l2p, rc, max_rep, local_of, True)
    out = out_np(layer.forward(inp.x.to(DEV), cfg.T).clone())
    got = route_np(layer.rt, cfg.T, cfg.K)
    assert got["status"] & B.MOE_STATUS_BAD_EP_MAP
    assert got["counts"].sum() == 0 and (got["row_of"] == -1).all() and (got["slot_of"] == -1).all()
    assert not out.any()


@pytest.mark.parametrize("name", ["mixtral_small_masked", "dsv3_small_fp8"])
def test_received_counts_run_the_dispatched_buffer(name):
    """A masked buffer filled as a dispatch would fill it (here: moe_permute
    of a routed batch) plus its per-slot counts gives, through
    moe_route_received, the tables moe_route wrote and bit-identical expert
    outputs on every valid row."""
    from test_gpu_parity import SMALL
    cfg = next(c for c in SMALL if c.name == name).with_(M_max=64)
    b = Built(cfg)
    b.run(b.oracle_logits(), fused_gather=False)
    L = b.layer
    T = b.T
    rt2 = B.RouteTables(b.d, DEV)
    B.moe_route_received(b.d, L.rt.counts.clone(), T, rt2)
    torch.cuda.synchronize()
    assert int(rt2.status.item()) == 0
    for key in ("counts", "masked_m", "offsets", "spill_off", "tile_off"):
        assert torch.equal(getattr(rt2, key), getattr(L.rt, key)), key
    h2 = torch.zeros_like(L.h)
    y2 = torch.zeros_like(L.y)
    B.moe_expert_gate_up(b.d, L.weights, rt2, T, L.xg, h2)
    B.moe_expert_down(b.d, L.weights, rt2, T, h2, y2)
    torch.cuda.synchronize()
    ysz = B.y_bytes(b.d, T)
    splits = B.down_splits(b.d, T)
    cnt = L.rt.counts.cpu().numpy()
    rows = [p * cfg.M_max + i for p in range(b.d.E_phys) for i in range(cnt[p])]
    if cfg.n_shared:
        base = B.shared_base(b.d)
        rows += [base + t for t in range(T)]
    rows = torch.tensor(rows, device=DEV)
    if splits == 1:
        a = L.y[:ysz].view(torch.bfloat16).view(-1, b.d.H)
        c = y2[:ysz].view(torch.bfloat16).view(-1, b.d.H)
    else:
        a = L.y[:ysz].view(torch.float32).view(splits, -1, b.d.H)[:, :].transpose(0, 1)
        c = y2[:ysz].view(torch.float32).view(splits, -1, b.d.H)[:, :].transpose(0, 1)
    assert torch.equal(a[rows], c[rows])
    # a count above M_max: flagged, clamped
    bad = L.rt.counts.clone()
    bad[0] = cfg.M_max + 3
    B.moe_route_received(b.d, bad, T, rt2)
    torch.cuda.synchronize()
    assert int(rt2.status.item()) & B.MOE_STATUS_RECV_OVERFLOW
    assert int(rt2.masked_m[0].item()) == cfg.M_max


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_received_counts_above_routed_total(packed):
    """A dispatch can deliver more rows to a rank than its own batch routed
    (T*K): here the slots of a masked buffer receive up to M_max rows, about
    six times T*K in all, with T*K = 64*E_phys so the large-group kernel
    runs.  Every received row's expert output must match the reference
    SwiGLU of that row (no row tile left out of the launch: 31 row tiles of
    128 against the 12 a routed batch of this size can have)."""
    cfg = _BASE.with_(name="recv_many", T=256, H=512, I=512, E=8, E_phys=8, K=2, act_dtype="bf16",
                      M_max=640)
    b = Built(cfg, packed=packed)
    d, L, T = b.d, b.layer, b.T
    counts = torch.tensor([640, 600, 513, 400, 390, 300, 257, 129], dtype=torch.int32, device=DEV)
    assert int(counts.sum()) > T * cfg.K and T * cfg.K >= 64 * cfg.E_phys
    rows_n = B.buffer_rows(d)
    g = torch.Generator(device="cpu").manual_seed(7)
    xg = torch.randn((rows_n, d.H), generator=g).to(torch.bfloat16).to(DEV)
    rt2 = B.RouteTables(d, DEV)
    B.moe_route_received(d, counts, T, rt2)
    h = torch.zeros_like(L.h)
    y = torch.zeros_like(L.y)
    B.moe_expert_gate_up(d, L.weights, rt2, T, xg, h)
    B.moe_expert_down(d, L.weights, rt2, T, h, y)
    torch.cuda.synchronize()
    assert int(rt2.status.item()) == 0
    splits = B.down_splits(d, T)
    ysz = B.y_bytes(d, T)
    if splits == 1:
        yv = y[:ysz].view(torch.bfloat16).view(-1, d.H).float()
    else:
        yv = y[:ysz].view(torch.float32).view(splits, -1, d.H).sum(0)
    xs = to_f64(xg.cpu())
    worst = 0.0
    for p in range(cfg.E_phys):
        ew = b.inp.expert(b.inp.slot_logical(p))
        W1, W3, W2 = to_f64(ew.w1), to_f64(ew.w3), to_f64(ew.w2)
        rows = np.arange(p * cfg.M_max, p * cfg.M_max + int(counts[p]))
        ref = O.swiglu_expert(xs[rows], W1, W3, W2)
        got = yv[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
        worst = max(worst, rel_err(got, ref))
    say(f"  received {int(counts.sum())} rows (T*K = {T * cfg.K}): rel err {worst:.3e}")
    assert worst <= TOL["bf16"]


@pytest.mark.parametrize("T", [1, 3])
def test_received_counts_on_more_slots_than_routed_choices(T):
    """Few tokens (T*K below the slot count) make the streaming launch run
    T*K workgroup rows over the slots that hold tokens instead of one row
    per slot; received counts can fill more slots than T*K, so each row then
    walks several slots.  Every slot's rows (M_max each, and an empty slot)
    must match the reference SwiGLU of those rows."""
    cfg = _BASE.with_(name=f"recv_t{T}", T=T, H=512, I=256, E=16, E_phys=16, K=2, act_dtype="bf16", M_max=4)
    b = Built(cfg, packed=True)
    d, L = b.d, b.layer
    counts = torch.tensor([4, 1, 0, 3, 2, 4, 1, 1, 4, 0, 2, 3, 4, 1, 2, 4], dtype=torch.int32, device=DEV)
    assert (counts > 0).sum() > T * cfg.K
    rows_n = B.buffer_rows(d)
    g = torch.Generator(device="cpu").manual_seed(11)
    xg = torch.randn((rows_n, d.H), generator=g).to(torch.bfloat16).to(DEV)
    rt2 = B.RouteTables(d, DEV)
    B.moe_route_received(d, counts, T, rt2)
    h = torch.zeros_like(L.h)
    y = torch.zeros_like(L.y)
    B.moe_expert_gate_up(d, L.weights, rt2, T, xg, h)
    B.moe_expert_down(d, L.weights, rt2, T, h, y)
    torch.cuda.synchronize()
    assert int(rt2.status.item()) == 0
    splits = B.down_splits(d, T)
    ysz = B.y_bytes(d, T)
    if splits == 1:
        yv = y[:ysz].view(torch.bfloat16).view(-1, d.H).float()
    else:
        yv = y[:ysz].view(torch.float32).view(splits, -1, d.H).sum(0)
    xs = to_f64(xg.cpu())
    worst = 0.0
    for p in range(cfg.E_phys):
        if int(counts[p]) == 0:
            continue
        ew = b.inp.expert(b.inp.slot_logical(p))
        W1, W3, W2 = to_f64(ew.w1), to_f64(ew.w3), to_f64(ew.w2)
        rows = np.arange(p * cfg.M_max, p * cfg.M_max + int(counts[p]))
        ref = O.swiglu_expert(xs[rows], W1, W3, W2)
        got = yv[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
        worst = max(worst, rel_err(got, ref))
    say(f"  T={T}: {int((counts > 0).sum())} slots with rows (T*K = {T * cfg.K}): rel err {worst:.3e}")
    assert worst <= TOL["bf16"]
