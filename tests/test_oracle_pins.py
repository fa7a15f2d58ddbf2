"""Pins for the CPU reference: every check compares it with something other
than itself -- textbook sorts, brute force, a third-party implementation of
the Mixtral MoE block, closed forms, and values the pages print."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from workloads import configs, generate
from oracle_adapt import oracle_forward, to_f64, expert_f64

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- formats

def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=50000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = O.decode_bf16(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_decoder_spec_values():
    # values fixed by the OCP 8-bit floating point format (E4M3FN)
    spec = {0x00: 0.0, 0x38: 1.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x40: 2.0, 0x3C: 1.5, 0xB8: -1.0}
    for code, val in spec.items():
        assert O.decode_e4m3fn(np.array([code], np.uint8))[0] == val, hex(code)
    assert np.isnan(O.decode_e4m3fn(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(O.decode_e4m3fn(np.array([0x80], np.uint8))[0])


def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.decode_e4m3fn(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_block_dequant_against_loop():
    rng = np.random.default_rng(2)
    q = rng.integers(0, 256, size=(256, 384), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x11      # no NaN codes
    s = rng.uniform(0.5, 2.0, size=(2, 3)).astype(np.float32)
    got = O.dequant_block128(q, s)
    for i in (0, 127, 128, 255):
        for j in (0, 129, 300, 383):
            assert got[i, j] == O.decode_e4m3fn(q[i:i + 1, j])[0] * float(s[i // 128, j // 128])


def test_synthetic_fp8_roundtrip_is_close():
    w = torch.randn(256, 256, generator=torch.Generator().manual_seed(0)) * 0.02
    q, s = generate.quantize_e4m3_block128(w)
    back = O.dequant_block128(q.numpy(), s.numpy())
    # e4m3 has 3 mantissa bits: relative rounding error <= 2^-4 on normals
    err = np.abs(back - w.double().numpy())
    assert err.max() <= 2 ** -4 * np.abs(w.double().numpy()).max() + 1e-12


# ---------------------------------------------------------------- top-K

def _topk_textbook(row, K):
    """Python's sorted() on (-value, id), NaN last: the definition of R1/R2."""
    items = []
    for e, v in enumerate(row):
        v = float(v)
        items.append(((1 if math.isnan(v) else 0), 0.0 if math.isnan(v) else -(v + 0.0), e))
    return [e for _, _, e in sorted(items)[:K]]


@pytest.mark.parametrize("E,K", [(8, 2), (8, 8), (16, 5), (64, 8), (33, 1)])
def test_topk_ids_match_textbook_sort_with_ties(E, K):
    rng = np.random.default_rng(E * 100 + K)
    for trial in range(40):
        # integer-valued logits force many exact ties
        lg = rng.integers(-3, 4, size=(7, E)).astype(np.float32)
        if trial % 2:
            lg = rng.standard_normal((7, E)).astype(np.float32)
        ids, w, _ = O.topk_route(lg, K)
        for t in range(lg.shape[0]):
            assert list(ids[t]) == _topk_textbook(lg[t], K)


def test_topk_signed_zero_and_nan():
    lg = np.array([[-0.0, 0.0, -1.0, np.nan, -np.inf, 0.0]], np.float32)
    ids, _, st = O.topk_route(lg, 6)
    assert list(ids[0]) == [0, 1, 5, 2, 4, 3]
    assert st & O.STATUS_NONFINITE


def test_topk_all_equal_and_full():
    lg = np.full((3, 8), 0.25, np.float32)
    ids, w, _ = O.topk_route(lg, 3)
    assert (ids == np.arange(3)).all() and (w == 1.0 / 3).all()
    lg = np.random.default_rng(3).standard_normal((5, 8)).astype(np.float32)
    ids, _, _ = O.topk_route(lg, 8)
    assert (ids == np.argsort(-lg, axis=1, kind="stable")).all()


def test_topk_weights_closed_forms():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((50, 16)).astype(np.float32)
    ids1, w1, _ = O.topk_route(lg, 1)
    assert (w1 == 1.0).all()
    ids2, w2, _ = O.topk_route(lg, 2)
    l0 = np.take_along_axis(lg, ids2[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(lg, ids2[:, 1:], 1)[:, 0].astype(np.float64)
    assert np.allclose(w2[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=0, atol=1e-15)
    _, w8, _ = O.topk_route(lg, 8)
    assert np.allclose(w8.sum(1), 1.0, atol=1e-14)
    assert (np.diff(w8, axis=1) <= 0).all()


def test_topk_weights_equal_full_softmax_renormalised():
    """Mixtral's top-K-then-softmax equals vLLM's softmax-then-renormalize."""
    rng = np.random.default_rng(5)
    lg = (rng.standard_normal((30, 12)) * 3).astype(np.float32)
    ids, w, _ = O.topk_route(lg, 4)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    sel = np.take_along_axis(p, ids, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-13, atol=0)


# ---------------------------------------------------------------- grouping

def _phys_random(T, K, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)


def test_counts_offsets_src_row_against_textbook():
    T, K, E = 37, 3, 11
    phys = _phys_random(T, K, E, 6)
    counts, offsets, row_of, src_of = O.group_rows(phys, E)
    assert counts.sum() == T * K                                  # sum_e T_e = B*K
    assert (counts == np.bincount(phys.ravel(), minlength=E)).all()
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
    pairs = sorted((int(phys[t, k]), t, k) for t in range(T) for k in range(K))
    assert list(src_of) == [t for _, t, _ in pairs]
    for r, (_, t, k) in enumerate(pairs):
        assert row_of[t, k] == r
    # permute then unpermute is the identity
    x = np.random.default_rng(7).standard_normal((T, 5))
    xg = x[src_of]
    for k in range(K):
        assert (xg[row_of[:, k]] == x).all()


def test_masked_layout_tables():
    T, K, E, M_max = 40, 4, 6, 5
    phys = _phys_random(T, K, E, 8)
    counts, offsets, row_of, _ = O.group_rows(phys, E)
    masked_m, spill_off, slot, st = O.layout_masked(counts, offsets, row_of, phys, M_max, E)
    assert (masked_m == np.minimum(counts, M_max)).all()
    assert spill_off[-1] == np.maximum(counts - M_max, 0).sum()
    assert st == (O.STATUS_SPILL if spill_off[-1] else 0)
    # slots are distinct, inside the static buffer + spill region, and each
    # masked slot lies inside its expert's valid rows
    assert len(set(slot.ravel().tolist())) == T * K
    cap = E * M_max + K * max(0, T - M_max)
    assert slot.min() >= 0 and slot.max() < cap
    for t in range(T):
        for k in range(K):
            p, s = phys[t, k], slot[t, k]
            if s < E * M_max:
                assert s // M_max == p and s % M_max < masked_m[p]
            else:
                assert spill_off[p] <= s - E * M_max < spill_off[p + 1]


def test_contig_layout_tables():
    T, K, E, BM = 33, 2, 7, 8
    phys = _phys_random(T, K, E, 9)
    counts, offsets, row_of, _ = O.group_rows(phys, E)
    pad_off, slot = O.layout_contig(counts, offsets, row_of, phys, BM)
    assert (pad_off % BM == 0).all() and (np.diff(pad_off) >= counts).all()
    assert (np.diff(pad_off) < counts + BM).all()
    for t in range(T):
        for k in range(K):
            p = phys[t, k]
            assert pad_off[p] <= slot[t, k] < pad_off[p] + counts[p]


# ---------------------------------------------------------------- replicas

def test_replica_tables_page_example():
    g = _gold("replica_map_eplb.json")
    l2p, count = O.replica_tables(np.array(g["physical_to_logical_map"]), 4)
    assert l2p.tolist() == g["logical_to_physical_map"]
    assert count.tolist() == g["logical_replica_count"]


def test_replica_round_robin_split():
    T, K, E = 50, 3, 6
    p2l = np.array([0, 1, 2, 3, 4, 5, 0, 0, 2], np.int32)
    l2p, count = O.replica_tables(p2l, E)
    ids = _phys_random(T, K, E, 10)
    phys, st = O.assign_physical(ids, len(p2l), l2p, count)
    assert st == 0
    assert (p2l[phys] == ids).all()                         # ids unchanged
    pc = np.bincount(phys.ravel(), minlength=len(p2l))
    lc = np.bincount(ids.ravel(), minlength=E)
    for l in range(E):
        reps = l2p[l, :count[l]]
        assert pc[reps].sum() == lc[l]                      # counts conserved
        assert pc[reps].max() - pc[reps].min() <= 1         # even split
        # round robin over ascending tokens
        toks = [t for t in range(T) for k in range(K) if ids[t, k] == l]
        got = [phys[t, list(ids[t]).index(l)] for t in toks]
        assert got == [reps[j % count[l]] for j in range(len(toks))]


@pytest.mark.parametrize("l2p,count", [
    ([[0, 9], [1, -1]], [2, 1]),      # slot outside [0, E_phys)
    ([[0, 2], [1, -1]], [2, 0]),      # a logical expert with no replica
    ([[0, 2], [2, -1]], [2, 1]),      # slot 2 listed twice
    ([[0, 2], [1, -1]], [3, 1]),      # count above max_replicas
])
def test_replica_invalid_map_is_ignored(l2p, count):
    ids = np.array([[0, 1], [1, 0]], np.int32)
    phys, st = O.assign_physical(ids, 3, np.array(l2p, np.int32), np.array(count, np.int32))
    assert st & O.STATUS_BAD_REPLICA
    assert phys.tolist() == [[0, 1], [1, 0]]
    ok, st = O.assign_physical(ids, 3, np.array([[0, 2], [1, -1]], np.int32), np.array([2, 1], np.int32))
    assert st == 0 and ok.tolist() == [[0, 1], [1, 2]]


# ---------------------------------------------------------------- FFN + combine

def _tiny_inputs(**kw):
    cfg = configs.tiny().with_(**kw)
    return generate.make_inputs(cfg)


@pytest.mark.parametrize("kw", [dict(), dict(K=1), dict(K=8), dict(E=5, E_phys=5, K=3, T=9),
                                dict(n_shared=1), dict(layout="contig", BM=4)])
def test_oracle_matches_bruteforce(kw):
    inp = _tiny_inputs(**kw)
    cfg = inp.cfg
    res = oracle_forward(inp)
    ew = lambda l: expert_f64(inp.expert(l), cfg.w_dtype)
    sh = expert_f64(inp.shared(), cfg.w_dtype) if cfg.n_shared else None
    bf = O.bruteforce_forward(to_f64(inp.x), to_f64(inp.w_router), None, cfg.K, ew, sh)
    assert np.allclose(res["out"], bf, rtol=1e-12, atol=1e-12)


def test_oracle_matches_transformers_mixtral_block():
    """Third-party pin: Hugging Face's Mixtral sparse-MoE block (router
    softmax -> top-k -> renormalise, SiLU(gate) * up -> down, weighted sum),
    run in float64 on the same weights."""
    from transformers import MixtralConfig
    from transformers.models.mixtral.modeling_mixtral import MixtralSparseMoeBlock
    inp = _tiny_inputs()
    cfg = inp.cfg
    hf = MixtralConfig(hidden_size=cfg.H, intermediate_size=cfg.I, num_local_experts=cfg.E,
                       num_experts_per_tok=cfg.K, hidden_act="silu")
    blk = MixtralSparseMoeBlock(hf).double().eval()
    with torch.no_grad():
        blk.gate.weight.copy_(torch.from_numpy(to_f64(inp.w_router)))
        for e in range(cfg.E):
            W1, W3, W2 = expert_f64(inp.expert(e), cfg.w_dtype)
            blk.experts.gate_up_proj[e].copy_(torch.from_numpy(np.concatenate([W1, W3], 0)))
            blk.experts.down_proj[e].copy_(torch.from_numpy(W2))
        _, _, hf_ids = blk.gate(torch.from_numpy(to_f64(inp.x)))
        ref = blk(torch.from_numpy(to_f64(inp.x))[None])[0].numpy()
    res = oracle_forward(inp)
    assert (np.sort(res["ids"], 1) == np.sort(hf_ids.numpy(), 1)).all()
    # the HF router takes its softmax in fp32: agreement to fp32 rounding
    assert np.abs(res["out"] - ref).max() <= 1e-6 * np.abs(ref).max()


def test_single_expert_reduces_to_dense_swiglu_and_shared_matches_mlp():
    """E=1, K=1: the layer is one dense SwiGLU FFN (torch linear + silu).
    The shared expert equals Hugging Face's DeepseekV3MLP on its weights."""
    inp = _tiny_inputs(E=1, E_phys=1, K=1)
    W1, W3, W2 = expert_f64(inp.expert(0), "bf16")
    x = torch.from_numpy(to_f64(inp.x))
    F = torch.nn.functional
    dense = F.linear(F.silu(F.linear(x, torch.from_numpy(W1))) * F.linear(x, torch.from_numpy(W3)),
                     torch.from_numpy(W2)).numpy()
    assert np.allclose(oracle_forward(inp)["out"], dense, rtol=1e-12, atol=1e-13)

    from transformers import DeepseekV3Config
    from transformers.models.deepseek_v3.modeling_deepseek_v3 import DeepseekV3MLP
    inp = _tiny_inputs(n_shared=1)
    S1, S3, S2 = expert_f64(inp.shared(), "bf16")
    mlp = DeepseekV3MLP(DeepseekV3Config(hidden_size=inp.cfg.H, intermediate_size=inp.cfg.I,
                                         hidden_act="silu")).double()
    with torch.no_grad():
        mlp.gate_proj.weight.copy_(torch.from_numpy(S1))
        mlp.up_proj.weight.copy_(torch.from_numpy(S3))
        mlp.down_proj.weight.copy_(torch.from_numpy(S2))
        shared_ref = mlp(torch.from_numpy(to_f64(inp.x))).numpy()
    with_sh = oracle_forward(inp)["out"]
    without = oracle_forward(generate.make_inputs(inp.cfg.with_(n_shared=0)))["out"]
    assert np.allclose(with_sh - without, shared_ref, rtol=1e-10, atol=1e-12)


def test_replica_map_leaves_output_unchanged():
    """Redundant-expert semantics: ids, weights and combine positions are
    unchanged, so the output must not change."""
    base = configs.tiny().with_(E=6, E_phys=6, K=2, T=24, layout="contig")
    rep = base.with_(E_phys=9)
    a = generate.make_inputs(base)
    b = generate.make_inputs(rep)
    b.p2l = np.array([0, 1, 2, 3, 4, 5, 2, 2, 0], np.int32)
    ra, rb = oracle_forward(a), oracle_forward(b)
    assert (ra["ids"] == rb["ids"]).all() and (ra["w"] == rb["w"]).all()
    assert np.allclose(ra["out"], rb["out"], rtol=1e-13, atol=1e-14)
    assert rb["counts"][[2, 6, 7]].sum() == ra["counts"][2]


def test_layouts_agree():
    inp = _tiny_inputs(T=16, M_max=3)        # forces spill
    rm = oracle_forward(inp, layout="masked")
    rc = oracle_forward(inp, layout="contig")
    assert rm["status"] & O.STATUS_SPILL
    assert np.array_equal(rm["out"], rc["out"])


def test_token_sample_matches_full_run():
    inp = _tiny_inputs(n_shared=1)
    full = oracle_forward(inp)
    part = oracle_forward(inp, tokens=[3, 0, 15])
    assert np.allclose(part["out"], full["out"][[3, 0, 15]], rtol=1e-13, atol=1e-14)


def test_fp8_weights_path():
    inp = _tiny_inputs(w_dtype="fp8", H=256, I=256)
    cfg = inp.cfg
    res = oracle_forward(inp)
    ew = lambda l: expert_f64(inp.expert(l), "fp8")
    bf = O.bruteforce_forward(to_f64(inp.x), to_f64(inp.w_router), None, cfg.K, ew)
    assert np.allclose(res["out"], bf, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- accounting

def test_accounting_pins_from_pages():
    g = _gold("accounting_pins.json")
    a = g["expert_bytes_fp8_dsv3_x8"]
    w_only = 3 * a["H"] * a["I"] * a["bytes_per_weight"] * a["n_experts"]
    assert round(w_only / 1e6) == a["total_mb_decimal"]
    for lat, tbs in zip(g["triton_bm_sweep"]["latency_us"], g["triton_bm_sweep"]["tb_per_s"]):
        assert round(w_only / (lat * 1e-6) / 1e12, 1) == tbs
    pw = g["pad_waste"]
    for c in pw["cases"]:
        assert O.pad_waste(pw["M_e"], c["BM"]) == pytest.approx(c["waste"])
    m = g["mixtral_expert_params"]
    assert O.expert_bytes(m["H"], m["I"], "bf16") // 2 * m["E"] * m["n_layers"] == m["total"]
    act = g["mixtral_active_params"]
    active = 2 * 4096 * 14336 * 3 * 32 + act["replicated"]
    assert round(active / 1e9, 2) == act["active_billions_2dp"]


def test_coverage_closed_form():
    # C(B) limits and a direct count over all k-subsets for a tiny case:
    # probability that a given expert is untouched by B tokens choosing
    # uniform k-subsets of E is ((E-k)/E)^B.
    assert O.coverage(0, 2, 8) == 0.0
    assert O.coverage(10 ** 6, 8, 256) == pytest.approx(1.0)
    E, k, B = 5, 2, 3
    subsets = list(itertools.combinations(range(E), k))
    miss = sum(1 for ch in itertools.product(subsets, repeat=B) if all(0 not in s for s in ch))
    assert miss / len(subsets) ** B == pytest.approx(1 - O.coverage(B, k, E))


@pytest.mark.parametrize("cfgf,B", [(configs.mixtral_decode, 8), (configs.dsv3_decode, 32),
                                    (configs.dsv3_decode, 128)])
def test_distinct_experts_track_coverage(cfgf, B):
    """The synthetic router is close to uniform, so the number of distinct
    experts a batch touches should sit near E*C(B).  Each seed redraws x and
    W_r; a non-uniform router would sit below E*C(B)."""
    counts = []
    for seed in range(24):
        cfg = cfgf(B).with_(seed=seed)
        inp = generate.make_inputs(cfg)
        lg = O.router_logits(to_f64(inp.x), to_f64(inp.w_router), None)
        ids, _, _ = O.topk_route(lg, cfg.K)
        counts.append(len(np.unique(ids)))
    exp = cfg.E * O.coverage(B, cfg.K, cfg.E)
    mean = float(np.mean(counts))
    se = float(np.std(counts, ddof=1) / np.sqrt(len(counts))) if np.std(counts) > 0 else 0.0
    assert mean <= exp + 3 * se + 1e-9
    assert mean >= exp * 0.97 - 3 * se


# ------------------------------------------------- grouped sigmoid router (R13-R15)

def _grouped_logits(T=64, E=64, seed=3):
    rng = np.random.default_rng(seed)
    return rng.normal(scale=1.5, size=(T, E)).astype(np.float32), rng


def test_grouped_router_matches_transformers_deepseek_v3_router():
    """Hugging Face's DeepSeek-V3 router (sigmoid scores, correction bias for
    the choice only, best groups by the sum of their two largest biased
    scores, then top-k inside them, weights from the unbiased scores,
    normalised and scaled) -- a third-party implementation -- chooses the
    same experts and gives the same weights from its own fp32 logits."""
    from transformers import DeepseekV3Config
    from transformers.models.deepseek_v3.modeling_deepseek_v3 import DeepseekV3TopkRouter
    H, E, K, G, TG, scale = 96, 64, 8, 8, 4, 2.5
    hf = DeepseekV3Config(hidden_size=H, n_routed_experts=E, num_experts_per_tok=K, n_group=G,
                          topk_group=TG, norm_topk_prob=True, routed_scaling_factor=scale)
    gate = DeepseekV3TopkRouter(hf).eval()
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.normal(size=(48, H)).astype(np.float32))
    bias = rng.normal(scale=0.3, size=E).astype(np.float32)
    with torch.no_grad():
        gate.weight.copy_(torch.from_numpy(rng.normal(scale=0.15, size=(E, H)).astype(np.float32)))
        gate.e_score_correction_bias.copy_(torch.from_numpy(bias))
        logits, hf_w, hf_ids = gate(x)
    logits = logits.float().numpy().reshape(-1, E)
    ids, w, st = O.grouped_topk_route(logits, K, G, TG, 2, bias, True, scale)
    hf_ids, hf_w = hf_ids.numpy().reshape(-1, K), hf_w.float().numpy().reshape(-1, K)
    assert st == 0
    for t in range(ids.shape[0]):
        assert set(ids[t].tolist()) == set(hf_ids[t].tolist()), t
        mine = dict(zip(ids[t].tolist(), w[t]))
        for e, v in zip(hf_ids[t].tolist(), hf_w[t]):
            # HF takes its sigmoid in fp32; the reading rounds an fp64 sigmoid
            assert abs(mine[e] - v) <= 1e-6 * scale, (t, e)


def test_grouped_router_one_group_is_sigmoid_topk():
    """One group kept out of one, no bias: the choice is the K largest
    scores, i.e. (sigmoid being increasing) the K largest logits -- the
    softmax router's choice -- and the renormalised weights are torch's
    sigmoid of those logits over their sum."""
    lg, _ = _grouped_logits()
    ids, w, _ = O.grouped_topk_route(lg, 6, 1, 1, 1, None, True, 1.0)
    ref_ids, _, _ = O.topk_route(lg, 6)
    assert (ids == ref_ids).all()
    s = torch.sigmoid(torch.from_numpy(lg).double()).numpy()
    sel = np.take_along_axis(s, ids, 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-6, atol=0)


def test_grouped_router_all_groups_kept_is_global_topk_of_biased_scores():
    """Keeping every group leaves a plain top-K of score + bias over all
    experts (any group size, any group_k): Python's sorted() on
    (-(s + b), id)."""
    lg, rng = _grouped_logits()
    b = rng.normal(scale=0.2, size=lg.shape[1]).astype(np.float32)
    s = O.sigmoid_scores_fp32(lg)
    key = (s + b[None, :]).astype(np.float32)
    for G, gk in ((4, 1), (8, 3), (16, 2)):
        ids, _, _ = O.grouped_topk_route(lg, 8, G, G, gk, b, True, 1.0)
        for t in range(lg.shape[0]):
            ref = [e for _, e in sorted((-float(key[t, e]), e) for e in range(lg.shape[1]))[:8]]
            assert ids[t].tolist() == ref


def test_grouped_router_bias_steers_choice_not_weights():
    """The correction bias only decides which experts are chosen: the
    weights are always the chosen experts' unbiased sigmoid scores over
    their sum, times the scale; a large bias on expert 5 forces it into
    every token's choice with its own (unbiased) score as weight."""
    lg, rng = _grouped_logits()
    E = lg.shape[1]
    s = torch.sigmoid(torch.from_numpy(lg).double()).numpy()
    for b in (rng.normal(scale=0.5, size=E).astype(np.float32), None):
        ids, w, _ = O.grouped_topk_route(lg, 8, 8, 4, 2, b, True, 2.5)
        sel = np.take_along_axis(s, ids, 1)
        assert np.allclose(w, 2.5 * sel / sel.sum(1, keepdims=True), rtol=1e-6, atol=0)
    b = np.zeros(E, np.float32)
    b[5] = 100.0
    ids, w, _ = O.grouped_topk_route(lg, 8, 8, 4, 2, b, False, 1.0)
    assert (ids[:, 0] == 5).all()
    assert np.allclose(w[:, 0], s[:, 5], rtol=1e-6, atol=0)


def test_grouped_router_keeps_only_the_best_groups():
    """Every chosen expert lies in one of the topk_group groups whose sums of
    group_k largest biased scores are highest (a brute force over the group
    subsets: the kept set has the largest score total among all subsets of
    that size)."""
    lg, rng = _grouped_logits(T=32, E=32)
    b = rng.normal(scale=0.3, size=32).astype(np.float32)
    key = (O.sigmoid_scores_fp32(lg) + b[None, :]).astype(np.float32).astype(np.float64)
    G, TG, gk, K = 8, 3, 2, 6
    ids, _, _ = O.grouped_topk_route(lg, K, G, TG, gk, b, True, 1.0)
    for t in range(32):
        gs = [np.sort(key[t, g * 4:(g + 1) * 4])[::-1][:gk].sum() for g in range(G)]
        best = max(itertools.combinations(range(G), TG), key=lambda c: sum(gs[g] for g in c))
        assert {int(e) // 4 for e in ids[t]} <= set(best), t


# ------------------------------------------------- expert parallelism (R16-R19)

def test_ep_local_map_page_examples():
    """[vllbc] EP section: 4 experts on 2 ranks -- linear gives rank 0 experts
    0, 1 and rank 1 experts 2, 3; round_robin gives rank 0 experts 0, 2 and
    rank 1 experts 1, 3; local ids count 0.. in expert order, -1 elsewhere.
    Uneven splits give the first remainder ranks one extra expert."""
    assert O.ep_local_map(4, 2, 0).tolist() == [0, 1, -1, -1]
    assert O.ep_local_map(4, 2, 1).tolist() == [-1, -1, 0, 1]
    assert O.ep_local_map(4, 2, 0, "round_robin").tolist() == [0, -1, 1, -1]
    assert O.ep_local_map(4, 2, 1, "round_robin").tolist() == [-1, 0, -1, 1]
    assert O.ep_local_map(5, 2, 0).tolist() == [0, 1, 2, -1, -1]
    assert O.ep_local_map(5, 2, 1).tolist() == [-1, -1, -1, 0, 1]
    assert O.ep_local_map(7, 3, 2).tolist() == [-1, -1, -1, -1, -1, 0, 1]


@pytest.mark.parametrize("layout", ["linear", "round_robin"])
def test_ep_local_maps_partition_the_slots(layout):
    for n, ep in [(8, 2), (9, 4), (256, 8), (5, 5), (3, 4)]:
        maps = np.stack([O.ep_local_map(n, ep, r, layout) for r in range(ep)])
        assert ((maps >= 0).sum(0) == 1).all()           # each slot on exactly one rank
        for m in maps:                                    # local ids 0..n_r-1 in slot order
            loc = m[m >= 0]
            assert loc.tolist() == list(range(len(loc)))


@pytest.mark.parametrize("layout", ["linear", "round_robin"])
@pytest.mark.parametrize("replicas", [False, True])
def test_ep_shares_sum_to_the_full_layer(layout, replicas):
    """R16: a remote choice contributes zero locally and is computed by the
    rank that owns its slot, so the ranks' outputs sum to the full layer's,
    and each rank's rows are exactly its local choices."""
    cfg = configs.tiny().with_(E=6, E_phys=9 if replicas else 6, K=2, T=24, layout="contig", BM=4)
    inp = generate.make_inputs(cfg)
    if replicas:
        inp.p2l = np.array([0, 1, 2, 3, 4, 5, 2, 2, 0], np.int32)
    full = oracle_forward(inp)
    ep = 3
    total = np.zeros_like(full["out"])
    rows = 0
    for r in range(ep):
        loc = O.ep_local_map(cfg.E_phys, ep, r, layout)
        res = oracle_forward(inp, local_of=loc)
        assert res["status"] == 0
        total += res["out"]
        local = loc[full["phys"]] >= 0
        assert ((res["row_of"] >= 0) == local).all()
        assert (res["slot_of"][~local] == -1).all()
        assert res["counts"].sum() == local.sum() == res["offsets"][-1]
        rows += res["counts"].sum()
    assert rows == cfg.T * cfg.K
    assert np.allclose(total, full["out"], rtol=1e-12, atol=1e-14)


def test_ep_rank_without_experts_and_invalid_map():
    cfg = configs.tiny().with_(E=4, E_phys=4, K=2, T=8)
    inp = generate.make_inputs(cfg)
    none = np.full(4, -1, np.int32)
    res = oracle_forward(inp, local_of=none, E_local=2)
    assert res["counts"].sum() == 0 and (res["row_of"] == -1).all()
    assert np.array_equal(res["out"], np.zeros_like(res["out"]))
    bad = np.array([0, 0, -1, 1], np.int32)                # local slot 0 named twice
    res = oracle_forward(inp, local_of=bad, E_local=2)
    assert res["status"] & O.STATUS_BAD_EP_MAP and res["counts"].sum() == 0


def test_eplb_replicas_minimise_the_largest_load_per_replica():
    """R17 against brute force: handing redundant slots one at a time to the
    largest load per replica reaches the least possible largest load per
    replica, on every small instance."""
    rng = np.random.default_rng(0)
    for _ in range(150):
        E, nr = int(rng.integers(2, 6)), int(rng.integers(0, 5))
        load = rng.integers(1, 50, size=E).astype(np.float64)
        rep = O.eplb_replicas(load, nr)
        assert rep.sum() == E + nr and (rep >= 1).all()
        best = min(max(load / np.array(r)) for r in itertools.product(range(1, nr + 2), repeat=E)
                   if sum(r) == E + nr)
        assert max(load / rep) == best


def test_eplb_plan_worked_examples():
    """[eplb] section 1.3: four experts, two redundant slots; with E0 and E2
    hot the redundant slots hold E0 and E2.  Worked by hand: replicas
    E0 x2, E2 x2 at 15 each, E1, E3 at 5; LPT puts the two copies of an
    expert on different ranks and balances 35 / 35."""
    p2l = O.eplb_plan(np.array([30.0, 5.0, 30.0, 5.0]), 2, 2)
    assert p2l.tolist() == [0, 2, 1, 0, 2, 3]
    # no redundancy: 8, 4, 2, 2 on two ranks of two slots -> {8, 2}, {4, 2}
    assert O.eplb_plan(np.array([8.0, 4.0, 2.0, 2.0]), 0, 2).tolist() == [0, 3, 1, 2]
    # every rank holds S slots and every expert at least one replica
    rng = np.random.default_rng(1)
    for _ in range(50):
        ep = int(rng.integers(1, 6)); S = int(rng.integers(1, 6))
        E = int(rng.integers(max(1, ep * S - 4), ep * S + 1))
        p2l = O.eplb_plan(rng.random(E) + 0.01, ep * S - E, ep)
        assert len(p2l) == ep * S and set(p2l.tolist()) == set(range(E))


def test_eplb_flattens_routing_hot_spots():
    """[infra5] EPLB: replicating hot experts and LPT packing bring the
    busiest rank's load back to about 1.1 x the mean under routing hot
    spots.  Zipf(1.1) loads over 256 experts, 32 redundant slots: linear
    placement without replicas is far above that, the plan within it."""
    E = 256
    ranks = np.random.default_rng(2).permutation(E) + 1
    load = ranks ** -1.1
    for ep in (8, 16, 32):
        S = (E + 32) // ep
        p2l = O.eplb_plan(load, 32, ep)
        rep = np.bincount(p2l, minlength=E)
        w = load[p2l] / rep[p2l]
        per_rank = w.reshape(ep, S).sum(1)
        assert per_rank.max() / per_rank.mean() <= 1.1
        lin = load.reshape(ep, E // ep).sum(1)
        assert lin.max() / lin.mean() > 1.5


def test_received_tables_match_routed_masked_tables():
    """R19 against the routing path: counts taken from a routed batch give
    back its masked_m and the 128-row tile prefix (no spill)."""
    inp = _tiny_inputs(T=40, M_max=40)
    res = oracle_forward(inp, layout="masked")
    rt = O.received_tables(res["counts"], inp.cfg.M_max)
    assert np.array_equal(rt["masked_m"], res["masked_m"]) and rt["status"] == 0
    assert np.array_equal(rt["offsets"], res["offsets"])
    tiles = np.concatenate([[0], np.cumsum(-(-res["counts"] // 128))])
    assert np.array_equal(rt["tile_off"], tiles)
    over = O.received_tables(np.array([3, 50]), 40)
    assert over["status"] & O.STATUS_RECV_OVERFLOW and over["masked_m"].tolist() == [3, 40]


# ------------------------------------------------------------------ W8A8 (R20-R22)

def test_e4m3_encoder_matches_torch_cast():
    """The reference's E4M3FN encoder against torch's float8_e4m3fn cast
    (round to nearest even) on a dense grid of fp32 values in [-448, 448],
    every midpoint between adjacent codes, subnormals and signed zeros; and
    every finite code decodes and re-encodes to itself."""
    pos = O.decode_e4m3fn(np.arange(127))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([np.linspace(-448, 448, 100001).astype(np.float32), mids, -mids,
                        np.float32([0.0, -0.0, 2 ** -10, 2 ** -11, 3 * 2 ** -11, -2 ** -9])])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3fn(v), ref)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(O.encode_e4m3fn(O.decode_e4m3fn(codes)), codes)
    assert O.encode_e4m3fn(np.array([500.0, -1e9])).tolist() == [0x7E, 0xFE]   # saturate


def test_quant_1x128_scales_and_error_bound():
    """R20: per row and 128-wide block the largest magnitude codes to exactly
    +-448; every value dequantizes within half a code step (2^-4 relative
    for normals, s * 2^-10 absolute below); an all-zero block has scale 1."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((5, 384)) * np.exp(rng.normal(0, 2, (5, 1)))).astype(np.float32)
    x[2, 128:256] = 0.0
    q, s = O.quant_1x128(x)
    assert q.shape == x.shape and s.shape == (5, 3) and s.dtype == np.float32
    dq = O.decode_e4m3fn(q).reshape(5, 3, 128) * s[:, :, None]
    xb = x.reshape(5, 3, 128).astype(np.float64)
    for r in range(5):
        for b in range(3):
            if r == 2 and b == 1:
                assert s[r, b] == 1.0 and not q[r, 128:256].any()
                continue
            k = int(np.argmax(np.abs(xb[r, b])))
            assert (q.reshape(5, 3, 128)[r, b, k] & 0x7F) == 0x7E          # |code| = 448
    bound = np.maximum(np.abs(xb) * 2.0 ** -4, s[:, :, None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(dq - xb) <= bound).all()


def test_w8a8_product_equals_dequantized_matmul():
    """R21 against the plain product of the dequantized operands (block
    scales applied elementwise first, one matmul after)."""
    rng = np.random.default_rng(1)
    T, N, K = 7, 256, 384
    qa, sa = O.quant_1x128(rng.standard_normal((T, K)).astype(np.float32))
    w = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32) * 0.02)
    qw, sw = generate.quantize_e4m3_block128(w)
    qw, sw = qw.numpy(), sw.numpy()
    A = O.decode_e4m3fn(qa) * np.repeat(sa, 128, axis=1)
    W = O.dequant_block128(qw, sw)
    assert np.allclose(O.w8a8_matmul(qa, sa, qw, sw), A @ W.T, rtol=1e-12, atol=1e-15)


def test_round_bf16_matches_torch():
    v = np.random.default_rng(2).standard_normal(10000) * 10.0 ** np.random.default_rng(3).integers(-5, 5, 10000)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(O.round_bf16(v), ref)


def test_w8a8_layer_against_w8a16_layer():
    """R22: quantizing the activations moves the fp8-weight layer by a few
    percent of its largest output (the 1x128 activation code steps); the
    routing is untouched."""
    from oracle_adapt import oracle_forward_w8a8
    cfg = configs.tiny().with_(T=20, H=512, I=256, E=8, E_phys=8, K=2, n_shared=1,
                               act_dtype="bf16", w_dtype="fp8", M_max=20)
    inp = generate.make_inputs(cfg)
    a = oracle_forward(inp)
    b = oracle_forward_w8a8(inp)
    e = np.abs(a["out"] - b["out"]).max() / np.abs(a["out"]).max()
    assert 5e-3 < e < 6e-2, e
    assert np.array_equal(a["row_of"], b["row_of"])


def _torch_q1x128(a: torch.Tensor):
    """Rows of fp32 values -> (E4M3FN codes as float64 values, fp32 scales
    [R, C/128]), written from R20 with torch's own float8_e4m3fn cast: per
    row and 128-wide block s = fp32(amax / 448) (1 for an all-zero block),
    codes = cast(fp32(x / s)) clamped to +-448."""
    R, C = a.shape
    blk = a.reshape(R, C // 128, 128)
    amax = blk.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    v = (blk / s[:, :, None]).clamp(-448.0, 448.0)
    codes = v.to(torch.float8_e4m3fn).to(torch.float64).reshape(R, C)
    return codes, s


def _torch_block_product(ca, sa, cw, sw):
    """R21 with torch matmuls, one per 128-wide K block: the block's sum of
    code products, times the row's and the weight block's scales, added to
    a float64 total."""
    T, K = ca.shape
    N = cw.shape[0]
    out = torch.zeros((T, N), dtype=torch.float64)
    for b in range(K // 128):
        part = ca[:, 128 * b:128 * (b + 1)] @ cw[:, 128 * b:128 * (b + 1)].T
        wscale = torch.repeat_interleave(sw[:, b].to(torch.float64), 128)      # [N]
        out += part * sa[:, b].to(torch.float64)[:, None] * wscale[None, :]
    return out


def _torch_w8a8_expert(x, ew, round_h=True, h_blocks_by_row=True):
    """R22 composed independently of the reference: x (bf16 values) coded per
    token, gate and up by R21, h = SiLU(g) * u rounded to bf16 through fp32,
    h coded per row, down by R21.  The switches plant the two mistakes the
    pin must catch: no bf16 rounding of h, and h coded with one scale per
    128-wide block shared by all rows (the weights' block rule) instead of
    one per row."""
    dec = lambda q: q.view(torch.float8_e4m3fn).to(torch.float64)
    cx, sx = _torch_q1x128(x.to(torch.float32))
    g = _torch_block_product(cx, sx, dec(ew.w1), ew.s1)
    u = _torch_block_product(cx, sx, dec(ew.w3), ew.s3)
    h = torch.nn.functional.silu(g) * u
    if round_h:
        h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    h32 = h.to(torch.float32)
    if h_blocks_by_row:
        ch, sh = _torch_q1x128(h32)
    else:                                   # one scale per block for all rows
        R, C = h32.shape
        blk = h32.reshape(R, C // 128, 128)
        amax = blk.abs().amax(dim=(0, 2))
        s1 = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        ch = (blk / s1[None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
        ch = ch.reshape(R, C)
        sh = s1[None, :].expand(R, -1)
    return _torch_block_product(ch, sh, dec(ew.w2), ew.s2)


def test_w8a8_expert_against_independent_torch_composition():
    """swiglu_expert_w8a8 (R20-R22) against the same composition written
    independently with torch: torch's float8_e4m3fn cast for both
    quantizations, one torch matmul per 128-wide K block, and the bf16
    rounding of h made explicit.  Agreement is to float64 rounding.  The
    same composition with the bf16 rounding of h dropped, or with h coded in
    blocks along the wrong axis, lies far outside that tolerance, so the pin
    catches either mistake in the reference."""
    cfg = configs.tiny().with_(T=6, H=384, I=256, E=1, E_phys=1, K=1, act_dtype="bf16", w_dtype="fp8")
    inp = generate.make_inputs(cfg)
    ew = inp.expert(0)
    x = inp.x.to(torch.float64)
    # rows of different magnitudes, one all-zero 128-block (scale 1)
    x = x * torch.tensor([1.0, 3.0, 0.25, 10.0, 1.0, 0.5], dtype=torch.float64)[:, None]
    x[4, 128:256] = 0.0
    x = x.to(torch.bfloat16)
    ref = O.swiglu_expert_w8a8(to_f64(x), (ew.w1.numpy(), ew.s1.numpy(), ew.w3.numpy(), ew.s3.numpy(),
                                           ew.w2.numpy(), ew.s2.numpy()))
    got = _torch_w8a8_expert(x, ew).numpy()
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() <= 1e-12 * scale
    no_round = _torch_w8a8_expert(x, ew, round_h=False).numpy()
    wrong_axis = _torch_w8a8_expert(x, ew, h_blocks_by_row=False).numpy()
    assert np.abs(no_round - ref).max() > 1e-6 * scale
    assert np.abs(wrong_axis - ref).max() > 1e-6 * scale
