"""GPU parity of the W8A8 path (fp8 activations on fp8 MFMA) through the C
ABI against the CPU reference's W8A8 definition (readings R20-R22)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from routing_grouped_expert_router_amd import binding as B
from workloads import configs
from gpu_util import DEV, TOL, Built, covering_tokens, out_np, rel_err, route_np, say

pytestmark = pytest.mark.gpu


def test_quantize_codes_and_scales_bit_exact():
    """moe_quantize_1x128 against the reference's quantizer on bf16 rows with
    magnitudes over many binades, an all-zero block and values that land on
    E4M3 subnormals; rows read through a stride wider than C."""
    g = torch.Generator().manual_seed(7)
    rows, C, ld = 37, 640, 768
    x = torch.randn(rows, ld, generator=g) * torch.exp2(torch.randint(-12, 12, (rows, 1), generator=g).float())
    x[3, 128:256] = 0.0
    x[5, :128] = torch.randn(128, generator=g) * 1e-4   # far below the block max: subnormal codes
    x[5, 7] = 9.0
    xb = x.to(torch.bfloat16)
    q = torch.zeros(rows, C, dtype=torch.uint8, device=DEV)
    s = torch.zeros(rows, C // 128, dtype=torch.float32, device=DEV)
    B.moe_quantize_1x128(xb.to(DEV), rows, q, s)
    torch.cuda.synchronize()
    ref_q, ref_s = O.quant_1x128(xb[:, :C].float().numpy())
    assert np.array_equal(s.cpu().numpy(), ref_s)
    got = q.cpu().numpy()
    assert np.array_equal(got, ref_q), np.argwhere(got != ref_q)[:5]
    assert ((got[5, :128] & 0x78) == 0).sum() > 10          # subnormal codes were exercised


A8_CASES = [
    configs.tiny().with_(name="a8_masked_shared", T=45, H=1024, I=256, E=64, E_phys=64, K=8, n_shared=1,
                         act_dtype="bf16", w_dtype="fp8", M_max=24),
    configs.tiny().with_(name="a8_contig_big_groups", T=120, H=512, I=256, E=8, E_phys=8, K=2, n_shared=1,
                         act_dtype="bf16", w_dtype="fp8", layout="contig", BM=16, bias="zipf1.1"),
    configs.tiny().with_(name="a8_spill_t1", T=1, H=512, I=384, E=16, E_phys=16, K=4,
                         act_dtype="bf16", w_dtype="fp8", M_max=1),
]


@pytest.mark.parametrize("cfg", A8_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("packed", [False, True])
def test_a8_layer_against_reference(cfg, packed):
    b = Built(cfg, packed=packed, a8=True)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    res = b.oracle(lg)
    e = rel_err(out, res["out"])
    say(f"  {cfg.name} packed={packed}: rel err {e:.3e}")
    assert e <= TOL["fp8"]


def test_a8_full_size_sampled():
    cfg = configs.dsv3_decode(256)
    b = Built(cfg, packed=True, a8=True)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    toks = np.array([0, 77, 181, 255])
    res = b.oracle(lg, tokens=toks)
    e = rel_err(out[toks], res["out"])
    say(f"  dsv3_decode_b256 W8A8, tokens {list(toks)}: rel err {e:.3e}")
    assert e <= TOL["fp8"]


def test_two_level_accumulation_at_k16k_all_positive():
    """[infra5] DeepGEMM section: with all-positive data and K = 16K, summing
    128-wide blocks on the matrix unit and accumulating the scaled block
    sums in fp32 stays at about the bf16 rounding of the output (0.17%
    there; without the promotion about 25%).  The gate/up outputs of one
    expert with H = 16384, all-positive codes and activations, against the
    exact two-level sums."""
    cfg = configs.tiny().with_(name="k16k", T=16, H=16384, I=128, E=1, E_phys=1, K=1,
                               act_dtype="bf16", w_dtype="fp8", M_max=16)
    b = Built(cfg, a8=True)
    w = b.layer.weights._keep[0]
    w["w1"].bitwise_and_(0x7F)
    w["w3"].bitwise_and_(0x7F)
    x = b.x.abs()
    L = b.layer
    B.moe_route(b.d, torch.zeros((cfg.T, 1), dtype=torch.float32, device=DEV), cfg.T, L.rt, L.ws)
    B.moe_quantize_1x128(x, cfg.T, L.xq, L.xs)
    B.moe_expert_gate_up_a8(b.d, L.weights, L.rt, cfg.T, L.xq, L.xs, L.h)
    torch.cuda.synchronize()
    qx, sx = L.xq[:cfg.T].cpu().numpy(), L.xs[:cfg.T].cpu().numpy()
    G = O.w8a8_matmul(qx, sx, w["w1"][0].cpu().numpy(), w["s1"][0].cpu().numpy())
    U = O.w8a8_matmul(qx, sx, w["w3"][0].cpu().numpy(), w["s3"][0].cpu().numpy())
    ref = O.silu(G) * U
    rows = L.rt.src_of[: cfg.T].cpu().numpy()          # row r of the group is token src_of[r]
    got = L.h[: cfg.T].float().cpu().numpy().astype(np.float64)
    e = float(np.abs(got - ref[rows]).max() / np.abs(ref).max())
    say(f"  K=16384 all-positive: max rel err {e:.3e} (bf16 rounding {2.0 ** -9:.3e})")
    assert (ref > 0).all() and e <= 2.0 ** -8


@pytest.mark.parametrize("nblk", [2, 4])
def test_a8_block_walk_gives_identical_outputs(nblk):
    """1, 2 or 4 output blocks per W8A8 workgroup (MOE_DEBUG_NBLK_MASK)
    reduce every output over the same K steps in the same order:
    bit-identical layer outputs, both size classes (T > 16)."""
    cfg = A8_CASES[0]
    b = Built(cfg, packed=True, a8=True)
    lg = b.oracle_logits()
    try:
        b.d.debug_flags = 1
        ref = b.run(lg).clone()
        b.d.debug_flags = nblk
        out = b.run(lg).clone()
    finally:
        b.d.debug_flags = 0
    assert torch.equal(ref, out), nblk


# groups large on average (T*K >= 64 E_phys): the W8A8 large-group kernel
# takes both projections; Zipf-skewed experts fill up to T rows, so groups
# span two 256-row tiles with a ragged second one, and small groups leave
# most of their one tile empty
A8_LARGE = [
    configs.tiny().with_(name="a8_tall_contig_shared", T=512, H=1024, I=1024, E=64, E_phys=64, K=8, n_shared=1,
                         act_dtype="bf16", w_dtype="fp8", layout="contig", BM=16, bias="zipf1.1"),
    configs.tiny().with_(name="a8_tall_masked_spill", T=520, H=1024, I=1024, E=64, E_phys=64, K=8, n_shared=0,
                         act_dtype="bf16", w_dtype="fp8", layout="masked", M_max=96, bias="zipf1.1"),
]


def _tall_both(b) -> bool:
    return all(B.expert_kernel_a8(b.d, b.T, w) == "ffn_a8_tall_kernel" for w in (0, 1))


@pytest.mark.parametrize("cfg", A8_LARGE, ids=lambda c: c.name)
def test_a8_large_groups_against_reference(cfg):
    """The large-group W8A8 kernel on every token against the reference's
    W8A8 layer; the claim counters are left zero."""
    b = Built(cfg, packed=True, a8=True)
    assert _tall_both(b)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    assert not b.layer.rt.claim.any()
    g = route_np(b.layer.rt, b.T, cfg.K)
    assert g["counts"].max() > 256                       # some groups span two tiles
    res = b.oracle(lg)
    e = rel_err(out, res["out"])
    say(f"  {cfg.name}: groups {g['counts'].min()}..{g['counts'].max()} rows, rel err {e:.3e}")
    assert e <= TOL["fp8"]


@pytest.mark.parametrize("cfg", A8_LARGE, ids=lambda c: c.name)
def test_a8_large_group_kernel_matches_streaming(cfg):
    """The large-group and the streaming W8A8 kernels reduce every output
    over the same 128-wide K blocks, in the same order, with the same
    products and scalings: bit-identical layer outputs."""
    b = Built(cfg, packed=True, a8=True)
    lg = b.oracle_logits()
    try:
        b.d.debug_flags = B.MOE_DEBUG_A8_STREAM << B.MOE_DEBUG_TILED_SHIFT
        assert B.expert_kernel_a8(b.d, b.T, 0) == "ffn_a8_kernel"
        ref = b.run(lg).clone()
        b.d.debug_flags = 0
        out = b.run(lg).clone()
    finally:
        b.d.debug_flags = 0
    assert _tall_both(b)
    assert torch.equal(ref, out), cfg.name


@pytest.mark.timeout(900)
def test_a8_prefill_full_size_sampled():
    """The DeepSeek-V3-shaped prefill (T = 8192) with fp8 weights on the W8A8
    path, in the launch configuration the benchmark times: routing tables
    bit-exact, and the tokens on the first and last row of every group and on
    both sides of every 256-row tile boundary compared with the reference."""
    cfg = configs.dsv3_prefill().with_(name="dsv3_prefill_t8192_fp8", w_dtype="fp8")
    b = Built(cfg, packed=True, a8=True)
    assert _tall_both(b)
    lg = b.oracle_logits()
    out = out_np(b.run(lg))
    assert not b.layer.rt.claim.any()
    g = route_np(b.layer.rt, b.T, cfg.K)
    toks = covering_tokens(g["counts"], g["offsets"], g["src_of"], b.T, cfg.n_shared, tiles=(256,))
    res = b.oracle(lg, tokens=toks)
    e = rel_err(out[toks], res["out"])
    say(f"  {cfg.name}: {len(toks)} tokens, rel err {e:.3e}")
    assert e <= TOL["fp8"]


@pytest.mark.parametrize("walk", [1, 2])
def test_a8_large_group_walks_give_identical_outputs(walk):
    """A large-group W8A8 work item walks several weight tiles as one
    pipeline (8 at these shapes by default); forcing 1 or 2 per item
    (MOE_DEBUG_NBLK_MASK) reduces every output over the same K blocks in
    the same order: bit-identical layer outputs, claim counters left zero."""
    cfg = A8_LARGE[0]
    b = Built(cfg, packed=True, a8=True)
    lg = b.oracle_logits()
    ref = b.run(lg).clone()
    try:
        b.d.debug_flags = walk
        assert _tall_both(b)
        out = b.run(lg).clone()
    finally:
        b.d.debug_flags = 0
    assert not b.layer.rt.claim.any()
    assert torch.equal(ref, out), walk
