"""GPU parity of the single-launch decode layer (moe_decode_fused).

Every output -- logits, route tables, h, y and the layer output -- must be
bit-identical to the multi-launch chain (moe_router_logits, moe_route or
moe_route_grouped, moe_grouped_ffn_x, moe_combine) on the same inputs and
buffers, and the layer output must meet the reference tolerance against the
CPU reference on the same fp32 logits.  Shapes span several 64-row weight
blocks and every routing-select shape the fused launch takes (E = 8 .. 256,
softmax and grouped), masked (with spill) and contiguous layouts, replicas,
a shared expert, bf16 and fp8 weights, the MFMA router (E > 64) and T from
0 to 16.
"""
import numpy as np
import pytest
import torch

from routing_grouped_expert_router_amd import binding as B
from workloads import configs
from gpu_util import Built, TOL, rel_err, out_np, route_np, say, DEV
from test_gpu_parity import check_route, _gparams, _sample

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_hygiene(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


_BASE = configs.tiny().with_(act_dtype="bf16")
# (config, grouped-router parameters or None)
CASES = [
    (_BASE.with_(name="f_e8_t16", T=16, H=512, I=768, M_max=16), None),
    (_BASE.with_(name="f_e8_t1", T=1, H=512, I=768, M_max=1), None),
    (_BASE.with_(name="f_e8_spill", T=16, H=512, I=768, M_max=2), None),
    (_BASE.with_(name="f_e16_contig_shared", T=13, H=256, I=384, E=16, E_phys=16, K=4, n_shared=1,
                 layout="contig", BM=16, bias="normal0.5"), None),
    (_BASE.with_(name="f_e32_replica", T=9, H=256, I=128, E=32, E_phys=40, K=4, layout="contig", BM=16,
                 bias="zipf1.1"), None),
    (_BASE.with_(name="f_e64_fp8_shared", T=11, H=512, I=256, E=64, E_phys=64, K=8, n_shared=1,
                 w_dtype="fp8", M_max=4), None),
    (_BASE.with_(name="f_e128_mfma_router", T=16, H=1024, I=256, E=128, E_phys=128, K=6, M_max=4), None),
    (_BASE.with_(name="f_e256_fp8_mfma", T=5, H=1024, I=256, E=256, E_phys=256, K=8, n_shared=1,
                 w_dtype="fp8", M_max=2), None),
    (_BASE.with_(name="f_g_e64", T=16, H=256, I=128, E=64, E_phys=64, K=8, n_shared=1, w_dtype="fp8",
                 M_max=4), _gparams(64, 8, 4, 2, 0.3, True, 2.5)),
    (_BASE.with_(name="f_g_e128", T=3, H=1024, I=128, E=128, E_phys=128, K=6, M_max=2),
     _gparams(128, 16, 4, 3, 0.2, True, 1.0)),
    (_BASE.with_(name="f_g_e256_shared", T=16, H=1024, I=256, E=256, E_phys=256, K=8, n_shared=1,
                 w_dtype="fp8", M_max=2), _gparams(256, 8, 4, 2, 0.1, True, 2.5)),
]


def _zero(b: Built):
    L = b.layer
    for t in (L.h, L.y, L.out, L.logits):
        t.zero_()
    for f, _ in B.moe_route_t._fields_:
        getattr(L.rt, f).zero_()


def _snapshot(b: Built, T: int) -> dict:
    L = b.layer
    s = {k: v.copy() if isinstance(v, np.ndarray) else v for k, v in route_np(L.rt, T, b.cfg.K).items()}
    s["logits"] = L.logits[:T].cpu().numpy().copy()
    s["h"] = L.h.view(torch.int16).cpu().numpy().copy()
    s["y"] = L.y.cpu().numpy().copy()
    s["out_bits"] = L.out[:T].view(torch.int16).cpu().numpy().copy()
    s["out"] = L.out[:T].float().cpu().numpy().copy()
    return s


def _multi(b: Built, T: int) -> dict:
    _zero(b)
    b.layer.forward(b.x, T)
    torch.cuda.synchronize()
    return _snapshot(b, T)


def _fused(b: Built, T: int) -> dict:
    _zero(b)
    b.layer.forward_fused(b.x, T)
    torch.cuda.synchronize()
    return _snapshot(b, T)


def _same(a: dict, f: dict, what: str):
    for k in a:
        if isinstance(a[k], np.ndarray):
            assert a[k].shape == f[k].shape, (what, k)
            # bit patterns: NaN-safe and sign-of-zero exact
            assert np.array_equal(a[k].view(np.uint8), f[k].view(np.uint8)), (what, k)
        else:
            assert a[k] == f[k], (what, k, a[k], f[k])
    assert (f["status"] & B.MOE_STATUS_SYNC_TIMEOUT) == 0, what


@pytest.mark.parametrize("cfg,gp", CASES, ids=[c.name for c, _ in CASES])
def test_fused_decode_matches_chain_and_reference(cfg, gp):
    b = Built(cfg, grouped=gp, packed=True)
    T = b.T
    ref = _multi(b, T)
    got = _fused(b, T)
    _same(ref, got, cfg.name)
    # against the CPU reference on the same fp32 logits
    res = b.oracle(got["logits"].astype(np.float64))
    check_route(b, res, wscale=1.0 if gp is None else gp["scale"])
    e = rel_err(got["out"].astype(np.float64), res["out"])
    say(f"  {cfg.name}: bit-identical to the chain, rel err {e:.3e}, status {got['status']}")
    assert e <= TOL[cfg.w_dtype]


def test_fused_decode_token_counts_and_repeats():
    """T = 16, 1, 0, 7, 16 in a row on one layer and one fused workspace: each
    call equals the chain at its T (the barrier words carry over correctly);
    T = 0 writes the empty tables."""
    cfg = _BASE.with_(name="f_seq", T=16, H=256, I=384, E=16, E_phys=16, K=4, n_shared=1, M_max=16)
    b = Built(cfg, packed=True)
    for T in (16, 1, 0, 7, 16):
        ref = _multi(b, T)
        got = _fused(b, T)
        _same(ref, got, f"T={T}")
        if T == 0:
            assert got["counts"].sum() == 0 and got["status"] == 0


def test_fused_decode_graph_replays_match_eager():
    """forward_fused captured in a HIP graph and replayed several times, with
    other eager work (the multi-launch chain of another layer) between the
    replays; every replay equals the eager result bit for bit."""
    cfg, gp = CASES[8]
    b = Built(cfg, grouped=gp, packed=True)
    other = Built(CASES[0][0], packed=True)
    eager = _fused(b, b.T)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.layer.forward_fused(b.x, b.T)
    for i in range(3):
        _zero(b)
        g.replay()
        torch.cuda.synchronize()
        _same(eager, _snapshot(b, b.T), f"replay {i}")
        other.layer.forward(other.x, other.T)
        torch.cuda.synchronize()
    del g


FULL = [
    (configs.mixtral_decode(1), None),
    (configs.mixtral_decode(8), None),
    (configs.dsv3_decode(32).with_(name="dsv3_decode_b8", T=8, M_max=4),
     _gparams(256, 8, 4, 2, 0.05, True, 2.5)),
]


@pytest.mark.parametrize("cfg,gp", FULL, ids=[c.name for c, _ in FULL])
def test_fused_decode_full_size(cfg, gp):
    """The decode workload shapes: bit-identical to the chain, sampled tokens
    against the CPU reference."""
    b = Built(cfg, grouped=gp, packed=True)
    say(f"  built {cfg.name}")
    T = b.T
    ref = _multi(b, T)
    got = _fused(b, T)
    _same(ref, got, cfg.name)
    toks = _sample(T, 4)
    res = b.oracle(got["logits"].astype(np.float64), tokens=toks)
    check_route(b, res, wscale=1.0 if gp is None else gp["scale"])
    e = rel_err(got["out"][toks].astype(np.float64), res["out"])
    say(f"  {cfg.name}: bit-identical to the chain, sampled tokens {list(toks)} rel err {e:.3e}")
    assert e <= TOL[cfg.w_dtype]


def test_fused_decode_timeout_path_and_recovery():
    """The bounded wait's failure path, forced from the host: with a wait
    bound of zero polls (MOE_DEBUG_FUSED_NO_WAIT) every workgroup that has to
    wait at a barrier aborts the launch, which ends normally with
    MOE_STATUS_SYNC_TIMEOUT in the status word.  After the fused workspace is
    zero-filled again the next call equals the multi-launch chain bit for
    bit."""
    cfg, gp = CASES[0]
    b = Built(cfg, grouped=gp, packed=True)
    ref = _multi(b, b.T)
    b.d.debug_flags = B.MOE_DEBUG_FUSED_NO_WAIT
    try:
        _zero(b)
        b.layer.forward_fused(b.x, b.T)
        torch.cuda.synchronize()
    finally:
        b.d.debug_flags = 0
    status = int(b.layer.rt.status.cpu().numpy()[0])
    assert status & B.MOE_STATUS_SYNC_TIMEOUT, status
    b.layer.fws.zero_()
    _same(ref, _fused(b, b.T), "after recovery")
