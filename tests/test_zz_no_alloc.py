"""The no-allocation routing entry point (moe_route_noalloc): its static
per-GPU workspace gives the tables moe_route gives with a caller's
workspace, call after call, whatever the previous call left in the array."""
import numpy as np
import pytest
import torch

from routing_grouped_expert_router_amd import binding as B
from workloads import configs, generate
from gpu_util import DEV, route_np, say

pytestmark = pytest.mark.gpu

TABLES = ("ids", "w", "phys", "row_of", "slot_of", "src_of", "counts", "offsets", "masked_m",
          "spill_off", "pad_off", "tile_off", "status")

_BASE = configs.tiny()
CASES = [
    # masked with spill, several 64-token blocks
    _BASE.with_(name="noalloc_masked", T=300, H=256, I=128, E=32, E_phys=32, K=4, act_dtype="bf16",
                M_max=30),
    # contiguous with a replica map (Zipf-skewed router bias)
    _BASE.with_(name="noalloc_replicas", T=300, H=256, I=128, E=32, E_phys=40, K=4, act_dtype="bf16",
                layout="contig", BM=16, bias="zipf1.1"),
]


def _logits(cfg, T, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, cfg.E)).astype(np.float32)
    lg[:, : cfg.E // 4] = np.round(lg[:, : cfg.E // 4])      # ties among the first experts
    return torch.from_numpy(lg).to(DEV)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_route_noalloc_matches_route(cfg):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    inp = generate.make_inputs(cfg)
    l2p = rc = None
    max_rep = 1
    if inp.p2l is not None:
        l2p_t, rc_t = B.moe_replica_map_from_p2l(inp.p2l, cfg.E, int(np.bincount(inp.p2l).max()))
        max_rep = l2p_t.shape[1]
        l2p, rc = l2p_t.to(DEV), rc_t.to(DEV)
    d = B.Desc.from_config(cfg, max_replicas=max_rep)
    ws = torch.zeros(B.route_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    # two calls in a row on the same static array, the second with fewer tokens
    for T, seed in ((cfg.T, 1), (37, 2)):
        lg = _logits(cfg, T, seed)
        ref_rt = B.RouteTables(d, DEV)
        got_rt = B.RouteTables(d, DEV)
        B.moe_route(d, lg, T, ref_rt, ws, l2p, rc)
        B.moe_route_noalloc(d, lg, T, got_rt, l2p, rc)
        torch.cuda.synchronize()
        ref, got = route_np(ref_rt, T, cfg.K), route_np(got_rt, T, cfg.K)
        for k in TABLES:
            assert np.array_equal(np.asarray(ref[k]), np.asarray(got[k])), (cfg.name, T, k)
        say(f"  {cfg.name} T={T}: every table bit-identical, status {got['status']}")
