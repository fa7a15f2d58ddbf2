"""Helpers for the GPU parity tests: build a layer on the device from the
synthetic workload, and compare against the CPU reference."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O
from routing_grouped_expert_router_amd import binding as B
from workloads import generate
from oracle_adapt import to_f64, oracle_forward

DEV = "cuda"

# max|d| / max|ref| bars for the layer output, by weight format
TOL = {"bf16": 1e-2, "fp8": 3e-2}


def say(*a):
    print(*a, flush=True)


_DEFAULT = object()


class Built:
    """A workload on the GPU: inputs, uploaded weights and a MoELayer."""

    def __init__(self, cfg, T=None, layout=None, M_max=None, p2l=_DEFAULT, packed=False, grouped=None,
                 a8=False):
        if layout is not None:
            cfg = cfg.with_(layout=layout)
        if M_max is not None:
            cfg = cfg.with_(M_max=M_max)
        self.cfg = cfg
        self.inp = generate.make_inputs(cfg, wdevice=DEV)
        if p2l is not _DEFAULT:
            self.inp.p2l = p2l
        self.T = cfg.T if T is None else T
        self.inp.x = self.inp.x[: self.T].contiguous()   # the reference sees T tokens
        self.weights = generate.upload_weights(self.inp, DEV)
        self.l2p = self.rcount = None
        max_rep = 1
        if self.inp.p2l is not None:
            l2p, cnt = O.replica_tables(self.inp.p2l, cfg.E)
            max_rep = l2p.shape[1]
            self.l2p = torch.from_numpy(l2p).to(DEV)
            self.rcount = torch.from_numpy(cnt).to(DEV)
        self.d = B.Desc.from_config(cfg, max_replicas=max_rep, w_packed=int(packed))
        if packed:
            self.weights = B.pack_expert_weights(self.d, self.weights)
        self.x = self.inp.x.to(DEV)
        self.wr = self.inp.w_router.to(DEV)
        self.bias = None if self.inp.bias is None else self.inp.bias.to(DEV)
        # grouped: grouped_topk_route's keyword arguments (score_bias as numpy)
        self.grouped = grouped
        router = None
        if grouped is not None:
            sb = grouped.get("score_bias")
            router = B.GroupedRouter(grouped["n_group"], grouped["topk_group"], grouped["group_k"],
                                     grouped.get("renormalize", True), grouped.get("scale", 1.0),
                                     None if sb is None else torch.from_numpy(np.asarray(sb, np.float32)).to(DEV))
        self.a8 = a8
        self.layer = B.MoELayer(self.d, self.weights, self.wr, self.bias, self.l2p, self.rcount, DEV,
                                router=router, a8=a8)

    def oracle_logits(self) -> np.ndarray:
        return O.router_logits(to_f64(self.inp.x), to_f64(self.inp.w_router),
                               None if self.inp.bias is None else self.inp.bias.numpy())

    def run(self, logits_np=None, fused_gather=True):
        lg = None if logits_np is None else torch.from_numpy(np.ascontiguousarray(logits_np)).to(DEV)
        out = self.layer.forward(self.x[: self.T], self.T, logits=lg, fused_gather=fused_gather)
        torch.cuda.synchronize()
        return out

    def oracle(self, logits_np=None, tokens=None, slots=None):
        if self.a8:
            from oracle_adapt import oracle_forward_w8a8
            assert self.grouped is None
            return oracle_forward_w8a8(self.inp, logits=logits_np, tokens=tokens)
        return oracle_forward(self.inp, logits=logits_np, tokens=tokens, grouped=self.grouped, slots=slots)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def out_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def route_np(rt: B.RouteTables, T: int, K: int) -> dict:
    g = lambda t, n: t[:n].cpu().numpy()
    return dict(ids=g(rt.topk_ids, T * K).reshape(T, K), w=g(rt.topk_w, T * K).reshape(T, K),
                phys=g(rt.topk_phys, T * K).reshape(T, K),
                row_of=g(rt.row_of, T * K).reshape(T, K), slot_of=g(rt.slot_of, T * K).reshape(T, K),
                src_of=g(rt.src_of, T * K), counts=rt.counts.cpu().numpy(),
                offsets=rt.offsets.cpu().numpy(), masked_m=rt.masked_m.cpu().numpy(),
                spill_off=rt.spill_off.cpu().numpy(), pad_off=rt.pad_off.cpu().numpy(),
                tile_off=rt.tile_off.cpu().numpy(), status=int(rt.status.cpu().numpy()[0]))


TILE_ROWS = 256   # token rows per work item of the large-group kernels (moe_route_t.tile_off)


def tile_off_expected(counts, T: int, n_shared: int):
    """tile_off as moe.h defines it: exclusive prefix sum of ceil(count/256)
    over the slots, the total, then the total plus the shared expert's
    ceil(T/256) tiles."""
    t = -(-np.asarray(counts, dtype=np.int64) // TILE_ROWS)
    pre = np.concatenate([[0], np.cumsum(t)])
    shared = -(-T // TILE_ROWS) if n_shared else 0
    return np.concatenate([pre, [pre[-1] + shared]]).astype(np.int32)


def weight_tol(K: int) -> float:
    """Bound on |w_gpu - w_ref| for the renormalised weights: each of the K
    fp32 exponentials carries <= 2 ulp, the sum K-1 roundings, the quotient
    one: (K + 4) * 2^-23 relative, on weights <= 1."""
    return (K + 4) * 2.0 ** -23


def covering_tokens(counts, offsets, src_of, T: int, n_shared: int, tiles=(128, 256)):
    """Token ids whose outputs cover every group of a routed batch at the
    places a tiled kernel can get wrong: the first and the last row of every
    slot with tokens, and the rows on both sides of every boundary between
    row tiles of the given heights (the last, partial tile of each group
    included); the shared expert's group is the tokens in order, so its
    boundaries are token ids."""
    counts = np.asarray(counts)
    offsets = np.asarray(offsets)
    src_of = np.asarray(src_of)
    toks = {0, T - 1}

    def ranks(R):
        r = {0, R - 1}
        for h in tiles:
            for j in range(1, (R - 1) // h + 1):
                r |= {h * j - 1, h * j}
        return r

    for p in np.nonzero(counts)[0]:
        for r in ranks(int(counts[p])):
            toks.add(int(src_of[offsets[p] + r]))
    if n_shared:
        toks |= ranks(T)
    return np.array(sorted(toks), dtype=np.int64)
