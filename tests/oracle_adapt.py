"""Adapters from the synthetic-input tensors (torch, CPU) to the numpy arrays
the CPU reference takes.  Test infrastructure: decoding uses the reference's
own bf16 / e4m3 decoders."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return O.decode_bf16(t.contiguous().view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    raise TypeError(t.dtype)


def expert_f64(ew, w_dtype: str):
    if w_dtype == "bf16":
        return to_f64(ew.w1), to_f64(ew.w3), to_f64(ew.w2)
    return (O.dequant_block128(ew.w1.numpy(), ew.s1.numpy()),
            O.dequant_block128(ew.w3.numpy(), ew.s3.numpy()),
            O.dequant_block128(ew.w2.numpy(), ew.s2.numpy()))


class _Ahead:
    """Decodes the fp64 weights of the slots the reference will ask for next
    on a few threads (numpy releases the GIL while it converts), keeping a
    bounded window in memory.  The reference walks the slots in ascending
    order, so ``order`` is that walk; a slot outside it is decoded on demand.
    Pure scheduling: every value is expert_f64 of the same tensors."""

    def __init__(self, order, fetch, depth=8):
        from concurrent.futures import ThreadPoolExecutor
        self.order = list(order)
        self.pos = {p: i for i, p in enumerate(self.order)}
        self.fetch = fetch
        self.depth = depth
        self.pool = ThreadPoolExecutor(max_workers=depth)
        self.futs = {}

    def get(self, p):
        i = self.pos.get(p)
        if i is None:
            return self.fetch(p)
        for j in range(i, min(len(self.order), i + self.depth)):
            q = self.order[j]
            if q not in self.futs:
                self.futs[q] = self.pool.submit(self.fetch, q)
        for q in [q for q in self.futs if self.pos[q] < i]:
            self.futs.pop(q)          # already consumed: drop the reference
        return self.futs.pop(p).result()

    def close(self):
        self.pool.shutdown(wait=True)


def oracle_forward(inp, logits=None, tokens=None, layout=None, grouped=None, local_of=None,
                   E_local=None, slots=None):
    """Runs the reference on workload inputs ``inp`` (workloads.generate).
    ``local_of`` (over the workload's physical slots) makes it one rank's
    expert-parallel share with ``E_local`` local slots (default: the number
    of local entries).  ``slots``, the ascending slots the reference will
    read (those with a sampled token), lets their weights be decoded ahead
    on several threads."""
    cfg = inp.cfg
    cache = {}
    E_phys = cfg.E_phys
    glob = None
    if local_of is not None:
        local_of = np.asarray(local_of, dtype=np.int32)
        E_phys = int((local_of >= 0).sum()) if E_local is None else E_local
        glob = {int(q): p for p, q in enumerate(local_of) if q >= 0}

    import threading
    lock = threading.Lock()

    def decode(p):
        if glob is not None:
            p = glob[p]
        with lock:                     # the inputs' expert cache is not thread-safe
            ew = inp.expert(inp.slot_logical(p))
        return expert_f64(ew, cfg.w_dtype)

    ahead = _Ahead(slots, decode) if slots is not None else None

    def slot_weights(p):
        if ahead is not None:
            return ahead.get(p)
        if glob is not None:
            p = glob[p]
        l = inp.slot_logical(p)
        if l not in cache:
            if len(cache) > 2:
                cache.pop(next(iter(cache)))
            cache[l] = expert_f64(inp.expert(l), cfg.w_dtype)
        return cache[l]

    shared = expert_f64(inp.shared(), cfg.w_dtype) if cfg.n_shared else None
    try:
        return O.moe_forward(
            to_f64(inp.x), to_f64(inp.w_router),
            None if inp.bias is None else inp.bias.numpy(),
            cfg.K, E_phys, slot_weights, shared, p2l=inp.p2l,
            layout=layout or cfg.layout, M_max=cfg.M_max, BM=cfg.BM,
            logits=logits, tokens=tokens, grouped=grouped, local_of=local_of)
    finally:
        if ahead is not None:
            ahead.close()


def expert_codes(ew):
    """fp8 weights -> (q1, s1, q3, s3, q2, s2) as numpy (W8A8 reference)."""
    return (ew.w1.numpy(), ew.s1.numpy(), ew.w3.numpy(), ew.s3.numpy(), ew.w2.numpy(), ew.s2.numpy())


def oracle_forward_w8a8(inp, logits=None, tokens=None, layout=None, local_of=None, E_local=None):
    """oracle_forward with the W8A8 experts (fp8 weights only)."""
    cfg = inp.cfg
    assert cfg.w_dtype == "fp8"
    cache = {}
    E_phys = cfg.E_phys
    glob = None
    if local_of is not None:
        local_of = np.asarray(local_of, dtype=np.int32)
        E_phys = int((local_of >= 0).sum()) if E_local is None else E_local
        glob = {int(q): p for p, q in enumerate(local_of) if q >= 0}

    def codes(p):
        if glob is not None:
            p = glob[p]
        l = inp.slot_logical(p)
        if l not in cache:
            if len(cache) > 2:
                cache.pop(next(iter(cache)))
            cache[l] = expert_codes(inp.expert(l))
        return cache[l]

    shared = expert_codes(inp.shared()) if cfg.n_shared else None
    return O.moe_forward(
        to_f64(inp.x), to_f64(inp.w_router),
        None if inp.bias is None else inp.bias.numpy(),
        cfg.K, E_phys, None, None, p2l=inp.p2l,
        layout=layout or cfg.layout, M_max=cfg.M_max, BM=cfg.BM,
        logits=logits, tokens=tokens, local_of=local_of, expert_codes=codes, shared_codes=shared)
