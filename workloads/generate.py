"""Seeded synthetic inputs for the MoE-layer workloads.

This module only draws and encodes inputs; it holds none of the layer's
arithmetic (no routing, grouping, FFN or combine).  Both the CPU reference and
the GPU path consume exactly the tensors produced here.

Recipe (every seed defaults to 0):
  * every tensor has its own torch generator, seeded from
    ``numpy.random.SeedSequence(seed, spawn_key=(tag, index, part))`` so any
    single expert can be regenerated without drawing the others;
  * x, W_r and the bias are always drawn on the CPU; expert weights are drawn
    on the device they are used on (torch's CPU and GPU generators give
    different streams, so a GPU run and a CPU run of one workload hold
    different expert weights; each run compares both sides on the same ones);
  * activations x ~ N(0, 1): fp32, or bf16 by round-to-nearest-even;
  * router weight W_r [E, H] and expert weights W1, W3 [I, H], W2 [H, I]
    ~ N(0, 0.02) in fp32, then bf16 (RNE) or OCP E4M3FN with one fp32 scale
    per 128x128 block: s = amax(block) / 448, q = RNE(clamp(w / s, +-448));
  * router bias: none, N(0, 0.5) per expert, or Zipf(1.1) over a seeded
    permutation of the experts: bias_e = ln(r_e^-1.1 / sum_i i^-1.1);
  * redundant physical slots (E_phys > E) go greedily to the logical expert
    with the largest expected load per replica, the load being the Zipf
    probability (the replicate-hot-experts step the EPLB passages describe).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from .configs import MoEConfig

# spawn-key tags
_TAG_X, _TAG_WR, _TAG_BIAS, _TAG_EXPERT, _TAG_SHARED = 0, 1, 2, 3, 4
_PART_W1, _PART_W3, _PART_W2 = 0, 1, 2

W_STD = 0.02
E4M3_MAX = 448.0
FP8_BLOCK = 128


def _gen(seed: int, *key: int, device="cpu") -> torch.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=tuple(key))
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    return g


def _normal(shape, std: float, seed: int, *key: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, *key, device=device)
    t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_e4m3_block128(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Synthetic fp8 encoding of a [R, C] fp32 matrix (R, C multiples of 128):
    returns (q uint8 [R, C] holding E4M3FN bytes, s fp32 [R/128, C/128])."""
    R, C = w.shape
    assert R % FP8_BLOCK == 0 and C % FP8_BLOCK == 0
    blk = w.reshape(R // FP8_BLOCK, FP8_BLOCK, C // FP8_BLOCK, FP8_BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (blk / s[:, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    q = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return q.contiguous(), s.contiguous()


@dataclass
class ExpertWeights:
    """One SwiGLU expert: W1 (gate) [I, H], W3 (up) [I, H], W2 (down) [H, I].
    bf16 tensors, or uint8 E4M3FN bytes with fp32 block scales s1, s3, s2."""
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    s1: torch.Tensor | None = None
    s3: torch.Tensor | None = None
    s2: torch.Tensor | None = None


def _encode(w: torch.Tensor, w_dtype: str):
    if w_dtype == "bf16":
        return w.to(torch.bfloat16), None
    if w_dtype == "fp8":
        return quantize_e4m3_block128(w)
    raise ValueError(w_dtype)


def make_expert(cfg: MoEConfig, tag: int, index: int, device="cpu") -> ExpertWeights:
    w1, s1 = _encode(_normal((cfg.I, cfg.H), W_STD, cfg.seed, tag, index, _PART_W1, device=device), cfg.w_dtype)
    w3, s3 = _encode(_normal((cfg.I, cfg.H), W_STD, cfg.seed, tag, index, _PART_W3, device=device), cfg.w_dtype)
    w2, s2 = _encode(_normal((cfg.H, cfg.I), W_STD, cfg.seed, tag, index, _PART_W2, device=device), cfg.w_dtype)
    return ExpertWeights(w1, w3, w2, s1, s3, s2)


def zipf_probs(cfg: MoEConfig) -> np.ndarray:
    """Zipf(1.1) probability of each logical expert, over a seeded permutation."""
    rng = np.random.default_rng(np.random.SeedSequence(cfg.seed, spawn_key=(_TAG_BIAS, 1)))
    rank = rng.permutation(cfg.E) + 1
    h = np.sum(np.arange(1, cfg.E + 1, dtype=np.float64) ** -1.1)
    return rank.astype(np.float64) ** -1.1 / h


def make_bias(cfg: MoEConfig) -> torch.Tensor | None:
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal0.5":
        return _normal((cfg.E,), 0.5, cfg.seed, _TAG_BIAS, 0)
    if cfg.bias == "zipf1.1":
        return torch.from_numpy(np.log(zipf_probs(cfg)).astype(np.float32))
    raise ValueError(cfg.bias)


def make_score_bias(cfg: MoEConfig, std: float = 0.05) -> torch.Tensor:
    """Per-expert selection bias [E] of the grouped sigmoid router, seeded
    ~N(0, std) (the load-balancing correction a trained model carries)."""
    return _normal((cfg.E,), std, cfg.seed, _TAG_BIAS, 2)


def make_p2l(cfg: MoEConfig) -> np.ndarray | None:
    """physical_to_logical map [E_phys]: slots [0, E) are home slots; each
    redundant slot replicates the logical expert with the largest
    expected-load / replica-count (ties to the lower id)."""
    if cfg.E_phys == cfg.E:
        return None
    load = zipf_probs(cfg) if cfg.bias == "zipf1.1" else np.ones(cfg.E)
    reps = np.ones(cfg.E, dtype=np.int64)
    p2l = list(range(cfg.E))
    for _ in range(cfg.E_phys - cfg.E):
        l = int(np.argmax(load / reps))   # first maximum = lower id
        reps[l] += 1
        p2l.append(l)
    return np.asarray(p2l, dtype=np.int32)


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor                      # [T, H] fp32 or bf16
    w_router: torch.Tensor               # [E, H] bf16
    bias: torch.Tensor | None            # [E] fp32
    p2l: np.ndarray | None               # [E_phys] int32
    wdevice: str = "cpu"                 # where expert weights are drawn
    _cache: dict = field(default_factory=dict, repr=False)

    def prefetch(self, ids) -> None:
        """Keeps the CPU copies of these logical experts (and the shared one)
        resident, so later reads do no generation or device copy."""
        pinned = self._cache.setdefault("pinned", {})
        for l in ids:
            if l not in pinned:
                pinned[l] = _to_cpu(make_expert(self.cfg, _TAG_EXPERT, int(l), self.wdevice))
        self.shared()

    def expert(self, l: int) -> ExpertWeights:
        """Weights of logical expert l as CPU tensors (drawn on ``wdevice``,
        regenerated on demand, small LRU)."""
        pinned = self._cache.get("pinned", {})
        if l in pinned:
            return pinned[l]
        if l not in self._cache:
            lru = [k for k in self._cache if k not in ("pinned", "shared")]
            if len(lru) >= 4:
                self._cache.pop(lru[0])
            self._cache[l] = _to_cpu(make_expert(self.cfg, _TAG_EXPERT, l, self.wdevice))
        return self._cache[l]

    def shared(self) -> ExpertWeights | None:
        if self.cfg.n_shared == 0:
            return None
        if "shared" not in self._cache:
            self._cache["shared"] = _to_cpu(make_expert(self.cfg, _TAG_SHARED, 0, self.wdevice))
        return self._cache["shared"]

    def slot_logical(self, p: int) -> int:
        return p if self.p2l is None else int(self.p2l[p])


def _to_cpu(ew: ExpertWeights) -> ExpertWeights:
    f = lambda t: None if t is None else t.cpu()
    return ExpertWeights(f(ew.w1), f(ew.w3), f(ew.w2), f(ew.s1), f(ew.s3), f(ew.s2))


def make_inputs(cfg: MoEConfig, T: int | None = None, wdevice="cpu") -> MoEInputs:
    """Inputs for ``cfg``; ``T`` (<= cfg.T) takes the first T tokens only;
    expert weights are drawn on ``wdevice``."""
    x = _normal((cfg.T, cfg.H), 1.0, cfg.seed, _TAG_X)
    if T is not None:
        x = x[:T].contiguous()
    if cfg.act_dtype == "bf16":
        x = x.to(torch.bfloat16)
    wr = _normal((cfg.E, cfg.H), W_STD, cfg.seed, _TAG_WR).to(torch.bfloat16)
    return MoEInputs(cfg, x, wr, make_bias(cfg), make_p2l(cfg), str(wdevice))


def upload_weights(inp: MoEInputs, device, slots=None) -> dict:
    """Stacks expert weights per physical slot on ``device``:
    w1, w3 [G, I, H], w2 [G, H, I] (+ fp8 scales), G = E_phys (+1 shared slot
    appended last).  Replica slots hold copies of their logical expert.
    ``slots`` restricts which slots are filled (others stay zero).  Weights
    are drawn on ``inp.wdevice`` (which must be ``device`` or "cpu")."""
    cfg = inp.cfg
    G = cfg.E_phys + cfg.n_shared
    wdt = torch.bfloat16 if cfg.w_dtype == "bf16" else torch.uint8
    out = {
        "w1": torch.zeros((G, cfg.I, cfg.H), dtype=wdt, device=device),
        "w3": torch.zeros((G, cfg.I, cfg.H), dtype=wdt, device=device),
        "w2": torch.zeros((G, cfg.H, cfg.I), dtype=wdt, device=device),
    }
    if cfg.w_dtype == "fp8":
        out["s1"] = torch.ones((G, cfg.I // 128, cfg.H // 128), dtype=torch.float32, device=device)
        out["s3"] = torch.ones((G, cfg.I // 128, cfg.H // 128), dtype=torch.float32, device=device)
        out["s2"] = torch.ones((G, cfg.H // 128, cfg.I // 128), dtype=torch.float32, device=device)
    want = range(G) if slots is None else slots
    # generate each logical expert once, copy into every slot that holds it
    by_logical: dict[int, list[int]] = {}
    for p in want:
        key = -1 if p == cfg.E_phys else inp.slot_logical(p)
        by_logical.setdefault(key, []).append(p)
    for l, ps in by_logical.items():
        if l == -1:
            ew = make_expert(cfg, _TAG_SHARED, 0, inp.wdevice)
        else:
            ew = make_expert(cfg, _TAG_EXPERT, l, inp.wdevice)
        for p in ps:
            out["w1"][p].copy_(ew.w1)
            out["w3"][p].copy_(ew.w3)
            out["w2"][p].copy_(ew.w2)
            if cfg.w_dtype == "fp8":
                out["s1"][p].copy_(ew.s1)
                out["s3"][p].copy_(ew.s3)
                out["s2"][p].copy_(ew.s2)
    return out
