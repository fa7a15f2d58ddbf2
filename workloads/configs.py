"""The synthetic MoE-layer workloads, with their sizes.

Each workload is one MoE layer forward on one GPU: a router over E logical
experts picks K per token, tokens are grouped per physical expert slot, each
slot runs a SwiGLU FFN (gate W1, up W3, down W2) and the route-weighted
results are summed back into token order, plus an always-on shared expert
where ``n_shared`` is 1.

Shapes follow the pages:
  * Mixtral 8x7B: E=8, K=2, H=4096, I=14336 (vllbc blog "MoE inference and
    expert parallelism", routing section, Table 3-1, and the parameter
    accounting that quotes Mixtral's Table 1).
  * DeepSeek-V3: 256 routed + 1 shared expert, K=8, I=2048 (same page,
    Table 3-1; the "推理 INFRA 方法论(5)" page, shape table), H=7168 (the same
    page's DeepEP section, d7168).
  * A fine-grained 512-expert layer with K=10 and redundant slots (the
    "推理 INFRA 方法论(5)" page, shape table row E=512, k=10; vLLM EPLB explainer
    for the physical/logical maps).

Layout terms:
  * ``masked``: a static [E_phys, M_max, H] buffer whose valid rows per slot are
    a device-side count ``masked_m`` (the "推理 INFRA 方法论(5)" page, DeepGEMM
    section); rows past M_max go to a spill region so no token is dropped.
  * ``contig``: expert-grouped rows, each slot's segment padded to BM rows
    (vllbc blog, vLLM forward path: sort and block-align).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens in the batch (B at decode)
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # logical routed experts
    K: int            # experts per token
    E_phys: int       # physical expert slots (== E without redundant slots)
    n_shared: int     # always-on shared experts (0 or 1)
    act_dtype: str    # "f32" | "bf16"  (x and out)
    w_dtype: str      # "bf16" | "fp8"  (fp8 = OCP E4M3FN + fp32 128x128 block scales)
    layout: str       # "masked" | "contig"
    M_max: int        # masked rows per physical slot (masked layout only)
    BM: int           # contiguous-segment padding (contig layout only)
    bias: str         # "none" | "normal0.5" | "zipf1.1"
    seed: int = 0

    @property
    def n_redundant(self) -> int:
        return self.E_phys - self.E

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


def tiny() -> MoEConfig:
    """T=16, H=128, E=8, K=2, I=256, fp32 activations, bf16 weights."""
    return MoEConfig("tiny_t16", T=16, H=128, I=256, E=8, K=2, E_phys=8,
                     n_shared=0, act_dtype="f32", w_dtype="bf16",
                     layout="masked", M_max=16, BM=16, bias="none")


def mixtral_decode(B: int) -> MoEConfig:
    """Mixtral-8x7B-shaped decode layer, B tokens, bf16, masked M_max = B."""
    assert B in (1, 8, 32, 64)
    return MoEConfig(f"mixtral_decode_b{B}", T=B, H=4096, I=14336, E=8, K=2,
                     E_phys=8, n_shared=0, act_dtype="bf16", w_dtype="bf16",
                     layout="masked", M_max=B, BM=16, bias="none")


def dsv3_decode(B: int) -> MoEConfig:
    """DeepSeek-V3-shaped decode layer, fp8 block-128 weights, masked
    M_max = B*K/E*4 (4, 16, 32 at B = 32, 128, 256)."""
    assert B in (32, 128, 256)
    return MoEConfig(f"dsv3_decode_b{B}", T=B, H=7168, I=2048, E=256, K=8,
                     E_phys=256, n_shared=1, act_dtype="bf16", w_dtype="fp8",
                     layout="masked", M_max=B * 8 // 256 * 4, BM=16,
                     bias="none")


def dsv3_prefill(T: int = 8192) -> MoEConfig:
    """DeepSeek-V3-shaped prefill, bf16 weights, contiguous layout, per-expert
    router bias ~ N(0, 0.5)."""
    return MoEConfig(f"dsv3_prefill_t{T}", T=T, H=7168, I=2048, E=256, K=8,
                     E_phys=256, n_shared=1, act_dtype="bf16", w_dtype="bf16",
                     layout="contig", M_max=0, BM=128, bias="normal0.5")


def dsv3_prefill_fp8(T: int = 8192) -> MoEConfig:
    """The DeepSeek-V3-shaped prefill with fp8 block-128 weights (timed on the
    W8A8 path: fp8 activations on fp8 MFMA)."""
    return dsv3_prefill(T).with_(name=f"dsv3_prefill_t{T}_fp8", w_dtype="fp8")


def replica_decode(B: int = 256) -> MoEConfig:
    """512 logical experts in 544 physical slots, K=10, bf16, Zipf(1.1) router
    bias, contiguous layout."""
    return MoEConfig(f"replica_decode_b{B}", T=B, H=4096, I=1024, E=512, K=10,
                     E_phys=544, n_shared=0, act_dtype="bf16", w_dtype="bf16",
                     layout="contig", M_max=0, BM=16, bias="zipf1.1")


def all_configs() -> list[MoEConfig]:
    return ([tiny()] + [mixtral_decode(b) for b in (1, 8, 32, 64)]
            + [dsv3_decode(b) for b in (32, 128, 256)]
            + [dsv3_prefill(), dsv3_prefill_fp8(), replica_decode()])


def by_name(name: str) -> MoEConfig:
    for c in all_configs():
        if c.name == name:
            return c
    raise KeyError(name)
