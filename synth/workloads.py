"""Shapes and recipes of the synthetic MoE-layer workloads.

Each workload is one MoE layer: T tokens of hidden size d, E routed SwiGLU
experts of width f, top-k routing, an optional always-on shared expert of
width f_shared, and the storage dtypes of activations and expert weights.
The model shapes echo the families the pages name (Mixtral 8x7B in
"Expert Parallelism for MoE Serving", §Deep Dive; DeepSeek-V3 with 256 routed
experts, top-8 and a shared expert in "Tensor vs Expert vs Data Parallelism
for MoE Serving", §Context and Background); only their shapes are used.

This module holds no arithmetic of the layer itself.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens in the batch
    d: int            # hidden size
    f: int            # routed-expert FFN width
    E: int            # routed experts
    k: int            # experts chosen per token
    score: str        # "softmax" | "sigmoid"
    renorm: bool      # gates divided by their sum over the chosen k
    n_group: int      # 0 = no group limit
    topk_group: int   # groups kept when n_group > 0
    f_shared: int     # 0 = no shared expert
    act: str          # activation storage: "f32" | "bf16"
    wdt: str          # expert-weight storage: "f32" | "bf16" | "e4m3"
    bias_scale: float  # router bias b_e = -bias_scale * ln(rank_e); 0 = no bias
    capacity_factor: float = 0.0  # 0 = dropless; else slots = ceil(cf * T * k / E)
    dispatch_fp8: bool = False    # dispatched rows as the block-scaled E4M3 payload
    overflow: str = "drop"        # with a capacity: "drop" or "reroute" (next-best expert)

    @property
    def assignments(self) -> int:
        return self.T * self.k

    def scaled(self, **kw) -> "Workload":
        """Same routing and dtype recipe at other sizes (for parity cases)."""
        return replace(self, **kw)


TINY_F32 = Workload("tiny_f32", T=64, d=128, f=256, E=8, k=2, score="softmax",
                    renorm=True, n_group=0, topk_group=0, f_shared=0,
                    act="f32", wdt="f32", bias_scale=0.0)

MIXTRAL_PREFILL = Workload("mixtral8x7b_prefill_bf16", T=4096, d=4096, f=14336,
                           E=8, k=2, score="softmax", renorm=True, n_group=0,
                           topk_group=0, f_shared=0, act="bf16", wdt="bf16",
                           bias_scale=0.0)

DSV3_DECODE = Workload("dsv3_decode_bf16", T=256, d=7168, f=2048, E=256, k=8,
                       score="sigmoid", renorm=True, n_group=0, topk_group=0,
                       f_shared=2048, act="bf16", wdt="bf16", bias_scale=0.0)

# b_e = 1.5 * log(1 / rank_e ** 1.2) = -1.8 * ln(rank_e)
DSV3_PREFILL_SKEW = Workload("dsv3_prefill_skew_bf16", T=16384, d=7168, f=2048,
                             E=256, k=8, score="sigmoid", renorm=True,
                             n_group=8, topk_group=4, f_shared=2048,
                             act="bf16", wdt="bf16", bias_scale=1.8)

# Zipf(1.0) popularity with the same 1.5 coefficient: b_e = -1.5 * ln(rank_e)
QWEN_FP8_SKEW = Workload("qwen_moe_fp8_skew", T=8192, d=4096, f=1536, E=128,
                         k=8, score="softmax", renorm=True, n_group=0,
                         topk_group=0, f_shared=0, act="bf16", wdt="e4m3",
                         bias_scale=1.5)

# One GPU's share of the DeepSeek-V3-shaped prefill layer under 8-way expert
# parallelism ("Expert-Parallel MoE Inference: Serving Sparse Models at
# Scale", section "Deeper Analysis", the worked sizing of rows per expert and
# GPU): 32 local experts and T*k/8 = 16384 routed rows; each GPU runs the
# replicated shared expert on its own 2048 tokens.  The cross-GPU exchange
# is not modelled -- only the per-GPU kernel shape.
DSV3_EP8_SHARD = Workload("dsv3_ep8_shard_bf16", T=2048, d=7168, f=2048, E=32,
                          k=8, score="sigmoid", renorm=True, n_group=0,
                          topk_group=0, f_shared=2048, act="bf16", wdt="bf16",
                          bias_scale=0.0)

ALL = (TINY_F32, MIXTRAL_PREFILL, DSV3_DECODE, DSV3_PREFILL_SKEW, QWEN_FP8_SKEW, DSV3_EP8_SHARD)
BY_NAME = {w.name: w for w in ALL}
# Default seed of each workload: its position in ALL, counting from 1.
DEFAULT_SEED = {w.name: i + 1 for i, w in enumerate(ALL)}
