"""Workload table: the five MoE-layer shapes the hot path is checked and timed on.

Shapes follow the models the pages name: Mixtral 8x7B (2-4 of 8 experts per GPU,
"MoE 服務的專家並行性", real-world deployments), DeepSeek-V3 (256 routed + 1 shared
expert, top-8, "总览" glossary and tbl-ep-02), Switch-style top-1/top-2 routing, and
the Kimi-K2 hot-expert skew ("Expert-Parallelism" wiki, observation 1).

Every field is a plain number or flag; the meaning of each flag is defined by the
oracle and by the C-ABI header, not here.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                  # tokens routed by this GPU (B on the pages)
    h: int                  # hidden size
    E: int                  # routed experts in the layer
    K: int                  # experts per token
    inter: int              # SwiGLU intermediate size of one routed expert
    dtype: str = "bf16"     # activation / expert-weight dtype: "f32" or "bf16"
    score: str = "softmax"  # "softmax" or "sigmoid"
    renorm: bool = True     # weights renormalised over the selected K
    n_groups: int = 1       # expert groups for group-limited routing (1 = off)
    topk_groups: int = 1    # groups a token may use
    capacity_factor: float = 0.0  # <= 0: no capacity limit
    pad: bool = False       # pad each local expert buffer to capacity
    n_ep: int = 1           # virtual EP ranks
    ep_rank: int = 0        # the rank this GPU plays
    n_shared: int = 0       # shared experts (0 or 1)
    shared_inter: int = 0
    bias: str = "none"      # "none" | "gauss" | "zipf"
    bias_var: float = 0.0   # variance of the gauss bias
    zipf_s: float = 0.0     # exponent of the zipf popularity bias
    keys: str = "router"    # "router": x @ W_r;  "uniform": iid U(0,1) keys, no x
    seed: int = 0

    @property
    def act_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def E_local(self) -> int:
        return self.E // self.n_ep

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    # Tiny fp32 layer: correctness at sizes a pure-Python walk finishes at once.
    "tiny_f32": MoEConfig(
        name="tiny_f32", T=64, h=128, E=8, K=2, inter=256, dtype="f32",
        score="softmax", capacity_factor=1.25),
    # Mixtral-shaped prefill on one GPU holding all 8 experts.
    "mixtral_prefill": MoEConfig(
        name="mixtral_prefill", T=4096, h=4096, E=8, K=2, inter=14336,
        dtype="bf16", score="softmax"),
    # DeepSeek-V3-shaped local share at EP=8: experts 0..31 plus one shared expert.
    "dsv3_ep8": MoEConfig(
        name="dsv3_ep8", T=4096, h=7168, E=256, K=8, inter=2048, dtype="bf16",
        score="sigmoid", n_groups=8, topk_groups=4, n_ep=8, ep_rank=0,
        n_shared=1, shared_inter=2048, bias="gauss", bias_var=0.01),
    # Zipf-skewed routing, capacity factor 1.0 (drops) and unlimited (no drops).
    "skew_cap1": MoEConfig(
        name="skew_cap1", T=8192, h=2048, E=64, K=6, inter=1408, dtype="bf16",
        score="softmax", bias="zipf", zipf_s=1.2, capacity_factor=1.0),
    "skew_nodrop": MoEConfig(
        name="skew_nodrop", T=8192, h=2048, E=64, K=6, inter=1408, dtype="bf16",
        score="softmax", bias="zipf", zipf_s=1.2),
    # Decode-sized batch with DeepSeek-V3 expert shapes, all 256 experts resident.
    "dsv3_decode": MoEConfig(
        name="dsv3_decode", T=32, h=7168, E=256, K=8, inter=2048, dtype="bf16",
        score="sigmoid", n_groups=8, topk_groups=4, bias="gauss", bias_var=0.01),
    # Layout only: B=512, top-8 of 256, EP=64, uniform random routing; h=7168 bf16
    # sizes the send-count matrix in bytes (the DeepSeek-V3 row of tbl-ep-02).
    "layout_ep64": MoEConfig(
        name="layout_ep64", T=512, h=7168, E=256, K=8, inter=0, dtype="bf16",
        score="softmax", n_ep=64, keys="uniform"),
}


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]
