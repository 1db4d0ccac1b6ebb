"""Workload shapes of the routed MoE layer.

Shapes follow the pages on DeepSeek V4 Flash:
- 256 routed experts with top-6 selection plus one shared expert, hidden size 4096,
  expert intermediate size 2048, vocabulary 129,280 (TensorSharp "DeepSeek V4 Flash"
  introduction; aimarketly model card "Speeds, Sizes, Times").
- A DSpark verify step of 64 requests x 8 rows = 512 rows and prefill dispatches of
  512 tokens (pypto.ai "DeepSeek V4-Flash, DSpark point", deployment configuration table).
- hash routing from a token-id -> expert-id table (model card "Model Architecture and
  Objective"; TensorSharp "How TensorSharp runs it").
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class MoEShape:
    name: str
    n_rows: int          # N token rows in one call
    d_model: int         # d, hidden size (K of gate/up, rows of down)
    n_experts: int       # E routed experts
    top_k: int           # k experts per row
    d_ff: int            # I, expert intermediate size
    routing: str         # "topk" (sqrt-softplus top-k) or "hash"
    weight_set: str      # which seeded weight family the experts come from
    bias: str = "none"   # "none" or "zipf": logit bias steering the expert load
    vocab: int = 129280  # hash-routing table rows
    route_scale: float = 1.0
    swiglu_limit: float = 10.0

    @property
    def pairs(self) -> int:
        return self.n_rows * self.top_k


SHAPES = {
    # 32 rows, d 256, 16 experts top-2 + 1 shared, intermediate 128
    "tiny": MoEShape("tiny", 32, 256, 16, 2, 128, "topk", "tiny"),
    # DSpark verify step: 64 requests x 8 rows
    "verify512": MoEShape("verify512", 512, 4096, 256, 6, 2048, "topk", "v4layer"),
    # one request's verify block
    "decode8": MoEShape("decode8", 8, 4096, 256, 6, 2048, "topk", "v4layer"),
    # 16 prefill chunks of 512 rows in one call
    "prefill8192": MoEShape("prefill8192", 8192, 4096, 256, 6, 2048, "topk", "v4layer"),
    # skewed load: logit bias so per-row selection probability follows Zipf(1.2) by rank
    "zipf2048": MoEShape("zipf2048", 2048, 4096, 256, 6, 2048, "topk", "v4layer", bias="zipf"),
    # hash-routed: experts from a seeded [129280][6] table, uniform token ids
    "hash2048": MoEShape("hash2048", 2048, 4096, 256, 6, 2048, "hash", "v4layer"),
    # DSpark drafter MoE slab: 64 requests x one 7-row draft query block
    "draft448": MoEShape("draft448", 448, 4096, 256, 6, 2048, "topk", "v4layer"),
    # the same slab at ds4's draft block size of 5 rows per request
    "draft320": MoEShape("draft320", 320, 4096, 256, 6, 2048, "topk", "v4layer"),
}

# Stable numeric tags for the seeded streams of each workload and weight family.
CFG_TAG = {"tiny": 0, "verify512": 1, "decode8": 2, "prefill8192": 3, "zipf2048": 4, "hash2048": 5,
           "draft448": 6, "draft320": 7}
SET_TAG = {"tiny": 100, "v4layer": 101}

# Parameters of the synthetic distributions (standard deviations).
ROUTER_STD = 0.02


def expert_std(fan_in: int) -> float:
    return 1.0 / fan_in ** 0.5
