"""The synthetic MoE workloads, by name.

  c1   tiny: 8 experts, K=256, N=512, 32 tokens each routed to 2 distinct experts
       uniformly at random -> 0..16 rows per expert
  c2   one dense GEMM, M = N = K = 8192 (a single expert)
  c3   decode gate+up shard: 256 experts, 512 tokens top-8 -> exactly 16 rows per
       expert, K=6144, N=512
  c4   decode down-projection shard: 256 experts, 1024 tokens top-8 -> exactly 32
       rows per expert, K=256, N=6144
  c5   skewed: 256 experts, 4096 tokens top-8, expert popularity Zipf(1.1),
       K=6144, N=512 (each token takes 8 distinct experts)
  c5b  skewed, i.i.d. reading: 4096 routed rows drawn independently from the same
       Zipf popularity (leaves some experts empty)

Activations and weights are N(0,1).  Activations are one row per token (BF16),
quantised once per token; the grouped problem reads them through a row index.
Weights have one tensor scale per expert.  Seeds: routing 100+i, activations
200+i, weights 300+i for workload ci (c5b uses i=6).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import gen


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    experts: int
    n: int
    k: int
    tokens: int
    topk: int
    routing: str  # "uniform", "balanced", "dense", "zipf_topk", "zipf_iid"
    zipf_s: float = 1.1

    @property
    def seed_routing(self) -> int:
        return 100 + self.index

    @property
    def seed_act(self) -> int:
        return 200 + self.index

    @property
    def seed_weight(self) -> int:
        return 300 + self.index


WORKLOADS = {
    "c1": Workload("c1", 1, 8, 512, 256, 32, 2, "uniform"),
    "c2": Workload("c2", 2, 1, 8192, 8192, 8192, 1, "dense"),
    "c3": Workload("c3", 3, 256, 512, 6144, 512, 8, "balanced"),
    "c4": Workload("c4", 4, 256, 6144, 256, 1024, 8, "balanced"),
    "c5": Workload("c5", 5, 256, 512, 6144, 4096, 8, "zipf_topk"),
    "c5b": Workload("c5b", 6, 256, 512, 6144, 4096, 1, "zipf_iid"),
}


def routing(w: Workload):
    """(row_token int32[m_total], offsets int32[E+1]) of a workload."""
    if w.routing == "uniform":
        assign = gen.route_uniform_topk(w.tokens, w.experts, w.topk, w.seed_routing)
    elif w.routing == "balanced":
        assign = gen.route_balanced(w.tokens, w.experts, w.topk, w.seed_routing)
    elif w.routing == "dense":
        assign = np.zeros((w.tokens, 1), dtype=np.int32)
    elif w.routing == "zipf_topk":
        assign = gen.route_zipf_topk(w.tokens, w.experts, w.topk, w.zipf_s, w.seed_routing)
    elif w.routing == "zipf_iid":
        assign = gen.route_zipf_iid(w.tokens, w.experts, w.zipf_s, w.seed_routing)
    else:
        raise ValueError(w.routing)
    return gen.group_by_expert(assign, w.experts)


def activations(w: Workload, tokens: int | None = None) -> np.ndarray:
    """BF16-valued float32 token activations [tokens][K]."""
    t = w.tokens if tokens is None else tokens
    return gen.bf16_round(gen.normal((t, w.k), w.seed_act))


def expert_weight(w: Workload, e: int) -> np.ndarray:
    """Float32 N(0,1) weights [N][K] of expert e."""
    return gen.expert_weight(e, w.n, w.k, w.seed_weight)
