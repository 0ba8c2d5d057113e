"""Seeded synthetic inputs for the routed-MoE routing step.

This module only draws random numbers and arranges them into the shapes of
the routing workloads. It holds none of the routing method's arithmetic
(no sigmoid, no bias add, no selection, no rounding of results), so both the
CPU oracle (``oracle/``) and the HIP path may take their inputs from here
without sharing any part of the method.

Shapes and distributions follow the pages' model: 896 routed experts with
top-k 16, selected per token by a sigmoid router with a correction bias and a
grouped top-k ("[kimi-k3] Rank-local expert ids for the EP routed MoE",
commit message; "[ROCm][Perf] Kimi-K3: token-sharded residual stream for long
prefills", author's reply on shard-routed test coverage). Expert-parallel
rank ranges are contiguous runs of 112 experts (EP8). The router weight is
[896, 7168] ("feat(kimi): tensor- and expert-parallel sharding for the K3.1
decoder", memory table: router 0.59 B parameters over 92 layers).

The grouping constants (8 groups of 112, keep 4, group score = sum of the top
2 biased scores) are the workload definition used throughout this repository.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

E = 896          # routed experts
G = 8            # expert groups
TG = 4           # groups kept per token
K = 16           # experts selected per token
TOPN = 2         # group score = sum of the top TOPN biased scores of a group
H = 7168         # hidden size of the router GEMM
EP = 8           # expert-parallel degree of the rank-range workloads
RANGE = E // EP  # 112 experts per rank
FUSED_TOKEN_CAP = 64

SEED_BASE = 20261000

# Zipf skew of the long-prefill bias: bias_e += ZIPF_ALPHA * rank_e ** -ZIPF_S,
# ranks 1..E assigned by a seeded permutation.  ZIPF_ALPHA was chosen so that
# the hottest expert receives about 10x the mean load; a CPU test checks the
# resulting load ratio with the oracle.
ZIPF_S = 1.1
ZIPF_ALPHA = 0.19

DECODE_SWEEP_T = (5, 8, 16, 24, 32, 64)

# Twin expert pairs (src -> dst) of the decode sweep: dst copies src's logit
# column and bias, so their biased scores tie exactly in every row.  Pairs sit
# inside one group / rank range and across groups and ranges; 9 of 896
# columns (~1%) are duplicates.
TWIN_PAIRS = (
    (10, 11),    # same group 0
    (120, 200),  # same group 1
    (340, 345),  # same group 3
    (450, 500),  # same group 4
    (100, 130),  # group 0 -> group 1
    (300, 700),  # group 2 -> group 6
    (560, 895),  # group 5 -> group 7
    (5, 890),    # group 0 -> group 7
    (420, 470),  # group 3 -> group 4
)


def seed_for(config: int, T: int, variant: int = 0) -> int:
    """Seed of workload `config` at T tokens (variant > 0: rotated copies)."""
    return SEED_BASE + 100 * config + T + 1_000_003 * variant


@dataclass
class RouteCase:
    """One routing invocation: inputs plus the rank range to relabel for."""
    name: str
    logits: np.ndarray                 # float32 [T, E]
    bias: np.ndarray                   # float32 [E]
    off: int = 0                       # local_expert_offset
    cnt: int = 0                       # num_local_experts (0 = global ids)
    n_groups: int = G
    topk_group: int = TG
    top_k: int = K
    group_topn: int = TOPN
    hidden: Optional[np.ndarray] = None   # uint16 bf16 bits [T, H] (router GEMM cases)
    weight: Optional[np.ndarray] = None   # uint16 bf16 bits [E, H]
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.logits.shape[0]) if self.logits is not None else int(self.hidden.shape[0])

    @property
    def E(self) -> int:
        return int(self.bias.shape[0])


def normal_logits(rng: np.random.Generator, T: int, e: int = E) -> np.ndarray:
    return rng.standard_normal((T, e), dtype=np.float32)


def normal_bias(rng: np.random.Generator, e: int = E) -> np.ndarray:
    return (0.01 * rng.standard_normal(e)).astype(np.float32)


def _to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with torch's own conversion; return raw bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def tiny_global(T: int = 8) -> RouteCase:
    """8 tokens x 896 experts, N(0,1) logits, N(0,0.01) bias, global ids."""
    rng = np.random.default_rng(seed_for(0, T))
    return RouteCase("tiny_global", normal_logits(rng, T), normal_bias(rng))


def decode_local(T: int = 16, rank: int = 3) -> RouteCase:
    """16 tokens, EP8 rank range [336, 448) -> 128 local ids."""
    rng = np.random.default_rng(seed_for(1, T))
    return RouteCase("decode_local", normal_logits(rng, T), normal_bias(rng),
                     off=RANGE * rank, cnt=RANGE)


def decode_sweep(T: int, rank: int) -> RouteCase:
    """Decode sweep: T tokens, rank range [112 r, 112 r + 112), exact twins.

    Every 4th row also moves one twin pair onto that row's 16th-largest logit,
    so the tie sits near the top-k boundary.
    """
    rng = np.random.default_rng(seed_for(2, T))
    logits = normal_logits(rng, T)
    bias = normal_bias(rng)
    for src, dst in TWIN_PAIRS:
        logits[:, dst] = logits[:, src]
        bias[dst] = bias[src]
    for t in range(0, T, 4):
        src, dst = TWIN_PAIRS[(t // 4) % len(TWIN_PAIRS)]
        v = np.sort(logits[t])[::-1][K - 1]
        logits[t, src] = v
        logits[t, dst] = v
    return RouteCase(f"decode_sweep_T{T}_r{rank}", logits, bias,
                     off=RANGE * rank, cnt=RANGE, meta={"rank": rank})


def router_case(T: int, e: int = E, h: int = H) -> RouteCase:
    """bf16 hidden [T, h] ~ N(0,1) and bf16 router weight [e, h] ~ N(0, 0.02)
    (by default the 896 x 7168 router)."""
    variant = 0 if (e, h) == (E, H) else 1 + e + h
    rng = np.random.default_rng(seed_for(3, T, variant))
    hidden = _to_bf16_bits(rng.standard_normal((T, h), dtype=np.float32))
    weight = _to_bf16_bits(np.float32(0.02) * rng.standard_normal((e, h), dtype=np.float32))
    bias = normal_bias(rng, e)
    name = f"router_T{T}" if variant == 0 else f"router_T{T}_E{e}_H{h}"
    return RouteCase(name, None, bias, hidden=hidden, weight=weight)


def zipf_bias(rng: np.random.Generator, e: int = E, alpha: float = ZIPF_ALPHA,
              s: float = ZIPF_S) -> np.ndarray:
    base = 0.01 * rng.standard_normal(e)
    ranks = rng.permutation(e) + 1
    return (base + alpha * ranks.astype(np.float64) ** (-s)).astype(np.float32)


def long_prefill(T: int = 32768, variant: int = 0, rank: int = 0) -> RouteCase:
    """Long prefill: T x 896 N(0,1) logits, Zipf-skewed bias, range [0, 112)."""
    rng = np.random.default_rng(seed_for(4, T, variant))
    logits = normal_logits(rng, T)
    bias = zipf_bias(rng)
    return RouteCase(f"long_prefill_T{T}_v{variant}", logits, bias,
                     off=RANGE * rank, cnt=RANGE)


def random_case(T: int, seed: int, e: int = E, off: int = 0, cnt: int = 0,
                n_groups: int = G, topk_group: int = TG, top_k: int = K,
                group_topn: int = TOPN, logit_scale: float = 1.0) -> RouteCase:
    """Generic seeded case for parity sweeps (edge shapes, other parameters)."""
    rng = np.random.default_rng(seed)
    logits = (np.float32(logit_scale) * normal_logits(rng, T, e)).astype(np.float32)
    return RouteCase(f"random_T{T}_s{seed}", logits, normal_bias(rng, e), off=off,
                     cnt=cnt, n_groups=n_groups, topk_group=topk_group,
                     top_k=top_k, group_topn=group_topn)
