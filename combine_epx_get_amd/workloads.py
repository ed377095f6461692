"""Seeded synthetic workloads for MoE expert-parallel dispatch/combine.

This module only draws inputs: token activations, router top-k choices and
gate weights. It holds none of the dispatch/combine arithmetic, so the CPU
oracle and the GPU path can both consume what it produces without sharing
any of the method's code.

Shapes follow the workloads of "Balancing and Beyond: Communication-Centric
Optimizations in Expert Parallelism" (research digest, section 5: DeepSeek-R1
with 256 experts, top-8, hidden 7168; decode with at most 128 tokens on a GPU,
section 1) and of "Poor HybridEP performance on dual-node 16x B300 GPUs"
(4096 tokens per rank, hidden 7168, top-8). The production routing traces of
the digest (section 2, Figure 2) are not available; uniform and Zipf-skewed
routing stand in for them.

Recipe (numpy ``Generator(PCG64(seed))``), drawn in this order:
  1. x ~ N(0, 1) as float32 [T, h]; for the outlier workload, a fixed set of
     round(0.01 h) channel ids (drawn without replacement, sorted) is scaled
     by 50 in float32. x is then rounded to bf16 (round to nearest even).
  2. Zipf workloads only: a random permutation of expert ids; popularity of
     expert perm[i-1] is proportional to i**(-s), i = 1..E.
  3. Routing keys: Gumbel-top-k. Uniform routing uses keys U(0,1) (equal
     logits); Zipf routing uses log p_e + Gumbel(0,1), which samples k
     distinct experts sequentially in proportion to remaining popularity.
     topk_idx[t, :] lists the k largest keys in descending key order, the
     order a router's top-k emits.
  4. Gate logits ~ N(0, 1) [T, k]; weights = softmax over the k chosen,
     computed in float64 and cast to float32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    topk: int
    num_ranks: int
    num_hosts: int
    routing: str            # "uniform" or "zipf"
    zipf_s: float = 0.0
    outlier_frac: float = 0.0   # fraction of channels scaled by outlier_scale
    outlier_scale: float = 50.0
    modes: tuple = ("per_expert",)
    dtypes: tuple = ("bf16",)
    seed: int = 1
    my_rank: int = 0

    @property
    def experts_per_rank(self) -> int:
        return self.num_experts // self.num_ranks

    @property
    def ranks_per_host(self) -> int:
        return self.num_ranks // self.num_hosts


# The five workloads: a tiny parity case, two decode shapes (uniform and
# skewed), the 4096-token large batch and the fp8 outlier batch. A Zipf(0.6)
# decode variant gives imbalance ratios inside the digest's measured range.
# The rank_* shapes are the source ranks of the DeepEP rank-imbalance issue
# (2 machines x 8 ranks): 384 tokens per rank on machine 1 and 64 on machine
# 2, against 224 everywhere when balanced. hybridep_bf16 is the HybridEP
# issue's benchmark shape with per-rank de-duplication.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 64, 256, 16, 2, 4, 2, "uniform",
                     modes=("per_expert", "relay"), dtypes=("bf16", "fp8"), seed=1),
    "decode_uniform": Workload("decode_uniform", 128, 7168, 256, 8, 32, 4, "uniform",
                               modes=("per_expert",), seed=2),
    "decode_skewed": Workload("decode_skewed", 128, 7168, 256, 8, 32, 4, "zipf", zipf_s=1.2,
                              modes=("per_expert", "relay"), seed=3),
    "decode_skewed_s06": Workload("decode_skewed_s06", 128, 7168, 256, 8, 32, 4, "zipf",
                                  zipf_s=0.6, modes=("per_expert", "relay"), seed=3),
    "large_batch": Workload("large_batch", 4096, 7168, 256, 8, 16, 2, "uniform",
                            modes=("per_expert",), seed=4),
    "fp8_dispatch": Workload("fp8_dispatch", 4096, 7168, 256, 8, 32, 4, "zipf", zipf_s=1.0,
                             outlier_frac=0.01, modes=("relay",), dtypes=("fp8",), seed=5),
    "rank_heavy": Workload("rank_heavy", 384, 7168, 256, 8, 16, 2, "uniform",
                           modes=("per_expert", "relay"), seed=6, my_rank=3),
    "rank_light": Workload("rank_light", 64, 7168, 256, 8, 16, 2, "uniform",
                           modes=("per_expert", "relay"), seed=7, my_rank=11),
    "rank_balanced": Workload("rank_balanced", 224, 7168, 256, 8, 16, 2, "uniform",
                              modes=("per_expert", "relay"), seed=8, my_rank=11),
    # the HybridEP benchmark's shape (4096 tokens per rank, hidden 7168,
    # top-8, 8 local experts on each of 16 ranks) with one copy per
    # destination rank: relay mode with every rank its own host
    "hybridep_bf16": Workload("hybridep_bf16", 4096, 7168, 128, 8, 16, 16, "uniform",
                              modes=("relay",), seed=9),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) with torch's CPU cast;
    return the raw 16-bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _topk_desc(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, in descending key order."""
    part = np.argpartition(-keys, k - 1, axis=1)[:, :k]
    pk = np.take_along_axis(keys, part, axis=1)
    order = np.argsort(-pk, axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1).astype(np.int32)


def draw_routing(rng: np.random.Generator, T: int, E: int, k: int, routing: str,
                 zipf_s: float = 0.0) -> np.ndarray:
    """Draw topk_idx [T, k] int32 of k distinct experts per token."""
    if routing == "uniform":
        keys = rng.random((T, E))
    elif routing == "zipf":
        perm = rng.permutation(E)
        logp = np.empty(E, dtype=np.float64)
        logp[perm] = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        keys = logp[None, :] + rng.gumbel(size=(T, E))
    else:
        raise ValueError(f"unknown routing {routing!r}")
    return _topk_desc(keys, k)


def draw_gate_weights(rng: np.random.Generator, T: int, k: int) -> np.ndarray:
    logits = rng.standard_normal((T, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None, num_tokens: Optional[int] = None) -> dict:
    """Draw (x_bf16_bits [T,h] uint16, topk_idx [T,k] int32, topk_weights [T,k] f32).

    ``num_tokens`` overrides T (used for ragged and scaled-down cases)."""
    seed = w.seed if seed is None else seed
    T = w.num_tokens if num_tokens is None else num_tokens
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((T, w.hidden), dtype=np.float32)
    outliers = np.zeros(0, dtype=np.int64)
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * w.hidden))
        outliers = np.sort(rng.choice(w.hidden, size=n_out, replace=False))
        x[:, outliers] *= np.float32(w.outlier_scale)
    x_bits = f32_to_bf16_bits(x)
    idx = draw_routing(rng, T, w.num_experts, w.topk, w.routing, w.zipf_s)
    wts = draw_gate_weights(rng, T, w.topk)
    return {"x": x_bits, "topk_idx": idx, "topk_weights": wts, "outlier_channels": outliers,
            "T": T, "seed": seed}


def random_bf16(shape, seed: int) -> np.ndarray:
    """N(0,1) values rounded to bf16, as uint16 bit patterns (used for
    stand-in expert outputs where their values do not matter)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
