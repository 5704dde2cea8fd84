"""Seeded synthetic inputs for the mixture-of-experts layer.

Like the rest of this package it only draws random numbers from fixed seeds and rounds
them once to the storage dtype; it holds none of the layer's arithmetic.

Recipe:

* Shape: the expert layer of Qwen3-30B-A3B, the model whose 128 experts the pages name
  ("Removing overhead: fusion, graphs and async scheduling", section "A MoE layer that
  never asks the host"): 128 experts, 8 per token, hidden 2048, expert width 768 (that
  model's published configuration; the pages give only the expert count).
* Token rows x: N(0, 1), the scale of a normed hidden state, rounded to the dtype.
* Expert weights: gate|up [E, 2I, D] and down [E, D, I], N(0, 0.02) per expert from seed
  (seed, expert, 1 or 2), rounded to the dtype, so one expert can be drawn on its own.
* Routing: each token takes k distinct experts, drawn without replacement with weights
  proportional to (rank + 1) ** -0.8 over a seeded ranking of the experts, so a few
  experts are hot and, in a small batch, some get no token at all.
* Router weights: uniform [0.05, 1) per slot, scaled to sum to 1 per token, fp32.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import _TORCH_DTYPE, _normal, _rng, to_storage


@dataclasses.dataclass(frozen=True)
class MoeShape:
    name: str
    experts: int
    top_k: int
    hidden: int
    inter: int
    dtype: str = "bf16"

    def replace(self, **kw) -> "MoeShape":
        return dataclasses.replace(self, **kw)


QWEN3_30B_A3B_MOE = MoeShape("qwen3-30b-a3b-moe", 128, 8, 2048, 768)
TINY_MOE = MoeShape("tiny-moe", 8, 2, 256, 128)


def expert_weights(s: MoeShape, e: int, seed: int = 0):
    """(gate_up [2I, D], down [D, I]) of expert e in the storage dtype."""
    gu = to_storage(_normal((2 * s.inter, s.hidden), 0.02, 0.0, seed, e, 1), s.dtype)
    dn = to_storage(_normal((s.hidden, s.inter), 0.02, 0.0, seed, e, 2), s.dtype)
    return gu, dn


def make_moe_weights(s: MoeShape, seed: int = 0):
    """(gate_up [E, 2I, D], down [E, D, I]) stacked, storage dtype, on the CPU."""
    gu = torch.empty((s.experts, 2 * s.inter, s.hidden), dtype=_TORCH_DTYPE[s.dtype])
    dn = torch.empty((s.experts, s.hidden, s.inter), dtype=_TORCH_DTYPE[s.dtype])
    for e in range(s.experts):
        gu[e], dn[e] = expert_weights(s, e, seed)
    return gu, dn


def token_rows(s: MoeShape, n: int, seed: int) -> torch.Tensor:
    return to_storage(_normal((n, s.hidden), 1.0, 0.0, seed, 11), s.dtype)


def routing(s: MoeShape, n: int, seed: int):
    """(expert_ids [n, k] int32, weights [n, k] fp32)."""
    rng = _rng(seed, 12)
    rank_of = rng.permutation(s.experts)
    p = (rank_of + 1.0) ** -0.8
    p /= p.sum()
    ids = np.empty((n, s.top_k), np.int32)
    for t in range(n):
        ids[t] = rng.choice(s.experts, size=s.top_k, replace=False, p=p)
    w = rng.uniform(0.05, 1.0, size=(n, s.top_k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True, dtype=np.float32)
    return ids, w.astype(np.float32)
