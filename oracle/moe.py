"""CPU oracle for a mixture-of-experts MLP layer served without host reads.

TEST INFRASTRUCTURE ONLY, under the same rule as the rest of this package: only the
tests, the smoke check and the benchmark's CPU baseline may import it, and it imports
nothing from the product.

Source: "Removing overhead: fusion, graphs and async scheduling", section "A MoE layer
that never asks the host". The layer takes, per token t, k expert ids e[t, j] and router
weights w[t, j], and returns

    out[t] = sum_j w[t, j] * down[e[t, j]] @ (silu(g) * u),   [g; u] = gate_up[e[t, j]] @ x[t]

with gate_up [E, 2I, D] (the first I rows are the gate, the last I the up projection, as
the page's SiLU-and-mul splits its input) and down [E, D, I]. That per-token sum is the
definition written here (`moe_layer`). The page computes it by grouping the N * k
assignments by expert, each group padded to a multiple of BLOCK_M rows, and running one
grouped GEMM per projection; `moe_align` is that grouping, written as its plain definition
(each expert's assignments in assignment order, then padding), and `moe_grouped` runs the
layer through the grouping exactly as the page's two grouped GEMMs read and write rows, so
that the tests can show that the grouped route equals the definition.

Readings (where the page leaves a step open):
* Expert ids outside [0, E) belong to no group: they get no row and contribute nothing.
  The page's scatter-add count would index out of bounds on them.
* Arithmetic is fp64 here; the page keeps the grouped GEMM's output rows in the input
  dtype. The HIP path keeps them in fp32 and rounds the activation to the input dtype.

Parity pins (tests/test_oracle_moe.py): a worked grouping example derived by hand from the
page's definition (tests/golden/moe_align_example.txt), a second grouping written as scalar
counting loops over the assignments (counts, group starts, running rank per expert), the
grouping invariants, brute-force scalar loops on tiny layers, the dense SwiGLU MLP that one
expert with weight 1 reduces to, linearity in the router weights, and invariance under a
relabelling of the experts and under a reordering of a token's k slots.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def align_rows(total: int, num_experts: int, block_m: int) -> int:
    """Rows of the grouped layout in the worst case: every expert's group padded by up to
    block_m - 1 rows, rounded up to whole blocks."""
    m = total + num_experts * (block_m - 1)
    return -(-m // block_m) * block_m


def moe_align(expert_ids: np.ndarray, num_experts: int, block_m: int):
    """Group the assignments (flat index token * k + slot) by expert.

    Returns (sorted_ids [m_max], block_expert [m_max // block_m], num_padded). Expert e's
    group holds its assignments in increasing index order, followed by padding rows up to a
    multiple of block_m; groups follow one another in expert order from row 0. Padding rows
    and the rows past num_padded hold `total` (one past the last assignment). Block b belongs
    to the expert whose group holds row b * block_m; blocks past num_padded say E - 1.
    """
    flat = np.asarray(expert_ids).reshape(-1).astype(np.int64)
    total = flat.size
    m_max = align_rows(total, num_experts, block_m)
    sorted_ids = np.full(m_max, total, np.int64)
    block_expert = np.full(m_max // block_m, num_experts - 1, np.int64)
    row = 0
    for e in range(num_experts):
        members = np.nonzero(flat == e)[0]          # ascending assignment order
        sorted_ids[row:row + members.size] = members
        padded = -(-members.size // block_m) * block_m
        block_expert[row // block_m:(row + padded) // block_m] = e
        row += padded
    return sorted_ids, block_expert, row


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u = g / (1 + exp(-g)) * u."""
    g = np.asarray(g, F64)
    return g / (1.0 + np.exp(-g)) * np.asarray(u, F64)


def expert_mlp(x: np.ndarray, gate_up: np.ndarray, down: np.ndarray) -> np.ndarray:
    """One expert's SwiGLU MLP on the rows of x [n, D]: down @ (silu(g) * u)."""
    inter = gate_up.shape[0] // 2
    h = np.asarray(x, F64) @ np.asarray(gate_up, F64).T
    return silu_mul(h[:, :inter], h[:, inter:]) @ np.asarray(down, F64).T


def moe_layer(x, gate_up, down, weights, expert_ids) -> np.ndarray:
    """The definition: out[t] = sum_j w[t, j] * expert_mlp(x[t]) of expert e[t, j]
    (ids outside [0, E) skipped). x [N, D], gate_up [E, 2I, D], down [E, D, I],
    weights / expert_ids [N, k]."""
    x = np.asarray(x, F64)
    n, k = np.asarray(expert_ids).shape
    E = gate_up.shape[0]
    out = np.zeros((n, down.shape[1]), F64)
    for t in range(n):
        for j in range(k):
            e = int(expert_ids[t, j])
            if 0 <= e < E:
                out[t] += F64(weights[t, j]) * expert_mlp(x[t:t + 1], gate_up[e], down[e])[0]
    return out


def moe_grouped(x, gate_up, down, weights, expert_ids, block_m: int = 16) -> np.ndarray:
    """The layer as the page's grouped route computes it: group with moe_align; for each block
    of block_m rows, gather the rows of its assignments (token rows for the first GEMM, the
    assignment rows for the second), multiply by the block's expert, mask padding rows, scale
    the second GEMM's rows by their router weight, and add each token's k rows."""
    x = np.asarray(x, F64)
    n, k = np.asarray(expert_ids).shape
    total = n * k
    E, two_i, _ = gate_up.shape
    inter = two_i // 2
    sorted_ids, block_expert, num_padded = moe_align(expert_ids, E, block_m)
    flat_w = np.asarray(weights, F64).reshape(-1)
    act = np.zeros((total, inter), F64)
    rows = np.zeros((total, down.shape[1]), F64)
    for b in range(num_padded // block_m):
        ids = sorted_ids[b * block_m:(b + 1) * block_m]
        live = ids[ids < total]
        e = int(block_expert[b])
        h = x[live // k] @ np.asarray(gate_up[e], F64).T
        act[live] = silu_mul(h[:, :inter], h[:, inter:])
    for b in range(num_padded // block_m):
        ids = sorted_ids[b * block_m:(b + 1) * block_m]
        live = ids[ids < total]
        e = int(block_expert[b])
        rows[live] = (act[live] @ np.asarray(down[e], F64).T) * flat_w[live][:, None]
    return rows.reshape(n, k, -1).sum(axis=1)
