"""Greedy and Gumbel-max sampling, and the Philox-4x32-10 uniforms (test infrastructure only).

Sampling follows Fast decode: syncs, CUDA graphs and compilation, section
"Sampling without the CPU": temperature 0 is argmax; otherwise uniforms are
clamped to [1e-10, 1], g = -log(-log u), and the sample is argmax(z / T + g),
all in fp32. That argmax is an exact draw from softmax(z / T) (the section's
Gumbel-max equation).

Reading: ties in the argmax go to the lowest index.

Top-k and top-p filtering follow the same section (the passage after the sampler listing): the
filters run before the argmax and set the filtered logits to -inf; top-k uses a fixed k, and top-p is
a sort and a mask. Readings of this build, where the passage does not fix the details:
  * both filters act only when T > 0, on z = logit / T computed in fp32 (the device's value), so
    every comparison that decides the kept set is the same fp32 comparison on both sides;
  * top-k keeps every z >= the k-th largest z (ties at the threshold are kept); k <= 0 or k >= V
    disables it;
  * top-p acts after top-k, on the softmax of the kept z: in the order (z descending, index
    ascending), a token is kept iff the mass strictly before it is < p (the shortest prefix whose
    mass reaches p); p >= 1 disables it.

The uniforms, where they are not passed in, come from Philox-4x32-10 as
defined by Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
1, 2, 3" (SC'11): ten rounds of two 32x32->64-bit multiplies with the
multipliers 0xD2511F53 and 0xCD9E8D57, and a Weyl key schedule with the
increments 0x9E3779B9 and 0xBB67AE85. Word mapping (a reading of this build):
key = (seed low, seed high); counter = (column // 4, row, step low, step high);
output word j belongs to column 4 * (column // 4) + j; u = (word >> 8) * 2^-24.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def argmax_lowest(x: np.ndarray) -> np.ndarray:
    """Index of the maximum along the last axis; the lowest index wins a tie."""
    return np.argmax(x, axis=-1)   # numpy returns the first occurrence


def gumbel_scores(z: np.ndarray, temperature: float, u: np.ndarray) -> np.ndarray:
    """z / T - log(-log(clamp(u, 1e-10, 1))), fp32."""
    u = np.clip(u.astype(F32), F32(1e-10), F32(1.0))
    g = -np.log(-np.log(u))
    return (z.astype(F32) / F32(temperature) + g).astype(F32)


def sample(z: np.ndarray, temperature: float, u: np.ndarray = None, top_k: int = 0,
           top_p: float = 1.0) -> np.ndarray:
    """Token ids [rows] from logits [rows, V]: greedy at T == 0, Gumbel-max otherwise, over the
    tokens that top-k / top-p keep (filtered scores are -inf)."""
    if temperature == 0:
        return argmax_lowest(z)
    sc = gumbel_scores(z, temperature, u)
    if (0 < top_k < z.shape[-1]) or top_p < 1.0:
        zs = np.atleast_2d(z.astype(F32) / F32(temperature))
        keep = np.stack([topk_topp_keep(r, top_k, top_p) for r in zs]).reshape(sc.shape)
        sc = np.where(keep, sc, F32(-np.inf)).astype(F32)
    return argmax_lowest(sc)


def topk_topp_keep(z32: np.ndarray, top_k: int, top_p: float) -> np.ndarray:
    """Kept-token mask [V] of one row of fp32 z = logit / T (see the module docstring)."""
    z32 = np.asarray(z32, dtype=F32)
    V = z32.shape[0]
    keep = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        kth = np.sort(z32)[::-1][top_k - 1]
        keep = z32 >= kth
    if top_p < 1.0:
        z = z32.astype(np.float64)
        w = np.where(keep, np.exp(z - z[keep].max()), 0.0)
        mass = w / w.sum()
        order = np.lexsort((np.arange(V), -z))          # z descending, then index ascending
        order = order[keep[order]]
        before = np.cumsum(mass[order]) - mass[order]
        kept = np.zeros(V, dtype=bool)
        kept[order] = before < top_p
        keep = kept
    return keep


def _mulhilo(a: np.ndarray, b: int):
    p = a.astype(np.uint64) * np.uint64(b)
    return (p >> np.uint64(32)).astype(np.uint64), (p & np.uint64(_MASK)).astype(np.uint64)


def philox4x32_10(counter, key):
    """Philox-4x32 with 10 rounds. counter: 4 arrays (or ints) of uint32, key: 2. Returns 4 uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(_MASK) for x in counter]
    k0 = np.asarray(key[0], dtype=np.uint64) & np.uint64(_MASK)
    k1 = np.asarray(key[1], dtype=np.uint64) & np.uint64(_MASK)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(_W0)) & np.uint64(_MASK)
            k1 = (k1 + np.uint64(_W1)) & np.uint64(_MASK)
        hi0, lo0 = _mulhilo(c[0], _M0)
        hi1, lo1 = _mulhilo(c[2], _M1)
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return [x.astype(np.uint32) for x in c]


def philox_uniforms(seed: int, step: int, rows: int, cols: int) -> np.ndarray:
    """Uniforms [rows, cols] in [1e-10, 1) for sampling step ``step`` (see the module docstring)."""
    groups = -(-cols // 4)
    g = np.arange(groups, dtype=np.uint64)[None, :].repeat(rows, 0)
    r = np.arange(rows, dtype=np.uint64)[:, None].repeat(groups, 1)
    lo = np.full_like(g, step & _MASK)
    hi = np.full_like(g, (step >> 32) & _MASK)
    words = philox4x32_10([g, r, lo, hi], [seed & _MASK, (seed >> 32) & _MASK])
    w = np.stack(words, axis=-1).reshape(rows, groups * 4)[:, :cols]
    u = (w >> np.uint32(8)).astype(F32) * F32(2.0 ** -24)
    return np.maximum(u, F32(1e-10))
