"""fp32 transformer step, one request at a time (test infrastructure only).

Follows the layer as the pages list its operations for Qwen3-0.6B (Fast decode:
syncs, CUDA graphs and compilation, section "Where the time goes"): RMSNorm,
the Q, K and V projections, the two per-head QK-norms, RoPE on Q and K, the
cache write, attention, the output projection and residual add, RMSNorm, the
gate and up projections, SiLU times up, the down projection and residual add.
The projections are three separate matmuls here, the unfused form that the
fused [W_Q | W_K | W_V] matmul must equal (Removing overhead, section "Fewer,
larger matmuls", the stacked-projection equation).

Readings where the pages are silent (each also listed in the design doc):
* RoPE is the rotate-half form with inverse frequencies theta^(-2i/d); the
  angle tables are computed in fp64 and rounded to fp32.
* QK-norm is an RMSNorm over each head's d values with one gain vector [d]
  per projection, applied before RoPE.
* Attention scale is 1/sqrt(d); query head h reads KV head h // (nq / nkv);
  softmax in fp32 with the max subtracted.
* The new token's K and V are written before the token attends, so a decode
  row sees seq_len = cached + 1 keys; keys at positions > the query's are
  hidden (the causal rule key_pos <= query_pos of Fast decode, section
  "Static shapes and a static cache").
* The residual stream and every intermediate are fp32.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

F32 = np.float32


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """y[..., i] = sum_k x[..., k] * w[i, k] (+ b[i]); w is row-major [out, in]."""
    y = np.matmul(x.astype(F32, copy=False), w.astype(F32, copy=False).T)
    if b is not None:
        y = y + b.astype(F32, copy=False)
    return y.astype(F32, copy=False)


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis, in fp32."""
    x = x.astype(F32, copy=False)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return (x / np.sqrt(ms + F32(eps)) * w.astype(F32, copy=False)).astype(F32, copy=False)


def rope_angles(positions: Sequence[int], head_dim: int, theta: float):
    """cos, sin tables [n, d/2] for absolute positions: angle = pos * theta^(-2i/d), fp64 then fp32."""
    half = head_dim // 2
    inv = np.power(np.float64(theta), -2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def rope(x: np.ndarray, positions: Sequence[int], theta: float) -> np.ndarray:
    """Rotate-half RoPE on x [n, heads, d] at the given absolute positions."""
    d = x.shape[-1]
    half = d // 2
    cos, sin = rope_angles(positions, d, theta)
    cos, sin = cos[:, None, :], sin[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1).astype(F32)


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """silu(g) * u = g / (1 + exp(-g)) * u, in fp32."""
    g = g.astype(F32, copy=False)
    return (g / (F32(1.0) + np.exp(-g)) * u.astype(F32, copy=False)).astype(F32)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: Sequence[int]) -> np.ndarray:
    """Causal attention of one request.

    q [n, nq, d] at absolute positions q_pos; k, v [L, nkv, d] hold the request's keys at
    positions 0 .. L-1. Query head h reads KV head h // (nq // nkv). A key is visible when
    its position <= the query's. A query that sees no key returns zeros.
    """
    n, nq, d = q.shape
    L, nkv, _ = k.shape
    group = nq // nkv
    out = np.zeros((n, nq, d), dtype=F32)
    scale = F32(1.0 / np.sqrt(d))
    kf, vf = k.astype(F32, copy=False), v.astype(F32, copy=False)
    for i in range(n):
        visible = min(int(q_pos[i]) + 1, L)
        if visible <= 0:
            continue
        for h in range(nq):
            g = h // group
            s = (kf[:visible, g, :] @ q[i, h, :].astype(F32)) * scale
            p = np.exp(s - np.max(s))
            p = p / np.sum(p, dtype=F32)
            out[i, h, :] = p.astype(F32) @ vf[:visible, g, :]
    return out


class RequestCache:
    """Contiguous per-layer K, V history of one request (positions 0 .. length-1)."""

    def __init__(self, layers: int):
        self.k: List[Optional[np.ndarray]] = [None] * layers
        self.v: List[Optional[np.ndarray]] = [None] * layers

    @property
    def length(self) -> int:
        return 0 if self.k[0] is None else int(self.k[0].shape[0])

    def set(self, layer: int, k: np.ndarray, v: np.ndarray) -> None:
        self.k[layer] = np.ascontiguousarray(k, dtype=F32)
        self.v[layer] = np.ascontiguousarray(v, dtype=F32)

    def write(self, layer: int, k_new: np.ndarray, v_new: np.ndarray, positions: Sequence[int]) -> None:
        """Store K, V of new tokens at their absolute positions (growing the history as needed)."""
        need = int(max(positions)) + 1
        k, v = self.k[layer], self.v[layer]
        if k is None:
            k = np.zeros((0,) + k_new.shape[1:], F32)
            v = np.zeros((0,) + v_new.shape[1:], F32)
        if need > k.shape[0]:
            pad = need - k.shape[0]
            k = np.concatenate([k, np.zeros((pad,) + k.shape[1:], F32)])
            v = np.concatenate([v, np.zeros((pad,) + v.shape[1:], F32)])
        k[np.asarray(positions)] = k_new
        v[np.asarray(positions)] = v_new
        self.k[layer], self.v[layer] = k, v


def forward_request(shape, weights: dict, cache: RequestCache, tokens: Sequence[int],
                    positions: Sequence[int]) -> np.ndarray:
    """Run new tokens of ONE request through every layer; return the final-normed hidden [n, H].

    ``weights`` holds fp32 arrays: embed [V,H], final_norm [H], layers[l][name] with the names
    in_norm, wq, wk, wv, bq, bk, bv, q_norm, k_norm, wo, post_norm, wg, wu, wd (None where the
    shape has no such tensor). The tokens are appended to ``cache`` (written before attending).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    nq, nkv, d, eps = shape.q_heads, shape.kv_heads, shape.head_dim, shape.eps
    r = weights["embed"][tokens].astype(F32)
    for l, w in enumerate(weights["layers"]):
        h = rmsnorm(r, w["in_norm"], eps)
        q = linear(h, w["wq"], w.get("bq")).reshape(n, nq, d)
        k = linear(h, w["wk"], w.get("bk")).reshape(n, nkv, d)
        v = linear(h, w["wv"], w.get("bv")).reshape(n, nkv, d)
        if shape.qk_norm:
            q = rmsnorm(q, w["q_norm"], eps)
            k = rmsnorm(k, w["k_norm"], eps)
        q = rope(q, positions, shape.theta)
        k = rope(k, positions, shape.theta)
        cache.write(l, k, v, positions)
        o = attend(q, cache.k[l], cache.v[l], positions)
        r = r + linear(o.reshape(n, nq * d), w["wo"])
        h2 = rmsnorm(r, w["post_norm"], eps)
        a = silu_mul(linear(h2, w["wg"]), linear(h2, w["wu"]))
        r = r + linear(a, w["wd"])
    return rmsnorm(r, weights["final_norm"], eps)


def final_logits(weights: dict, hidden: np.ndarray) -> np.ndarray:
    """logits = hidden @ lm_head^T in fp32 (lm_head is the embedding when tied)."""
    return linear(hidden, weights["lm_head"])
