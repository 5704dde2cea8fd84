"""Seeded synthetic inputs for the decode / mixed transformer step.

This module is shared by the tests, the benchmark and the smoke check. It holds
no arithmetic of the model: it only draws random numbers from fixed seeds and
rounds them once to the storage dtype, so that the CPU oracle and the HIP path
read the exact same bits.

Recipe (every draw uses ``numpy.random.default_rng`` with a tuple seed, so any
tensor can be regenerated on its own):

* Weights: every linear and embedding matrix is N(0, 0.02) drawn in fp32 and
  rounded once to the storage dtype with round-to-nearest-even. QKV bias is
  N(0, 0.02). RMSNorm gains are 1 + N(0, 0.02), so a dropped gain still shows.
  Weight seed 0.
* Token ids: integer-uniform over the vocabulary.
* Decode contexts: integer-uniform inclusive draws, or draws from a set of
  lengths plus an integer-uniform tail, per workload below.
* Block tables: a random permutation of block ids 0 .. num_blocks-2 handed out
  to requests in order; block num_blocks-1 is reserved as the scratch block.
* Injected KV history: N(0, 1) per (request, layer), rounded to the storage
  dtype, standing in for a prefill that is too slow to run on the host.
* Uniforms for sampling: fp32 uniform [0, 1) clamped below at 1e-10.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Shape:
    """Architecture of a dense decoder-only transformer with RMSNorm and SwiGLU."""
    name: str
    layers: int
    hidden: int
    q_heads: int
    kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    qk_norm: bool
    qkv_bias: bool
    tied: bool
    dtype: str
    eps: float = 1e-6
    theta: float = 1e6

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def qkv_out(self) -> int:
        return (self.q_heads + 2 * self.kv_heads) * self.head_dim

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The shapes the workloads are quoted on.
TINY = Shape("tiny", 2, 256, 4, 2, 64, 768, 1024, qk_norm=True, qkv_bias=False, tied=True, dtype="f32")
TINY_BIAS = TINY.replace(name="tiny-bias", qk_norm=False, qkv_bias=True)
QWEN3_0_6B = Shape("qwen3-0.6b", 28, 1024, 16, 8, 128, 3072, 151936, qk_norm=True, qkv_bias=False,
                   tied=True, dtype="bf16")
QWEN2_5_1_5B = Shape("qwen2.5-1.5b", 28, 1536, 12, 2, 128, 8960, 151936, qk_norm=False, qkv_bias=True,
                     tied=True, dtype="f16")

BLOCK_SIZE = 16
LAYER_TENSORS = ("in_norm", "wq", "wk", "wv", "bq", "bk", "bv", "q_norm", "k_norm", "wo", "post_norm",
                 "wg", "wu", "wd")


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Round an fp32 array once to the storage dtype (round-to-nearest-even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_TORCH_DTYPE[dtype])


def _normal(shape: Sequence[int], std: float, mean: float, *key: int) -> np.ndarray:
    x = _rng(*key).standard_normal(size=tuple(shape), dtype=np.float32)
    x *= np.float32(std)
    if mean:
        x += np.float32(mean)
    return x


def layer_tensor_shapes(s: Shape) -> Dict[str, Optional[tuple]]:
    d = s.head_dim
    return {
        "in_norm": (s.hidden,),
        "wq": (s.q_heads * d, s.hidden),
        "wk": (s.kv_heads * d, s.hidden),
        "wv": (s.kv_heads * d, s.hidden),
        "bq": (s.q_heads * d,) if s.qkv_bias else None,
        "bk": (s.kv_heads * d,) if s.qkv_bias else None,
        "bv": (s.kv_heads * d,) if s.qkv_bias else None,
        "q_norm": (d,) if s.qk_norm else None,
        "k_norm": (d,) if s.qk_norm else None,
        "wo": (s.hidden, s.q_heads * d),
        "post_norm": (s.hidden,),
        "wg": (s.intermediate, s.hidden),
        "wu": (s.intermediate, s.hidden),
        "wd": (s.hidden, s.intermediate),
    }


def make_layer_tensor(s: Shape, layer: int, name: str, seed: int = 0) -> Optional[torch.Tensor]:
    shp = layer_tensor_shapes(s)[name]
    if shp is None:
        return None
    key = (seed, 1 + layer, LAYER_TENSORS.index(name))
    gain = name.endswith("norm")
    x = _normal(shp, 0.02, 1.0 if gain else 0.0, *key)
    return to_storage(x, s.dtype)


def make_weights(s: Shape, seed: int = 0) -> dict:
    """All weights of one model as CPU tensors in the storage dtype.

    Layout: every matrix is row-major [out_features, in_features]. ``lm_head`` is
    the embedding itself when the shape ties them.
    """
    embed = to_storage(_normal((s.vocab, s.hidden), 0.02, 0.0, seed, 0, 0), s.dtype)
    final_norm = to_storage(_normal((s.hidden,), 0.02, 1.0, seed, 0, 1), s.dtype)
    lm_head = embed if s.tied else to_storage(_normal((s.vocab, s.hidden), 0.02, 0.0, seed, 0, 2), s.dtype)
    layers = [{n: make_layer_tensor(s, l, n, seed) for n in LAYER_TENSORS} for l in range(s.layers)]
    return {"embed": embed, "final_norm": final_norm, "lm_head": lm_head, "layers": layers}


def tokens(n: int, vocab: int, seed: int) -> np.ndarray:
    return _rng(seed, 7).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def block_tables(lengths: Sequence[int], num_blocks: int, seed: int, shuffled: bool = True,
                 block_size: int = BLOCK_SIZE) -> List[List[int]]:
    """Hand out ceil(len/block_size) blocks per request from a (shuffled) free list.

    Block ``num_blocks - 1`` is the scratch block and never appears in a table.
    """
    ids = np.arange(num_blocks - 1, dtype=np.int64)
    if shuffled:
        ids = _rng(seed, 11).permutation(ids)
    out, at = [], 0
    for n in lengths:
        k = -(-int(n) // block_size)
        if at + k > len(ids):
            raise ValueError("pool too small for the requested lengths")
        out.append([int(b) for b in ids[at:at + k]])
        at += k
    return out


def injected_kv(s: Shape, seed: int, request: int, layer: int, n: int):
    """Seeded KV history of one request at one layer: (K, V), each [n, kv_heads, head_dim], storage dtype."""
    x = _normal((2, n, s.kv_heads, s.head_dim), 1.0, 0.0, seed, 101, request, layer)
    t = to_storage(x, s.dtype)
    return t[0], t[1]


def uniforms(rows: int, cols: int, seed: int, step: int = 0) -> np.ndarray:
    """fp32 uniforms in [1e-10, 1) for explicit-uniform sampling."""
    u = _rng(seed, 13, step).random(size=(rows, cols), dtype=np.float32)
    return np.maximum(u, np.float32(1e-10))


# ----------------------------------------------------------------------------------------------
# The five workloads. Each returns plain integers / arrays; no model arithmetic.

@dataclasses.dataclass
class DecodeWorkload:
    name: str
    shape: Shape
    contexts: List[int]            # keys already in the cache per request (before the first step)
    steps: int                     # decode steps
    temperature: float
    shuffled: bool
    buckets: List[int]
    prompt: Optional[np.ndarray] = None   # real prefill prompt (batch 1), else KV is injected
    input_seed: int = 0


def workload_tiny() -> DecodeWorkload:
    return DecodeWorkload("tiny-f32-bs1", TINY, [64], 16, 0.0, False, [1], tokens(64, TINY.vocab, 1001), 1001)


def workload_q3_bs1() -> DecodeWorkload:
    return DecodeWorkload("qwen3-0.6b-bf16-bs1-ctx1024", QWEN3_0_6B, [1024], 256, 0.0, False, [1],
                          tokens(1024, QWEN3_0_6B.vocab, 1002), 1002)


def workload_q3_bs32() -> DecodeWorkload:
    ctx = _rng(1003, 3).integers(128, 2048, size=32, endpoint=True).tolist()
    return DecodeWorkload("qwen3-0.6b-bf16-bs32-ctx128-2048", QWEN3_0_6B, [int(c) for c in ctx], 256, 1.0,
                          True, [1, 2, 4, 8, 16, 32], None, 1003)


def workload_q3_bs256() -> DecodeWorkload:
    r = _rng(1005, 3)
    base = r.choice(np.array([16, 64, 256, 1024, 4096]), size=256)
    extra = r.integers(64, 256, size=256, endpoint=True)
    ctx = (base + extra).tolist()
    return DecodeWorkload("qwen3-0.6b-bf16-bs256", QWEN3_0_6B, [int(c) for c in ctx], 256, 0.7, True,
                          [1, 2, 4, 8, 16, 32, 64, 128, 256], None, 1005)


@dataclasses.dataclass
class MixedWorkload:
    name: str
    shape: Shape
    prefill_lens: List[int]        # new prompt tokens per prefill request (fresh prompts unless prefix given)
    prefill_prefix: List[int]      # tokens already cached before the chunk, per prefill request
    decode_contexts: List[int]     # cached keys per decode request
    input_seed: int


def workload_q25_mixed() -> MixedWorkload:
    ctx = _rng(1004, 3).choice(np.array([16, 64, 256, 1024, 4096]), size=32).tolist()
    return MixedWorkload("qwen2.5-1.5b-f16-mixed-512+32", QWEN2_5_1_5B, [16, 240, 256], [0, 0, 0],
                         [int(c) for c in ctx], 1004)


def num_params(s: Shape) -> int:
    """Parameter count (tied embeddings counted once)."""
    per_layer = sum(math.prod(v) for v in layer_tensor_shapes(s).values() if v is not None)
    emb = s.vocab * s.hidden * (1 if s.tied else 2)
    return s.layers * per_layer + emb + s.hidden
