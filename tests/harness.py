"""Helpers shared by the GPU parity tests: build a Decoder, inject seeded KV histories into the paged
pools, and run the oracle on the same inputs, one request at a time."""
from __future__ import annotations

import sys
import time
from typing import List, Optional, Sequence

import numpy as np

import oracle
import synth
from conftest import oracle_weights

TOL = {"f32": 1e-4, "bf16": 3e-2, "f16": 3e-2}


def log(*a):
    print("[harness %.1fs]" % time.monotonic(), *a, flush=True)
    sys.stdout.flush()


def blocks_for(n: int) -> int:
    return -(-n // 16)


class Scenario:
    """A decode batch over injected KV histories (or empty histories)."""

    def __init__(self, shape, weights, contexts: Sequence[int], steps: int, seed: int, shuffled: bool = True,
                 extra_blocks: int = 4):
        self.shape = shape
        self.weights = weights
        self.contexts = [int(c) for c in contexts]
        self.steps = steps
        self.seed = seed
        need = [c + steps + 1 for c in self.contexts]
        self.num_blocks = sum(blocks_for(n) for n in need) + extra_blocks + 1
        self.tables = synth.block_tables(need, self.num_blocks, seed, shuffled)
        self.width = max(len(t) for t in self.tables)
        self.tokens = synth.tokens(len(self.contexts), shape.vocab, seed + 77)

    def kv(self, req: int, layer: int):
        return synth.injected_kv(self.shape, self.seed, req, layer, self.contexts[req])

    def inject(self, dec) -> None:
        """Write every request's seeded history into the GPU pools at its block-table slots."""
        torch = dec.torch
        for l in range(self.shape.layers):
            ks, vs, blk, off = [], [], [], []
            for j, c in enumerate(self.contexts):
                if c == 0:
                    continue
                k, v = self.kv(j, l)
                ks.append(k)
                vs.append(v)
                p = np.arange(c)
                blk.append(np.asarray(self.tables[j])[p // 16])
                off.append(p % 16)
            if not ks:
                continue
            bi = torch.as_tensor(np.concatenate(blk), device=dec.device, dtype=torch.long)
            oi = torch.as_tensor(np.concatenate(off), device=dec.device, dtype=torch.long)
            dec.k_pool[l][bi, :, oi, :] = torch.cat(ks).to(dec.device)
            dec.v_pool[l][bi, :, :, oi] = torch.cat(vs).to(dec.device)   # V is dim-major
        torch.cuda.synchronize(dec.device)

    def table_array(self, rows: Optional[Sequence[int]] = None) -> np.ndarray:
        rows = range(len(self.contexts)) if rows is None else rows
        out = np.full((len(rows), self.width), -1, np.int32)
        for i, j in enumerate(rows):
            out[i, :len(self.tables[j])] = self.tables[j]
        return out

    def step_inputs(self, tokens, positions):
        pos = np.asarray(positions, np.int32)
        slots = np.array([oracle.slot_of(self.tables[j], int(pos[j]), 16) for j in range(len(pos))], np.int32)
        return np.asarray(tokens, np.int32), pos, pos + 1, slots, self.table_array()

    def oracle_cache(self, req: int) -> oracle.RequestCache:
        cache = oracle.RequestCache(self.shape.layers)
        if self.contexts[req]:
            for l in range(self.shape.layers):
                k, v = self.kv(req, l)
                cache.set(l, k.float().numpy(), v.float().numpy())
        return cache


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def near_tie_ok(gpu_tok: int, ref_logits: np.ndarray, tol: float) -> bool:
    """Token agreement rule: a mismatch is tolerated only when the reference's top-2 margin is below 2 * tol."""
    top = np.sort(ref_logits)[-2:]
    ref_tok = int(oracle.argmax_lowest(ref_logits))
    return gpu_tok == ref_tok or (top[1] - top[0]) < 2 * tol


def fp32_weights(weights) -> dict:
    return oracle_weights(weights)
