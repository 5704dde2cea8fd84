"""Integer bookkeeping of the paged KV pool and of bucketed graphs (test infrastructure only).

* Slot of a token: the block table row maps block index pos // block_size to a
  pool block; the slot is block * block_size + pos % block_size. Padding rows
  carry slot -1, which the kernel sends to a scratch block that no table
  holds (Removing overhead, section "CUDA graphs for a changing batch").
* Bucket: the smallest captured batch size >= the step's row count; rows past
  the step's count are padding (the same section's 13 -> 16 example).
* Padding row values: token 0, position 0, slot -1, length 0, zero
  block-table row (GraphRunner.run in that section).
"""
from __future__ import annotations

from typing import Sequence


def slot_of(block_row: Sequence[int], pos: int, block_size: int) -> int:
    return int(block_row[pos // block_size]) * block_size + pos % block_size


def bucket_for(rows: int, buckets: Sequence[int]) -> int:
    for b in sorted(buckets):
        if b >= rows:
            return int(b)
    raise ValueError("row count above the largest bucket")


def pad_rows(rows: int, bucket: int, width: int):
    """Values the padding rows rows .. bucket-1 carry: (token, position, slot, seq_len, block_row)."""
    return [(0, 0, -1, 0, [0] * width) for _ in range(rows, bucket)]
