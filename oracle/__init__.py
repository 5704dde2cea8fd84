"""CPU oracle for one decode / mixed step of a dense decoder-only transformer.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU
baseline are the only callers allowed to import anything here. The product
path (the HIP library and its Python binding) never imports, links or runs
this package, and this package imports nothing from the product.

What it computes is the plain, unfused, unpacked, eager transformer step, in
fp32 NumPy, one request at a time. The pages state that fusing the
projections, fusing the elementwise work, packing prefill and decode rows into
one forward, and replaying the step as a graph all leave the outputs unchanged
(Removing overhead: fusion, graphs and async scheduling, sections "Fewer,
larger matmuls" and "CUDA graphs for a changing batch"; One forward per step,
section "What changed"), so the unfused per-request step is the definition the
fast path must reproduce. Sampling is the Gumbel-max trick (Fast decode: syncs,
CUDA graphs and compilation, section "Sampling without the CPU").

Parity pins: every function is pinned by a test in tests/test_oracle_*.py
against closed forms, brute force or published known-answer vectors. The only
part with no outside pin is the whole-model logit value for random weights:
the pages print no logits, so whole-step logits are "parity unpinned" beyond
the invariants (incremental == full-sequence, MHA == duplicated-GQA, closed
form single-token layer, zero-layer closed form).
"""
from .model import (RequestCache, attend, final_logits, forward_request, linear, rmsnorm, rope,
                    rope_angles, silu_mul)
from .sampling import argmax_lowest, gumbel_scores, philox4x32_10, philox_uniforms, sample, topk_topp_keep
from .paging import bucket_for, pad_rows, slot_of

__all__ = ["RequestCache", "attend", "final_logits", "forward_request", "linear", "rmsnorm", "rope", "topk_topp_keep",
           "rope_angles", "silu_mul", "argmax_lowest", "gumbel_scores", "philox4x32_10", "philox_uniforms",
           "sample", "bucket_for", "pad_rows", "slot_of"]
