"""The C-ABI library loads on the host and exports every symbol include/step.h declares (no GPU calls)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "step.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(step_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary_calls():
    names = _declared()
    for n in ("step_init", "step_decode", "step_mixed", "step_sample", "step_workspace_bytes", "step_destroy",
              "step_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import graph_replay_amd._lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libstep.so not built")
    lib = C.CDLL(L.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(L.EXPORTS)


def test_workspace_size_is_host_only_and_validates():
    import graph_replay_amd as g
    import graph_replay_amd._lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libstep.so not built")
    cfg = L.StepConfig(dtype=L.STEP_BF16, layers=2, hidden=1024, q_heads=16, kv_heads=8, head_dim=128,
                       intermediate=3072, vocab=151936, qk_norm=1, qkv_bias=0, rms_eps=1e-6, rope_theta=1e6,
                       block_size=16, num_blocks=100, max_blocks_per_seq=80, max_position=1280, max_batch=32,
                       max_tokens=0, max_reqs=0, max_logit_rows=0, num_buckets=2, use_graphs=1)
    cfg.buckets[0], cfg.buckets[1] = 16, 32
    assert g.step_workspace_bytes(cfg) > 0
    cfg.head_dim = 96
    assert g.step_workspace_bytes(cfg) == 0           # unsupported head_dim
    cfg.head_dim = 128
    cfg.buckets[1] = 31                               # last bucket must equal max_batch
    assert g.step_workspace_bytes(cfg) == 0


def test_binding_fails_loudly_without_the_library(tmp_path):
    import graph_replay_amd._lib as L
    with pytest.raises(RuntimeError):
        L._lib = None
        L.load(str(tmp_path / "missing.so"))
    L._lib = None


def test_persistent_decode_config_is_validated():
    """persistent_decode is accepted only at the widths its kernel is built for, with bucket 1,
    max_position <= 64 keys x 256 blocks / 8 KV heads = 2048 and 2048 <= vocab <= 262144 (every one of
    the 2048 LM-head waves owns 1 to 128 rows); the workspace grows by its hand-off words."""
    import graph_replay_amd as g
    import graph_replay_amd._lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libstep.so not built")

    def cfg(**kw):
        c = L.StepConfig(dtype=L.STEP_BF16, layers=28, hidden=1024, q_heads=16, kv_heads=8, head_dim=128,
                         intermediate=3072, vocab=151936, qk_norm=1, qkv_bias=0, rms_eps=1e-6, rope_theta=1e6,
                         block_size=16, num_blocks=100, max_blocks_per_seq=80, max_position=1280, max_batch=1,
                         max_tokens=0, max_reqs=0, max_logit_rows=0, num_buckets=1, use_graphs=1)
        c.buckets[0] = 1
        for k, v in kw.items():
            setattr(c, k, v)
        return c

    base = g.step_workspace_bytes(cfg())
    assert base > 0
    with_p = g.step_workspace_bytes(cfg(persistent_decode=1))
    assert with_p > base
    assert g.step_workspace_bytes(cfg(persistent_decode=1, dtype=L.STEP_F16)) > 0
    for bad in (dict(dtype=L.STEP_F32), dict(hidden=1536), dict(intermediate=8960), dict(kv_heads=4),
                dict(max_position=2049), dict(vocab=2047), dict(vocab=262145), dict(persistent_decode=2)):
        kw = dict(persistent_decode=1)
        kw.update(bad)
        assert g.step_workspace_bytes(cfg(**kw)) == 0, bad
    for good in (dict(max_position=2048), dict(vocab=2048), dict(vocab=262144)):
        assert g.step_workspace_bytes(cfg(persistent_decode=1, **good)) > 0, good
    c = cfg(persistent_decode=1, max_batch=2, num_buckets=1)
    c.buckets[0] = 2
    assert g.step_workspace_bytes(c) == 0            # bucket 1 is what the persistent step serves
