"""The C-ABI library loads on the host and exports every symbol include/*.h declares (no GPU calls)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("step.h", "moe.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b((?:step|moe)_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary_calls():
    names = _declared()
    for n in ("step_init", "step_decode", "step_mixed", "step_sample", "step_workspace_bytes", "step_destroy",
              "step_last_error"):
        assert n in names
    for n in ("moe_align", "moe_align_rows", "moe_forward", "moe_workspace_bytes", "moe_last_error"):
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
    max_position <= 128 keys x 256 blocks / 8 KV heads = 4096 (64-key items up to 2048) and
    2048 <= vocab <= 262144 (every one of the 2048 LM-head waves owns 1 to 128 rows); the workspace
    grows by its hand-off words."""
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
                dict(max_position=4097), dict(vocab=2047), dict(vocab=262145), dict(persistent_decode=2)):
        kw = dict(persistent_decode=1)
        kw.update(bad)
        assert g.step_workspace_bytes(cfg(**kw)) == 0, bad
    for good in (dict(max_position=2048), dict(max_position=2049, max_blocks_per_seq=257),
                 dict(max_position=4096, max_blocks_per_seq=256), dict(vocab=2048), dict(vocab=262144)):
        assert g.step_workspace_bytes(cfg(persistent_decode=1, **good)) > 0, good
    # the 128-key items halve the split count: the partials of 4,096 positions take what 2,048 did
    w2k = g.step_workspace_bytes(cfg(persistent_decode=1, max_position=2048))
    w4k = g.step_workspace_bytes(cfg(persistent_decode=1, max_position=4096, max_blocks_per_seq=256))
    assert w4k - w2k == g.step_workspace_bytes(cfg(max_position=4096, max_blocks_per_seq=256)) - \
        g.step_workspace_bytes(cfg(max_position=2048))
    c = cfg(persistent_decode=1, max_batch=2, num_buckets=1)
    c.buckets[0] = 2
    assert g.step_workspace_bytes(c) == 0            # bucket 1 is what the persistent step serves


def test_moe_sizes_are_host_only_and_validate():
    """moe_align_rows and moe_workspace_bytes run on the host; bad sizes give -1 / 0, and the
    worst-case row count is total + E * (block_m - 1) rounded up to block_m."""
    import graph_replay_amd._lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libstep.so not built")
    lib = L.load()
    assert lib.moe_align_rows(6, 4, 4) == 20
    assert lib.moe_align_rows(256, 128, 16) == 2176
    assert lib.moe_align_rows(0, 1, 1) == 0
    for bad in ((-1, 4, 4), (6, 0, 4), (6, 1025, 4), (6, 4, 0), (2**31 - 8, 1024, 16)):
        assert lib.moe_align_rows(*bad) == -1, bad

    def layer(**kw):
        m = L.MoeLayer(dtype=L.STEP_BF16, n_tokens=32, top_k=8, num_experts=128, hidden=2048, inter=768)
        for k, v in kw.items():
            setattr(m, k, v)
        return m

    ws = lib.moe_workspace_bytes(C.byref(layer()))
    total = 32 * 8
    assert ws >= 2176 * 4 + 136 * 4 + 4 + total * 768 * 2 + total * 2048 * 4
    for bad in (dict(dtype=L.STEP_F32), dict(n_tokens=-1), dict(top_k=0), dict(num_experts=0),
                dict(num_experts=1025), dict(hidden=2047), dict(inter=700), dict(hidden=0)):
        assert lib.moe_workspace_bytes(C.byref(layer(**bad))) == 0, bad
    assert lib.moe_forward(C.byref(layer(dtype=L.STEP_F32)), None, 0, None) == L.STEP_EUNSUPPORTED
    assert b"dtype" in lib.moe_last_error()
    assert lib.moe_forward(C.byref(layer(inter=700)), None, 0, None) == L.STEP_EINVAL


def _q3_cfg(L, max_position, max_batch=8, max_tokens=0):
    cfg = L.StepConfig(dtype=L.STEP_BF16, layers=2, hidden=1024, q_heads=16, kv_heads=8, head_dim=128,
                       intermediate=3072, vocab=151936, qk_norm=1, qkv_bias=0, rms_eps=1e-6, rope_theta=1e6,
                       block_size=16, num_blocks=100, max_blocks_per_seq=(max_position + 15) // 16,
                       max_position=max_position, max_batch=max_batch, max_tokens=max_tokens,
                       max_reqs=max(max_batch, 1) if max_tokens else 0, max_logit_rows=max_batch if max_tokens else 0,
                       num_buckets=1, use_graphs=1)
    cfg.buckets[0] = max_batch
    return cfg


@pytest.mark.parametrize("max_position,max_batch,max_tokens,dtype,bal", [
    (9000, 8, 32, "bf16", 0), (9000, 8, 0, "bf16", 0), (20000, 64, 600, "bf16", 0), (2304, 32, 0, "bf16", 0),
    (2304, 32, 0, "bf16", 9), (8192, 1, 0, "bf16", 0), (16384, 256, 0, "bf16", 0), (4096, 1100, 1500, "bf16", 0),
    (4096, 300, 0, "bf16", 40), (4096, 300, 0, "bf16", 2000), (9000, 8, 600, "f32", 0), (2304, 64, 0, "f32", 9)])
def test_attention_partials_hold_every_launch(max_position, max_batch, max_tokens, dtype, bal):
    """For every row count and key bound a launch can use, its partial slots fit the workspace's. On
    the split grid the split count is not monotone in the key bound (the split length doubles past
    128 splits), so the sweep covers every key bound, not just max_position; the balanced kernel's
    demand is fixed by the row count alone."""
    import graph_replay_amd as g
    import graph_replay_amd._lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libstep.so not built")
    cfg = _q3_cfg(L, max_position, max_batch, max_tokens)
    cfg.dtype = L.STEP_BF16 if dtype == "bf16" else L.STEP_F32
    cfg.balanced_attention_rows = bal
    tm = max(max_batch, max_tokens)
    G = cfg.q_heads // cfg.kv_heads
    flat_extra = -(-2048 * G // cfg.q_heads)   # one slot of G heads per wave of the balanced launch
    _, cap = g.step_attention_slots(cfg, 1, 1)
    assert cap > 0
    rows_set = {1, 2, 7, 8, 9, 32, 39, 40, 63, 64, 65, 127, 128, 1023, 1024, 1025, tm} & set(range(1, tm + 1))
    for rows in sorted(rows_set):
        flat = dtype == "bf16" and (bal or 128) <= rows <= 1024
        for max_len in list(range(1, max_position + 1, 7 if max_position > 10000 else 3)) + [max_position]:
            n, c = g.step_attention_slots(cfg, rows, max_len)
            assert c == cap and rows <= n <= cap, (rows, max_len, n, cap)
            if flat:   # the balanced kernel's demand, or the split grid's where that is larger
                assert n == rows + flat_extra or (n > rows + flat_extra and n % rows == 0)
            else:
                assert n % rows == 0 and 1 <= n // rows <= 128
    # the case that once overflowed: 8 rows at 8,192 keys under a 9,000-position bound use 128 splits
    if max_position == 9000:
        assert g.step_attention_slots(cfg, 8, 8192)[0] == 8 * 128 <= cap
    assert g.step_attention_slots(cfg, tm + 1, 16)[0] == L.STEP_EINVAL
    assert g.step_attention_slots(cfg, 1, max_position + 1)[0] == L.STEP_EINVAL
    cfg.balanced_attention_rows = 8   # the split grid keeps 8 rows and fewer
    assert g.step_attention_slots(cfg, 1, 1)[0] == L.STEP_EINVAL


def test_split_lengths_leave_no_short_last_split():
    """The split grid's split count for a key bound (seen through the partial-slot demand, rows x
    splits, with the balanced kernel off): from 256-key splits up the length is spread over the
    splits the bound needs, so a bound just past a multiple of the nominal length (2,048 keys for up
    to 64 rows whose bound stays within 2,560, else 512) takes no extra split for its last few keys,
    the average split never falls below the nominal length, and no bound takes more splits than
    the nominal length would give it."""
    import graph_replay_amd as g
    import graph_replay_amd._lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libstep.so not built")
    cfg = _q3_cfg(L, 9000, 128, 0)
    cfg.balanced_attention_rows = 2000   # the split grid at every row count
    # the mixed step's decode rows at a 4,097-key bound: 8 splits, not 9 with one key in the last
    assert g.step_attention_slots(cfg, 32, 4097)[0] == 32 * 8
    # up to 64 rows at 2,049 keys: one split of 2,064 keys, not a second one holding one key
    assert g.step_attention_slots(cfg, 32, 2049)[0] == 32
    for rows in (9, 32, 64, 65, 128):
        for max_len in range(1, 9001, 13):
            n = g.step_attention_slots(cfg, rows, max_len)[0]
            assert n > 0 and n % rows == 0, (rows, max_len, n)
            splits = n // rows
            nominal = 2048 if rows <= 64 and max_len <= 2560 else 512
            assert splits <= -(-max_len // nominal), (rows, max_len, splits)
            assert splits == 1 or max_len / splits >= nominal, (rows, max_len, splits)
            assert splits == max(1, max_len // nominal), (rows, max_len, splits)
