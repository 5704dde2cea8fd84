"""GPU parity of the whole step against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from harness import TOL, Scenario, fp32_weights, log, max_abs, near_tie_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _decoder(shape, weights, **kw):
    import graph_replay_amd as g
    return g.Decoder(shape, weights, **kw)


@pytest.mark.parametrize("shape", [synth.TINY, synth.TINY_BIAS], ids=["qk_norm", "qkv_bias"])
def test_tiny_f32_prefill_then_greedy_decode(torch_cuda, shape):
    """64-token prompt through step_mixed, then 16 greedy graph replays continuing on the device."""
    torch = torch_cuda
    log("tiny f32", shape.name)
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    prompt = synth.tokens(64, shape.vocab, 1001)
    steps = 16
    table = synth.block_tables([64 + steps + 1], 16, 1001, shuffled=True)[0]
    dec = _decoder(shape, W, num_blocks=16, max_blocks_per_seq=8, max_position=128, max_batch=1, buckets=[1],
                   max_tokens=64, max_reqs=1, max_logit_rows=1, history=True)
    bt = np.full((1, 8), -1, np.int32)
    bt[0, :len(table)] = table
    pos = np.arange(64, dtype=np.int32)
    slots = np.array([oracle.slot_of(table, int(p), 16) for p in pos], np.int32)
    dec.mixed([0, 64], [64], prompt, pos, slots, bt, [63], num_prefill_reqs=1)
    torch.cuda.synchronize()
    cache = oracle.RequestCache(shape.layers)
    hid = oracle.forward_request(shape, W32, cache, prompt, list(range(64)))
    ref = oracle.final_logits(W32, hid[-1:])[0]
    got = dec.logits[0].cpu().numpy()
    assert max_abs(got, ref) <= TOL["f32"], max_abs(got, ref)
    tok = int(dec.tokens[0].item())
    assert near_tie_ok(tok, ref, TOL["f32"])
    toks = [tok]
    for i in range(steps):
        p = 64 + i
        if i == 0:
            dec.decode([tok], [p], [p + 1], [oracle.slot_of(table, p, 16)], bt)
        else:
            dec.decode_continue()
        torch.cuda.synchronize()
        got = dec.logits[0].cpu().numpy()
        hid = oracle.forward_request(shape, W32, cache, [toks[-1]], [p])
        ref = oracle.final_logits(W32, hid)[0]
        assert max_abs(got, ref) <= TOL["f32"], (i, max_abs(got, ref))
        tok = int(dec.tokens[0].item())
        assert near_tie_ok(tok, ref, TOL["f32"]), i
        toks.append(tok)
    hist = dec.history[0, 64:64 + steps].cpu().numpy().tolist()
    assert hist == toks[1:]
    dec.close()


@pytest.mark.parametrize("balanced", [0, 9])
def test_decode_all_bucket_paths_bf16(torch_cuda, balanced):
    """bf16 decode at row counts that hit every matmul path (VALU <= 8, MFMA 16/32, tiled 64) and pad;
    with balanced = 9 the attention of 9 rows and more runs on the balanced kernel."""
    torch = torch_cuda
    shape = synth.TINY.replace(name="tiny-bf16", dtype="bf16")
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    rng = np.random.default_rng(5)
    contexts = rng.integers(1, 200, size=64).tolist()
    sc = Scenario(shape, W, contexts, steps=2, seed=2024)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=256, max_batch=64,
                   buckets=[1, 2, 4, 8, 16, 32, 64], use_graphs=True, balanced_attention_rows=balanced)
    sc.inject(dec)
    for r in (1, 3, 8, 13, 32, 50, 64):
        log("bf16 tiny rows", r)
        toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
        dec.decode(toks[:r], pos[:r], lens[:r], slots[:r], bt[:r])
        torch.cuda.synchronize()
        got = dec.logits[:r].cpu().numpy()
        for j in range(r):
            hid = oracle.forward_request(shape, W32, sc.oracle_cache(j), [toks[j]], [pos[j]])
            ref = oracle.final_logits(W32, hid)[0]
            assert max_abs(got[j], ref) <= TOL["bf16"], (r, j, max_abs(got[j], ref))
        assert dec.last_bucket() == min(b for b in [1, 2, 4, 8, 16, 32, 64] if b >= r)
    dec.close()


def test_lm_head_ragged_vocab_9_to_32_rows(torch_cuda):
    """The streaming LM-head GEMV (9-32 rows) with a vocabulary that is not a multiple of its 16-row
    tiles: the last tile's rows past the vocabulary are loaded clamped and never stored."""
    torch = torch_cuda
    shape = synth.TINY.replace(name="tiny-bf16-v1000", dtype="bf16", vocab=1000)
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    rng = np.random.default_rng(6)
    contexts = rng.integers(1, 120, size=32).tolist()
    sc = Scenario(shape, W, contexts, steps=2, seed=2025)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=256, max_batch=32,
                   buckets=[16, 32], use_graphs=True)
    sc.inject(dec)
    for r in (13, 32):
        log("bf16 tiny vocab 1000 rows", r)
        toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
        dec.logits.fill_(float("nan"))
        dec.decode(toks[:r], pos[:r], lens[:r], slots[:r], bt[:r])
        torch.cuda.synchronize()
        got = dec.logits[:r].cpu().numpy()
        assert got.shape[1] == 1000
        for j in range(r):
            hid = oracle.forward_request(shape, W32, sc.oracle_cache(j), [toks[j]], [pos[j]])
            ref = oracle.final_logits(W32, hid)[0]
            assert max_abs(got[j], ref) <= TOL["bf16"], (r, j, max_abs(got[j], ref))
    dec.close()


@pytest.mark.parametrize("balanced", [0, 9])
def test_qwen3_width_two_layers_bs32_gumbel(torch_cuda, balanced):
    """Qwen3-0.6B widths (2 layers) at batch 32 over shuffled paged KV, Gumbel-max at T = 1 with Philox;
    the attention on the split grid (balanced = 0) and on the balanced kernel (balanced = 9)."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2)
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    ctx = np.random.default_rng(1003).integers(128, 2048, size=32, endpoint=True).tolist()
    sc = Scenario(shape, W, ctx, steps=2, seed=1003)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=2304, max_batch=32,
                   buckets=[1, 2, 4, 8, 16, 32], balanced_attention_rows=balanced)
    sc.inject(dec)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    seed = 0x1234_5678_9ABC
    dec.decode(toks, pos, lens, slots, bt, temperature=np.ones(32, np.float32), seed=seed)
    torch.cuda.synchronize()
    got = dec.logits[:32].cpu().numpy()
    gtok = dec.tokens[:32].cpu().numpy()
    u = oracle.philox_uniforms(seed, 0, 32, shape.vocab)
    mism = 0
    for j in range(32):
        hid = oracle.forward_request(shape, W32, sc.oracle_cache(j), [toks[j]], [pos[j]])
        ref = oracle.final_logits(W32, hid)[0]
        err = max_abs(got[j], ref)
        assert err <= TOL["bf16"], (j, err)
        # kernel exactness: the GPU's token is the Gumbel argmax over its own logits with the same uniforms
        s = oracle.gumbel_scores(got[j], 1.0, u[j])
        top = np.sort(s)[-2:]
        if int(np.argmax(s)) != int(gtok[j]):
            assert top[1] - top[0] < 1e-5 * max(1.0, abs(top[1])), j
            mism += 1
        # oracle agreement under the near-tie rule
        sref = oracle.gumbel_scores(ref, 1.0, u[j])
        assert near_tie_ok(int(gtok[j]), sref, TOL["bf16"]), j
    assert mism <= 1
    dec.close()


@pytest.mark.parametrize("bal", [9, 0])
def test_balanced_attention_long_short_and_padding_rows(torch_cuda, bal):
    """The balanced attention kernel (balanced_attention_rows = 9) on a batch that stresses its share
    arithmetic: one 8,001-key row spread over ~60 waves (a merge of that many pieces), rows of 1 to
    18 keys (pieces of one or two tiles, tile edges), a 3,001-key row, and six padding rows of the
    16-row bucket. Every real row's logits against the oracle. With bal = 0 the same batch runs on
    the split grid (16 rows), where the long row takes 15 splits and the blocks take the live
    pieces in packed order past a row without keys and the padding rows."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2, vocab=4096)
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    contexts = [8000, 0, 1, 15, 16, 17, 3000, 5, 100, 63]
    sc = Scenario(shape, W, contexts, steps=2, seed=3301)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=8016,
                   max_batch=16, buckets=[16], balanced_attention_rows=bal)
    sc.inject(dec)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    dec.decode(toks, pos, lens, slots, bt)
    torch.cuda.synchronize()
    assert dec.last_bucket() == 16
    got = dec.logits[:len(contexts)].cpu().numpy()
    assert np.all(np.isfinite(dec.logits[:16].cpu().numpy()))
    for j, c in enumerate(contexts):
        log("balanced attention row", j, "context", c)
        hid = oracle.forward_request(shape, W32, sc.oracle_cache(j), [toks[j]], [pos[j]])
        ref = oracle.final_logits(W32, hid)[0]
        assert max_abs(got[j], ref) <= TOL["bf16"], (j, c, max_abs(got[j], ref))
    dec.close()


def test_balanced_attention_qwen25_fp16_six_heads_per_kv(torch_cuda):
    """The balanced attention kernel's fp16, six-query-heads-per-KV-head instance (Qwen2.5-1.5B widths:
    12 query heads over 2 KV heads, QKV bias, no QK-norm), 2 layers, 13 rows padded to 16, against
    the oracle and against the split grid on the same state."""
    torch = torch_cuda
    shape = synth.QWEN2_5_1_5B.replace(layers=2, vocab=4096, dtype="f16")
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    contexts = np.random.default_rng(3402).integers(1, 1500, size=13).tolist()
    sc = Scenario(shape, W, contexts, steps=2, seed=3402)
    kw = dict(num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=1536, max_batch=16, buckets=[16])
    db = _decoder(shape, W, balanced_attention_rows=9, **kw)
    ds = _decoder(shape, W, **kw)
    sc.inject(db)
    sc.inject(ds)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    for dec in (db, ds):
        dec.decode(toks, pos, lens, slots, bt)
    torch.cuda.synchronize()
    gb = db.logits[:13].cpu().numpy()
    gs = ds.logits[:13].cpu().numpy()
    assert max_abs(gb, gs) <= TOL["f16"], max_abs(gb, gs)
    for j in range(13):
        hid = oracle.forward_request(shape, W32, sc.oracle_cache(j), [toks[j]], [pos[j]])
        ref = oracle.final_logits(W32, hid)[0]
        assert max_abs(gb[j], ref) <= TOL["f16"], (j, max_abs(gb[j], ref))
    db.close()
    ds.close()


def test_split_grid_packed_pieces_past_256_rows(torch_cuda):
    """The split grid over 260 rows (balanced kernel off), where each thread of the block's piece
    count takes two rows: contexts of 0 to 1,100 keys under a 1,152-position bound (at most two
    576-key splits per row; rows of 576 and 577 keys on either side of the split edge, and a row
    without keys), against the balanced kernel on the same state for every row and against the
    oracle for a sample of rows."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2, vocab=4096)
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    contexts = np.random.default_rng(3501).integers(0, 1101, size=260).tolist()
    contexts[5], contexts[200], contexts[257], contexts[258], contexts[259] = 0, 1100, 574, 575, 576
    sc = Scenario(shape, W, contexts, steps=1, seed=3501)
    kw = dict(num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=1152, max_batch=260,
              buckets=[260])
    ds = _decoder(shape, W, balanced_attention_rows=2000, **kw)
    db = _decoder(shape, W, **kw)
    sc.inject(ds)
    sc.inject(db)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    for dec in (ds, db):
        dec.decode(toks, pos, lens, slots, bt)
    torch.cuda.synchronize()
    gs = ds.logits[:260].cpu().numpy()
    gb = db.logits[:260].cpu().numpy()
    assert np.all(np.isfinite(gs))
    assert max_abs(gs, gb) <= TOL["bf16"], max_abs(gs, gb)
    for j in (0, 5, 100, 200, 257, 258, 259):
        log("split grid row", j, "context", contexts[j])
        hid = oracle.forward_request(shape, W32, sc.oracle_cache(j), [toks[j]], [pos[j]])
        ref = oracle.final_logits(W32, hid)[0]
        assert max_abs(gs[j], ref) <= TOL["bf16"], (j, contexts[j], max_abs(gs[j], ref))
    ds.close()
    db.close()
