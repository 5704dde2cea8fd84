"""GPU parity at the full scope of the workloads: the batch-32 workload at full depth over eight
device-continued graph replays (teacher-forced oracle, Gumbel-max with the same Philox uniforms), a
prefill chunk that continues a request over its cached prefix inside the mixed step, and the
integer invariant of the paged cache: a step changes no pool byte outside the slots it writes and
the scratch block."""
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


def test_bs32_full_depth_gumbel_eight_device_continued_replays(torch_cuda):
    """Qwen3-0.6B bf16, all 28 layers, 32 rows with contexts U[128, 2048] over a shuffled block table,
    Gumbel-max at T = 1 with Philox uniforms: one host-fed step, then seven graph replays that
    continue on the device. At every step and every row the logits are within 3e-2 of the oracle
    teacher-forced on the GPU's own tokens; every token is the Gumbel argmax over the GPU's own logits
    with the step's uniforms (kernel exactness) and the oracle's Gumbel-max token under the near-tie
    rule (oracle agreement).

    Each row's context is the KV the model itself writes for random tokens: all rows take prefixes
    of one random prompt (of the longest context), which the GPU prefills into every row's own
    blocks and the oracle prefills once (a row's keys below position c depend on the tokens below c
    only). Seeded N(0, 1) histories are not used at this depth: with them the bf16 rounding of the
    matmul inputs alone moves the fp32 step's logits by 0.06-0.09 at 28 layers (on real KV: 0.01)."""
    torch = torch_cuda
    wl = synth.workload_q3_bs32()
    shape = wl.shape
    steps = 8
    W = synth.make_weights(shape, 0)
    ctx = wl.contexts
    n_max = max(ctx)
    prompt = synth.tokens(n_max, shape.vocab, wl.input_seed + 7)
    sc = Scenario(shape, W, ctx, steps=steps, seed=wl.input_seed, shuffled=True)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width,
                   max_position=n_max + steps + 16, max_batch=32, buckets=wl.buckets, max_tokens=n_max,
                   max_reqs=1, max_logit_rows=1)
    bt = sc.table_array()
    log("bs32 full depth: prefilling", len(ctx), "contexts on the GPU")
    for j, c in enumerate(ctx):
        dec.mixed([0, c], [c], prompt[:c], list(range(c)), _slots(sc.tables[j], range(c)), bt[j:j + 1], [c - 1],
                  num_prefill_reqs=1)
    torch.cuda.synchronize()
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    seed = 0x5EED_1003
    temp = np.ones(32, np.float32)
    logits, tokens = [], []
    for i in range(steps):
        if i == 0:
            dec.decode(toks, pos, lens, slots, bt, temperature=temp, seed=seed)
        else:
            dec.decode_continue()
        torch.cuda.synchronize()
        logits.append(dec.logits[:32].cpu().numpy().copy())
        tokens.append(dec.tokens[:32].cpu().numpy().copy())
    assert dec.last_bucket() == 32
    dec.close()
    del dec
    W32 = fp32_weights(W)
    log("bs32 full depth: oracle prefill of", n_max, "tokens")
    full = oracle.RequestCache(shape.layers)
    oracle.forward_request(shape, W32, full, prompt, list(range(n_max)))
    mism = 0
    for j in range(32):
        cache = oracle.RequestCache(shape.layers)
        for l in range(shape.layers):
            cache.set(l, full.k[l][:ctx[j]], full.v[l][:ctx[j]])
        inputs = [int(toks[j])] + [int(tokens[i][j]) for i in range(steps - 1)]
        positions = list(range(int(pos[j]), int(pos[j]) + steps))
        hid = oracle.forward_request(shape, W32, cache, inputs, positions)
        ref = oracle.final_logits(W32, hid)
        for i in range(steps):
            err = max_abs(logits[i][j], ref[i])
            assert err <= TOL["bf16"], (j, i, err)
            # every step moves the Philox step counter on by one, the 32 prefill steps included
            u = oracle.philox_uniforms(seed, len(ctx) + i, 32, shape.vocab)[j]
            s = oracle.gumbel_scores(logits[i][j], 1.0, u)
            top = np.sort(s)[-2:]
            if int(np.argmax(s)) != int(tokens[i][j]):
                assert top[1] - top[0] < 1e-5 * max(1.0, abs(top[1])), (j, i)
                mism += 1
            assert near_tie_ok(int(tokens[i][j]), oracle.gumbel_scores(ref[i], 1.0, u), TOL["bf16"]), (j, i)
        if j % 8 == 7:
            log("bs32 full depth: oracle rows up to", j)
    assert mism <= 2, mism


def _slots(table, positions):
    return [oracle.slot_of(table, int(p), 16) for p in positions]


def test_continuation_chunk_over_cached_prefix(torch_cuda):
    """Qwen2.5-1.5B shape fp16 at full depth: the 240-token request of the mixed workload continues a
    256-token prompt prefilled by an earlier step (its chunk holds positions 256..495 and attends to
    the cached prefix), packed with two fresh prompts (16 and 256 tokens) and the 32 decode rows. The
    packed prefill kernel == per-row attention == the oracle, on every sampled row."""
    torch = torch_cuda
    wl = synth.workload_q25_mixed()
    shape = wl.shape
    W = synth.make_weights(shape, 0)
    seed = wl.input_seed + 50
    fresh = [16, 256]
    prefix, cont = 256, 240
    prompts = [synth.tokens(n, shape.vocab, seed + j) for j, n in enumerate([fresh[0], prefix + cont, fresh[1]])]
    dctx = wl.decode_contexts
    need = [fresh[0] + 1, prefix + cont + 1, fresh[1] + 1] + [c + 1 for c in dctx]
    num_blocks = sum(-(-n // 16) for n in need) + 2
    tables = synth.block_tables(need, num_blocks, seed, shuffled=True)
    width = max(len(t) for t in tables)
    bt = np.full((len(tables), width), -1, np.int32)
    for j, t in enumerate(tables):
        bt[j, :len(t)] = t
    sc = Scenario(shape, None, [0, 0, 0] + dctx, steps=0, seed=seed)
    sc.tables, sc.width = tables, width
    dec_tok = synth.tokens(len(dctx), shape.vocab, seed + 99)
    n_tok = sum(fresh) + cont + len(dctx)
    nreq = 3 + len(dctx)
    out = {}
    for mode in (0, 1):
        dec = _decoder(shape, W, num_blocks=num_blocks, max_blocks_per_seq=width, max_position=max(dctx) + 512,
                       max_batch=1, buckets=[1], max_tokens=n_tok, max_reqs=nreq, max_logit_rows=nreq,
                       use_graphs=False)
        sc.inject(dec)
        # step 1: the prefix alone, as a one-request prefill
        log("continuation: prefix prefill, mode", mode)
        dec.mixed([0, prefix], [prefix], prompts[1][:prefix], list(range(prefix)),
                  _slots(tables[1], range(prefix)), bt[1:2], [prefix - 1], num_prefill_reqs=1,
                  prefill_attention=mode)
        torch.cuda.synchronize()
        first = dec.logits[0].cpu().numpy().copy()
        # step 2: fresh 16, the continuation 240, fresh 256, then the decode rows
        toks, poss, sl, qsl, lens, lidx = [], [], [], [0], [], []
        chunks = [(0, range(fresh[0])), (1, range(prefix, prefix + cont)), (2, range(fresh[1]))]
        for j, rng_ in chunks:
            p = list(rng_)
            toks += [int(prompts[j][q]) for q in p]
            poss += p
            sl += _slots(tables[j], p)
            qsl.append(qsl[-1] + len(p))
            lens.append(p[-1] + 1)
            lidx.append(qsl[-1] - 1)
        for i, c in enumerate(dctx):
            toks.append(int(dec_tok[i])); poss.append(c); sl += _slots(tables[3 + i], [c])
            qsl.append(qsl[-1] + 1); lens.append(c + 1); lidx.append(qsl[-1] - 1)
        log("continuation: packed step, mode", mode)
        dec.mixed(qsl, lens, toks, poss, sl, bt, lidx, num_prefill_reqs=3, prefill_attention=mode)
        torch.cuda.synchronize()
        out[mode] = (first, dec.logits[:nreq].cpu().numpy().copy(), dec.tokens[:nreq].cpu().numpy().copy())
        dec.close()
    assert max_abs(out[0][1], out[1][1]) <= TOL["f16"], max_abs(out[0][1], out[1][1])
    W32 = fp32_weights(W)
    log("continuation: oracle")
    refs = []
    cache = oracle.RequestCache(shape.layers)
    hid = oracle.forward_request(shape, W32, cache, prompts[1][:prefix], list(range(prefix)))
    ref_first = oracle.final_logits(W32, hid[-1:])[0]
    assert max_abs(out[0][0], ref_first) <= TOL["f16"], max_abs(out[0][0], ref_first)
    c0 = oracle.RequestCache(shape.layers)
    refs.append(oracle.final_logits(W32, oracle.forward_request(shape, W32, c0, prompts[0], list(range(fresh[0])))[-1:])[0])
    hid = oracle.forward_request(shape, W32, cache, prompts[1][prefix:prefix + cont], list(range(prefix, prefix + cont)))
    refs.append(oracle.final_logits(W32, hid[-1:])[0])
    c2 = oracle.RequestCache(shape.layers)
    refs.append(oracle.final_logits(W32, oracle.forward_request(shape, W32, c2, prompts[2], list(range(fresh[1])))[-1:])[0])
    for i, c in enumerate(dctx):
        hid = oracle.forward_request(shape, W32, sc.oracle_cache(3 + i), [int(dec_tok[i])], [c])
        refs.append(oracle.final_logits(W32, hid)[0])
    for r, ref in enumerate(refs):
        assert max_abs(out[0][1][r], ref) <= TOL["f16"], (r, max_abs(out[0][1][r], ref))
        assert near_tie_ok(int(out[0][2][r]), ref, TOL["f16"]), r


def _pool_bits(dec):
    torch = dec.torch
    return [(k.view(torch.int16).clone(), v.view(torch.int16).clone()) for k, v in zip(dec.k_pool, dec.v_pool)]


def _check_only_slots_changed(dec, before, written, num_blocks):
    """Every pool element outside the written (block, offset) slots and the scratch block keeps its
    bits; every written slot changed (the pools start as random bits, the new keys are fresh)."""
    torch = dec.torch
    for l, (kb, vb) in enumerate(before):
        ka, va = dec.k_pool[l].view(torch.int16), dec.v_pool[l].view(torch.int16)
        dk = (ka != kb).any(dim=3).any(dim=1)          # [num_blocks, 16] changed K slots
        dv = (va != vb).any(dim=2).any(dim=1)          # [num_blocks, 16] changed V slots
        allowed = torch.zeros_like(dk)
        for slot in written:
            allowed[slot // 16, slot % 16] = True
        allowed[num_blocks - 1, :] = True                # the scratch block
        assert not bool((dk & ~allowed).any().item()), (l, "K", torch.nonzero(dk & ~allowed)[:4].tolist())
        assert not bool((dv & ~allowed).any().item()), (l, "V", torch.nonzero(dv & ~allowed)[:4].tolist())
        for slot in written:
            assert bool(dk[slot // 16, slot % 16].item()) and bool(dv[slot // 16, slot % 16].item()), (l, slot)


def _randomise(dec, seed):
    torch = dec.torch
    gen = torch.Generator(device=dec.device)
    gen.manual_seed(seed)
    for l in range(len(dec.k_pool)):
        dec.k_pool[l].normal_(generator=gen)
        dec.v_pool[l].normal_(generator=gen)
    torch.cuda.synchronize()


@pytest.mark.parametrize("persistent,balanced", [(False, 0), (True, 0), (False, 9)])
def test_decode_changes_only_its_slots_and_the_scratch_block(torch_cuda, persistent, balanced):
    """A host-fed decode step padded to its bucket (13 rows -> 16; the persistent step at 1 row) and
    two device-continued steps after it leave every pool byte bit-unchanged except the slots of the
    rows' new tokens and the scratch block, which padding rows write (balanced = 9: the attention
    of the 16-row bucket, which writes the new keys, on the balanced kernel)."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2, vocab=4096)
    W = synth.make_weights(shape, 0)
    rows = 1 if persistent else 13
    ctx = np.random.default_rng(2500).integers(20, 400, size=rows).tolist()
    sc = Scenario(shape, W, ctx, steps=4, seed=2500)
    buckets = [1] if persistent else [1, 4, 16]
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=512,
                   max_batch=buckets[-1], buckets=buckets, persistent_decode=persistent,
                   balanced_attention_rows=balanced)
    _randomise(dec, 2501)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    before = _pool_bits(dec)
    dec.decode(toks, pos, lens, slots, bt)
    torch.cuda.synchronize()
    dec.device_status()
    log("decode slots, persistent", persistent)
    _check_only_slots_changed(dec, before, [int(s) for s in slots], sc.num_blocks)
    before = _pool_bits(dec)
    dec.decode_continue()
    dec.decode_continue()
    torch.cuda.synchronize()
    dec.device_status()
    written = [oracle.slot_of(sc.tables[j], int(pos[j]) + d, 16) for j in range(rows) for d in (1, 2)]
    _check_only_slots_changed(dec, before, written, sc.num_blocks)
    dec.close()


def test_mixed_step_changes_only_its_slots_and_the_scratch_block(torch_cuda):
    """A packed mixed step (two prefill chunks, one continuing a cached prefix, and three decode rows),
    exact-size and bucketed, writes the slots of its tokens and nothing else outside the scratch
    block."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2, vocab=4096)
    W = synth.make_weights(shape, 0)
    ctx = [0, 40, 100, 33, 257]
    sc = Scenario(shape, W, ctx, steps=40, seed=2502)
    for buckets in (None, [64]):
        dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=512,
                       max_batch=1, buckets=[1], max_tokens=64, max_reqs=5, max_logit_rows=5,
                       mixed_buckets=buckets)
        _randomise(dec, 2503)
        bt = sc.table_array()
        chunks = [range(0, 20), range(40, 57)]           # a fresh prompt, a continuation over 40 cached keys
        toks, poss, qsl, lens, lidx = [], [], [0], [], []
        for j, r in enumerate(chunks):
            p = list(r)
            toks += synth.tokens(len(p), shape.vocab, 2504 + j).tolist()
            poss += p
            qsl.append(qsl[-1] + len(p)); lens.append(p[-1] + 1); lidx.append(qsl[-1] - 1)
        for j in (2, 3, 4):
            toks.append(int(sc.tokens[j])); poss.append(ctx[j])
            qsl.append(qsl[-1] + 1); lens.append(ctx[j] + 1); lidx.append(qsl[-1] - 1)
        req_of = [0] * 20 + [1] * 17 + [2, 3, 4]
        written = [oracle.slot_of(sc.tables[r], p, 16) for r, p in zip(req_of, poss)]
        before = _pool_bits(dec)
        dec.mixed(qsl, lens, toks, poss, written, bt, lidx, num_prefill_reqs=2)
        torch.cuda.synchronize()
        log("mixed slots, buckets", buckets, "last bucket", dec.last_mixed_bucket())
        _check_only_slots_changed(dec, before, written, sc.num_blocks)
        dec.close()
