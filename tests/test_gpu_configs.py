"""GPU parity at the workload shapes: the mixed (packed prefill + decode) step, the batch-1 greedy
loop after a real prefill, batch-256 buckets with padding, and the invariants of graph replay."""
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


class MixedCase:
    """Prefill chunks of fresh prompts first, then decode rows over injected KV, in one packed step."""

    def __init__(self, shape, prefill_lens, decode_ctx, seed):
        self.shape = shape
        self.prefill_lens = list(prefill_lens)
        self.decode_ctx = list(decode_ctx)
        self.seed = seed
        self.prompts = [synth.tokens(n, shape.vocab, seed + 10 + j) for j, n in enumerate(prefill_lens)]
        self.dec_tokens = synth.tokens(len(decode_ctx), shape.vocab, seed + 99)
        self.sc = Scenario(shape, None, [0] * len(prefill_lens) + self.decode_ctx, steps=0, seed=seed)
        # the prefill requests need blocks for their prompts: rebuild tables over prompt + context lengths
        need = [n + 1 for n in prefill_lens] + [c + 1 for c in decode_ctx]
        self.num_blocks = sum(-(-n // 16) for n in need) + 2
        self.tables = synth.block_tables(need, self.num_blocks, seed, shuffled=True)
        self.width = max(len(t) for t in self.tables)
        self.sc.tables = self.tables
        self.sc.width = self.width

    def packed(self):
        P = len(self.prefill_lens)
        toks, pos, slots, qsl, lens, lidx = [], [], [], [0], [], []
        for j, n in enumerate(self.prefill_lens):
            toks += list(self.prompts[j]); pos += list(range(n))
            slots += [oracle.slot_of(self.tables[j], p, 16) for p in range(n)]
            qsl.append(qsl[-1] + n); lens.append(n); lidx.append(qsl[-1] - 1)
        for i, c in enumerate(self.decode_ctx):
            j = P + i
            toks.append(int(self.dec_tokens[i])); pos.append(c)
            slots.append(oracle.slot_of(self.tables[j], c, 16))
            qsl.append(qsl[-1] + 1); lens.append(c + 1); lidx.append(qsl[-1] - 1)
        bt = np.full((len(self.tables), self.width), -1, np.int32)
        for j, t in enumerate(self.tables):
            bt[j, :len(t)] = t
        return dict(query_start_loc=qsl, seq_lens=lens, tokens=toks, positions=pos, slots=slots, block_table=bt,
                    logits_indices=lidx, num_prefill_reqs=P)

    def inject(self, dec):
        self.sc.contexts = [0] * len(self.prefill_lens) + self.decode_ctx
        self.sc.inject(dec)

    def oracle_logits(self, W32):
        out = []
        for j, n in enumerate(self.prefill_lens):
            cache = oracle.RequestCache(self.shape.layers)
            hid = oracle.forward_request(self.shape, W32, cache, self.prompts[j], list(range(n)))
            out.append(oracle.final_logits(W32, hid[-1:])[0])
        for i, c in enumerate(self.decode_ctx):
            j = len(self.prefill_lens) + i
            cache = self.sc.oracle_cache(j)
            hid = oracle.forward_request(self.shape, W32, cache, [int(self.dec_tokens[i])], [c])
            out.append(oracle.final_logits(W32, hid)[0])
        return np.stack(out)


def _run_mixed(case, W, mode, torch):
    n_tok = sum(case.prefill_lens) + len(case.decode_ctx)
    nreq = len(case.prefill_lens) + len(case.decode_ctx)
    dec = _decoder(case.shape, W, num_blocks=case.num_blocks, max_blocks_per_seq=case.width,
                   max_position=max(case.decode_ctx + case.prefill_lens) + 16, max_batch=1, buckets=[1],
                   max_tokens=n_tok, max_reqs=nreq, max_logit_rows=nreq, use_graphs=False)
    case.inject(dec)
    dec.mixed(**case.packed(), prefill_attention=mode)
    torch.cuda.synchronize()
    out = dec.logits[:nreq].cpu().numpy().copy(), dec.tokens[:nreq].cpu().numpy().copy()
    dec.close()
    return out


@pytest.mark.parametrize("layers", [2, 28], ids=["2-layers", "full"])
def test_qwen25_mixed_step_packed_prefill(torch_cuda, layers):
    """Qwen2.5-1.5B shape fp16: one packed step of prefill chunks 16/240/256 and 32 decode rows with
    contexts from {16, 64, 256, 1024, 4096}; packed MFMA prefill attention == per-row attention ==
    the oracle."""
    torch = torch_cuda
    wl = synth.workload_q25_mixed()
    shape = wl.shape.replace(layers=layers)
    log("q25 mixed layers", layers)
    W = synth.make_weights(shape, 0)
    case = MixedCase(shape, wl.prefill_lens, wl.decode_contexts, wl.input_seed)
    packed, ptok = _run_mixed(case, W, 0, torch)
    rows, rtok = _run_mixed(case, W, 1, torch)
    assert max_abs(packed, rows) <= TOL["f16"], max_abs(packed, rows)
    log("oracle")
    W32 = fp32_weights(W)
    ref = case.oracle_logits(W32)
    for r in range(ref.shape[0]):
        assert max_abs(packed[r], ref[r]) <= TOL["f16"], (r, max_abs(packed[r], ref[r]))
        assert near_tie_ok(int(ptok[r]), ref[r], TOL["f16"]), r


def test_qwen3_bs1_prefill_then_graph_greedy_loop(torch_cuda):
    """Qwen3-0.6B bf16, 1,024-token prompt prefilled through the packed MFMA path, then 64 greedy graph
    replays continuing on the device. The logits of every step and every generated token are
    checked against the oracle, teacher-forced on the GPU's tokens."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    n, steps = 1024, 64
    prompt = synth.tokens(n, shape.vocab, 1002)
    table = synth.block_tables([n + steps + 2], -(-(n + steps + 2) // 16) + 2, 1002, shuffled=True)[0]
    bt = np.asarray([table], np.int32)
    dec = _decoder(shape, W, num_blocks=len(table) + 2, max_blocks_per_seq=len(table), max_position=n + steps + 16,
                   max_batch=1, buckets=[1], max_tokens=n, max_reqs=1, max_logit_rows=1, history=True)
    pos = np.arange(n, dtype=np.int32)
    slots = np.array([oracle.slot_of(table, int(p), 16) for p in pos], np.int32)
    log("gpu prefill")
    dec.mixed([0, n], [n], prompt, pos, slots, bt, [n - 1], num_prefill_reqs=1)
    torch.cuda.synchronize()
    prefill_logits = dec.logits[0].cpu().numpy().copy()
    first = int(dec.tokens[0].item())
    step_logits = []
    dec.decode([first], [n], [n + 1], [oracle.slot_of(table, n, 16)], bt)
    torch.cuda.synchronize()
    step_logits.append(dec.logits[0].cpu().numpy().copy())
    for i in range(1, steps):
        dec.decode_continue()
        torch.cuda.synchronize()
        step_logits.append(dec.logits[0].cpu().numpy().copy())
    torch.cuda.synchronize()
    hist = dec.history[0, n:n + steps].cpu().numpy()
    dec.close()
    log("oracle prefill")
    cache = oracle.RequestCache(shape.layers)
    hid = oracle.forward_request(shape, W32, cache, prompt, list(range(n)))
    ref0 = oracle.final_logits(W32, hid[-1:])[0]
    assert max_abs(prefill_logits, ref0) <= TOL["bf16"], max_abs(prefill_logits, ref0)
    assert near_tie_ok(first, ref0, TOL["bf16"])
    # teacher forcing: the GPU's inputs (first token, then its own outputs) through the oracle at once
    inputs = [first] + hist[:-1].tolist()
    log("oracle decode over", len(inputs), "tokens")
    hid = oracle.forward_request(shape, W32, cache, inputs, list(range(n, n + steps)))
    ref = oracle.final_logits(W32, hid)
    for i, lg in enumerate(step_logits):
        assert max_abs(lg, ref[i]) <= TOL["bf16"], (i, max_abs(lg, ref[i]))
    bad = [i for i in range(steps) if not near_tie_ok(int(hist[i]), ref[i], TOL["bf16"])]
    assert not bad, bad


def _bs256_setup(torch, layers, use_graphs=True, buckets=(1, 2, 4, 8, 16, 32, 64, 128, 256)):
    wl = synth.workload_q3_bs256()
    shape = wl.shape.replace(layers=layers)
    W = synth.make_weights(shape, 0)
    sc = Scenario(shape, W, wl.contexts, steps=4, seed=wl.input_seed)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=max(wl.contexts) + 32,
                   max_batch=buckets[-1], buckets=list(buckets), use_graphs=use_graphs)
    return wl, shape, W, sc, dec


def _fill_random(dec, seed):
    torch = dec.torch
    gen = torch.Generator(device=dec.device)
    gen.manual_seed(seed)
    for l in range(len(dec.k_pool)):
        dec.k_pool[l].normal_(generator=gen)
        dec.v_pool[l].normal_(generator=gen)


def test_bs256_sampled_rows_vs_oracle_and_padding(torch_cuda):
    """Qwen3-0.6B bf16 (2 layers), 256 rows, contexts {16..4096} + 64..256, T = 0.7 Gumbel. A 16-row
    sample is checked against the oracle (the batch-256 attention runs on the balanced kernel); in
    padded buckets (13 -> 16, 100 -> 128, 200 -> 256) the padding rows' contents never change the
    real rows' bits."""
    torch = torch_cuda
    wl, shape, W, sc, dec = _bs256_setup(torch, 2)
    _fill_random(dec, 7)
    sample = list(range(0, 256, 16))
    sub = Scenario(shape, W, [wl.contexts[j] for j in sample], steps=4, seed=wl.input_seed)
    # inject the sampled rows' seeded histories at their own table slots
    for l in range(shape.layers):
        for i, j in enumerate(sample):
            k, v = sub.kv(i, l)
            c = wl.contexts[j]
            p = np.arange(c)
            blk = torch.as_tensor(np.asarray(sc.tables[j])[p // 16], device=dec.device)
            off = torch.as_tensor(p % 16, device=dec.device)
            dec.k_pool[l][blk, :, off, :] = k.to(dec.device)
            dec.v_pool[l][blk, :, :, off] = v.to(dec.device)   # V is dim-major
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    temp = np.full(256, 0.7, np.float32)
    seed = 0xC0FFEE
    dec.decode(toks, pos, lens, slots, bt, temperature=temp, seed=seed)
    torch.cuda.synchronize()
    full = dec.logits[:256].cpu().numpy().copy()
    ftok = dec.tokens[:256].cpu().numpy().copy()
    W32 = fp32_weights(W)
    u = oracle.philox_uniforms(seed, 0, 256, shape.vocab)
    for i, j in enumerate(sample):
        hid = oracle.forward_request(shape, W32, sub.oracle_cache(i), [toks[j]], [pos[j]])
        ref = oracle.final_logits(W32, hid)[0]
        assert max_abs(full[j], ref) <= TOL["bf16"], (j, max_abs(full[j], ref))
        assert near_tie_ok(int(ftok[j]), oracle.gumbel_scores(ref, 0.7, u[j]), TOL["bf16"]), j
    # Padding: r rows padded up to a bucket. Whatever the padding rows hold (here: other tokens and
    # positions, no keys, slot -1), the real rows get the same bits. Up to 127 rows the attention
    # is the split grid, which sees each row alone, so there the real rows also match a run of the
    # bucket's size in real rows bit for bit; from 128 rows the balanced kernel's split points
    # follow every row's length, so such a run matches to the rounding bound.
    for r, bucket in ((13, 16), (100, 128), (200, 256)):
        dec.decode(toks[:r], pos[:r], lens[:r], slots[:r], bt[:r])
        torch.cuda.synchronize()
        assert dec.last_bucket() == bucket
        got = dec.logits[:r].cpu().numpy().copy()
        assert np.all(np.isfinite(dec.logits[:bucket].cpu().numpy()))
        pt, pp, pl, ps, pb = (x[:bucket].copy() for x in (toks, pos, lens, slots, bt))
        pt[r:], pp[r:], pl[r:], ps[r:], pb[r:] = 5, 3, 0, -1, 0
        dec.decode(pt, pp, pl, ps, pb)
        torch.cuda.synchronize()
        other = dec.logits[:r].cpu().numpy()
        assert np.array_equal(got, other), (r, max_abs(got, other))
        dec.decode(toks[:bucket], pos[:bucket], lens[:bucket], slots[:bucket], bt[:bucket])
        torch.cuda.synchronize()
        full = dec.logits[:r].cpu().numpy()
        if bucket < 128:
            assert np.array_equal(got, full), (r, max_abs(got, full))
        else:
            assert max_abs(got, full) <= TOL["bf16"], (r, max_abs(got, full))
    dec.close()


def test_graph_equals_eager_and_replays_are_deterministic(torch_cuda):
    torch = torch_cuda
    outs = {}
    for graphs in (True, False):
        wl, shape, W, sc, dec = _bs256_setup(torch, 2, use_graphs=graphs, buckets=(8, 16, 32))
        _fill_random(dec, 11)
        toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
        r = 20
        # Gumbel step with the first Philox counter on a fresh context, then greedy replays
        dec.decode(toks[:r], pos[:r], lens[:r], slots[:r], bt[:r], temperature=np.ones(r, np.float32), seed=5)
        torch.cuda.synchronize()
        gumbel = (dec.logits[:r].cpu().numpy().copy(), dec.tokens[:r].cpu().numpy().copy())
        res = []
        for rep in range(2):
            dec.decode(toks[:r], pos[:r], lens[:r], slots[:r], bt[:r])
            dec.decode_continue()
            torch.cuda.synchronize()
            res.append((dec.logits[:r].cpu().numpy().copy(), dec.tokens[:r].cpu().numpy().copy()))
        assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
        outs[graphs] = (gumbel, res[0])
        dec.close()
    for i in range(2):
        assert np.array_equal(outs[True][i][0], outs[False][i][0])
        assert np.array_equal(outs[True][i][1], outs[False][i][1])


def test_nan_poisoned_foreign_blocks_change_nothing(torch_cuda):
    """Every pool block no request owns (and the scratch block) is filled with NaN; the outputs of the
    real rows stay bit-identical and finite (padding rows read nothing)."""
    torch = torch_cuda
    wl, shape, W, sc, dec = _bs256_setup(torch, 2, buckets=(16, 32))
    _fill_random(dec, 13)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    r = 13
    dec.decode(toks[:r], pos[:r], lens[:r], slots[:r], bt[:r])
    torch.cuda.synchronize()
    clean = dec.logits[:r].cpu().numpy().copy()
    owned = np.zeros(sc.num_blocks, bool)
    for j in range(r):
        owned[np.asarray(sc.tables[j])[:-(-(sc.contexts[j] + 1) // 16)]] = True
    foreign = torch.as_tensor(np.nonzero(~owned)[0], device=dec.device)
    for l in range(shape.layers):
        dec.k_pool[l][foreign] = float("nan")
        dec.v_pool[l][foreign] = float("nan")
        # and the not-yet-written slots past each row's new token in its own last block
        for j in range(r):
            c = sc.contexts[j] + 1
            if c % 16:
                blk = sc.tables[j][(c - 1) // 16]
                dec.k_pool[l][blk, :, c % 16:, :] = float("nan")
                dec.v_pool[l][blk, :, :, c % 16:] = float("nan")
    # the step writes K/V at the same slots again, so rerun from the same inputs
    dec.decode(toks[:r], pos[:r], lens[:r], slots[:r], bt[:r])
    torch.cuda.synchronize()
    poisoned = dec.logits[:r].cpu().numpy()
    assert np.array_equal(clean, poisoned)
    assert np.all(np.isfinite(dec.logits[:16].cpu().numpy()))
    dec.close()


def test_step_sample_explicit_uniforms_and_philox(torch_cuda):
    torch = torch_cuda
    shape = synth.TINY.replace(dtype="bf16", vocab=151936, layers=1)
    W = synth.make_weights(shape.replace(vocab=1024), 0)
    W["embed"] = torch.zeros(shape.vocab, shape.hidden, dtype=torch.bfloat16)
    W["lm_head"] = W["embed"]
    dec = _decoder(shape, W, num_blocks=4, max_blocks_per_seq=2, max_position=32, max_batch=8, buckets=[8])
    rng = np.random.default_rng(3)
    rows = 8
    z = (rng.standard_normal((rows, shape.vocab)) * 2).astype(np.float32)
    u = synth.uniforms(rows, shape.vocab, 21)
    temp = np.array([0.0, 0.7, 1.0, 1.0, 0.5, 2.0, 1.0, 0.0], np.float32)
    zt = torch.as_tensor(z, device=dec.device)
    got = dec.sample(zt, temperature=temp, uniforms=torch.as_tensor(u, device=dec.device)).cpu().numpy()
    for i in range(rows):
        sc = z[i] if temp[i] == 0 else oracle.gumbel_scores(z[i], float(temp[i]), u[i])
        top = np.sort(sc)[-2:]
        if int(got[i]) != int(oracle.argmax_lowest(sc)):
            assert top[1] - top[0] < 1e-5 * max(1.0, abs(top[1])), i
    # Philox uniforms drawn on the device == the oracle's Philox-4x32-10 stream
    got = dec.sample(zt, temperature=temp, seed=77, counter=5).cpu().numpy()
    up = oracle.philox_uniforms(77, 5, rows, shape.vocab)
    for i in range(rows):
        sc = z[i] if temp[i] == 0 else oracle.gumbel_scores(z[i], float(temp[i]), up[i])
        top = np.sort(sc)[-2:]
        if int(got[i]) != int(oracle.argmax_lowest(sc)):
            assert top[1] - top[0] < 1e-5 * max(1.0, abs(top[1])), i
    dec.close()


def test_invalid_calls_raise(torch_cuda):
    shape = synth.TINY.replace(dtype="bf16")
    W = synth.make_weights(shape, 0)
    dec = _decoder(shape, W, num_blocks=8, max_blocks_per_seq=2, max_position=32, max_batch=4, buckets=[2, 4])
    bt = np.array([[0, 1]] * 5, np.int32)
    with pytest.raises(ValueError):          # more rows than the largest bucket
        dec.decode([1] * 5, [3] * 5, [4] * 5, [3] * 5, bt)
    with pytest.raises(ValueError):          # seq_len must be position + 1
        dec.decode([1], [3], [5], [3], bt[:1])
    with pytest.raises(ValueError):          # slot must be the table's slot for the position
        dec.decode([1], [3], [4], [4], bt[:1])
    with pytest.raises(ValueError):          # token outside the vocabulary
        dec.decode([5000], [3], [4], [3], bt[:1])
    with pytest.raises(ValueError):          # continue before any batch
        dec.decode_continue()
    with pytest.raises(ValueError):          # no mixed-step buffers
        dec.mixed([0, 1], [1], [1], [0], [0], bt[:1], [0], num_prefill_reqs=1)
    dec.close()
