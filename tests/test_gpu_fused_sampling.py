"""The sampler fused into the LM head of multi-row steps (the streaming LM-head GEMV of 9-48 rows)
against the separate sampling kernel: batch 32 and a padded batch of 13 rows (bucket 16) at the full
151,936-token vocabulary, greedy and Gumbel-max rows mixed, over device-continued graph replays; and
the mixed step's sampled rows, bucketed and exact-size. Tokens, logits, history and continued state
are bit-identical, and each token equals step_sample's draw from the kernel's own logits."""
import numpy as np
import pytest

import synth
from harness import Scenario, log

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


@pytest.mark.parametrize("rows", [32, 13])
def test_decode_fused_lm_head_sampler_equals_separate_sampler(torch_cuda, rows):
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2)
    W = synth.make_weights(shape, 0)
    ctx = np.random.default_rng(2600 + rows).integers(60, 700, size=rows).tolist()
    sc = Scenario(shape, W, ctx, steps=6, seed=2600 + rows)
    kw = dict(num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=800, max_batch=32,
              buckets=[1, 2, 4, 8, 16, 32], history=True)
    df = _decoder(shape, W, **kw)                          # sampler in the LM head
    ds = _decoder(shape, W, sampling_filters=True, **kw)   # separate filter + sampler, filters off
    for d in (df, ds):
        sc.inject(d)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    temp = np.array([0.0 if j % 4 == 0 else (0.7 if j % 4 == 1 else 1.0 + 0.1 * (j % 3)) for j in range(rows)],
                    np.float32)
    seed = 0x5EED_2600
    out = {}
    for name, d in (("fused", df), ("separate", ds)):
        res = []
        for i in range(4):
            if i == 0:
                d.decode(toks, pos, lens, slots, bt, temperature=temp, seed=seed)
            else:
                d.decode_continue()
            torch.cuda.synchronize()
            lg = d.logits[:rows].clone()
            res.append((lg.cpu().numpy(), d.tokens[:rows].cpu().numpy().copy()))
            if name == "fused":
                want = d.sample(lg, temperature=temp, seed=seed, counter=i).cpu().numpy()
                assert np.array_equal(res[-1][1], want), (rows, i, np.nonzero(res[-1][1] != want))
        out[name] = (res, d.history[:rows].cpu().numpy().copy())
    log("fused sampler rows", rows)
    (rf, hf), (rs, hs) = out["fused"], out["separate"]
    for i in range(4):
        assert np.array_equal(rf[i][0], rs[i][0]), i
        assert np.array_equal(rf[i][1], rs[i][1]), i
    assert np.array_equal(hf, hs)
    assert df.kernels_per_decode(32) == ds.kernels_per_decode(32) - 2   # no filter, no sampler launch
    assert df.kernels_per_decode(16) == ds.kernels_per_decode(16) - 2
    df.close()
    ds.close()


def test_mixed_fused_lm_head_sampler_equals_step_sample(torch_cuda):
    """Qwen2.5-1.5B shape fp16 (2 layers): prefill chunks 16/240/256 and 32 decode rows, 35 sampled
    rows (greedy and T = 0.8 mixed), exact-size and bucketed (device row count): every sampled row's
    token equals step_sample on the step's own logits at its Philox counter."""
    torch = torch_cuda
    wl = synth.workload_q25_mixed()
    shape = wl.shape.replace(layers=2)
    W = synth.make_weights(shape, 0)
    P = len(wl.prefill_lens)
    need = [n + 1 for n in wl.prefill_lens] + [c + 1 for c in wl.decode_contexts]
    nb = sum(-(-n // 16) for n in need) + 2
    tables = synth.block_tables(need, nb, wl.input_seed, shuffled=True)
    width = max(len(t) for t in tables)
    bt = np.full((len(tables), width), -1, np.int32)
    for j, t in enumerate(tables):
        bt[j, :len(t)] = t
    toks, pos, slots, qsl, lens, lidx = [], [], [], [0], [], []
    for j, n in enumerate(wl.prefill_lens):
        toks += list(synth.tokens(n, shape.vocab, wl.input_seed + 10 + j))
        pos += list(range(n))
        slots += [int(bt[j][p // 16] * 16 + p % 16) for p in range(n)]
        qsl.append(qsl[-1] + n); lens.append(n); lidx.append(qsl[-1] - 1)
    dtok = synth.tokens(len(wl.decode_contexts), shape.vocab, wl.input_seed + 99)
    for i, c in enumerate(wl.decode_contexts):
        j = P + i
        toks.append(int(dtok[i])); pos.append(c); slots.append(int(bt[j][c // 16] * 16 + c % 16))
        qsl.append(qsl[-1] + 1); lens.append(c + 1); lidx.append(qsl[-1] - 1)
    T, R = qsl[-1], len(lens)
    temp = np.array([0.0 if r % 3 == 0 else 0.8 for r in range(R)], np.float32)
    seed = 0x5EED_2601
    for buckets in (None, [576]):
        dec = _decoder(shape, W, num_blocks=nb, max_blocks_per_seq=width, max_position=max(need) + 16, max_batch=1,
                       buckets=[1], max_tokens=576, max_reqs=R, max_logit_rows=R, mixed_buckets=buckets)
        gen = torch.Generator(device=dec.device)
        gen.manual_seed(2601)
        for l in range(shape.layers):
            dec.k_pool[l].normal_(generator=gen)
            dec.v_pool[l].normal_(generator=gen)
        for step in range(2):
            dec.mixed(qsl, lens, toks, pos, slots, bt, lidx, num_prefill_reqs=P, temperature=temp, seed=seed)
            torch.cuda.synchronize()
            lg = dec.logits[:R].clone()
            got = dec.tokens[:R].cpu().numpy().copy()
            want = dec.sample(lg, temperature=temp, seed=seed, counter=step).cpu().numpy()
            log("mixed fused sampler, buckets", buckets, "step", step, "bucket", dec.last_mixed_bucket())
            assert np.array_equal(got, want), (buckets, step, np.nonzero(got != want))
        dec.close()
