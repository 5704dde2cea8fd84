"""GPU parity of the persistent single-row decode step (persistent_decode = 1): one kernel per step
at the Qwen3-0.6B widths, against the oracle and against the multi-kernel step on the same state."""
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


# histories before the step: the first token of a request (no keys), one split exactly (128 keys
# with the new one), the new key alone in the second split, ragged splits and tiles, and the
# 1,024-key context of the batch-1 workload
CONTEXTS = [0, 127, 128, 300, 1023, 1500]
# past 2,048 positions the items hold 128 keys: one item exactly (128 with the new key), the last
# 64-key width, the new key alone in an item, ragged items and tiles, and a 4,001-key row
CONTEXTS_WIDE = [0, 127, 2047, 2048, 2100, 3001, 4000]


@pytest.mark.parametrize("dtype,flags,wide", [("bf16", "qwen3", False), ("f16", "qwen3", False),
                                              ("bf16", "bias-no-qknorm", False), ("bf16", "qwen3", True)])
def test_persistent_step_matches_oracle_and_multikernel(torch_cuda, dtype, flags, wide):
    """Qwen3-0.6B widths, 2 layers, full vocabulary, bf16 and fp16, and the Qwen2.5 flags (QKV bias,
    no QK-norm) at the same widths: every context above as a batch-1 step through the persistent
    kernel; logits vs the oracle (3e-2) and vs the multi-kernel step (same inputs), greedy tokens
    under the near-tie rule, the new K/V the kernel writes to its slot, and then three
    device-continued steps against the multi-kernel step's. wide: max_position 4,096, where the
    kernel's attention items hold 128 keys."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2, dtype=dtype)
    if flags != "qwen3":
        shape = shape.replace(qk_norm=False, qkv_bias=True)
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    contexts = CONTEXTS_WIDE if wide else CONTEXTS
    sc = Scenario(shape, W, contexts, steps=4, seed=1101)
    kw = dict(num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=4096 if wide else 1536 + 16,
              max_batch=1, buckets=[1])
    dp = _decoder(shape, W, persistent_decode=True, **kw)
    dm = _decoder(shape, W, persistent_decode=False, **kw)
    sc.inject(dp)
    sc.inject(dm)
    bt_all = sc.table_array()
    for j, c in enumerate(contexts):
        log("persistent step", dtype, "context", c)
        tok = int(sc.tokens[j])
        slot = oracle.slot_of(sc.tables[j], c, 16)
        args = ([tok], [c], [c + 1], [slot], bt_all[j:j + 1])
        dp.decode(*args)
        dm.decode(*args)
        torch.cuda.synchronize()
        dp.device_status()
        gp, gm = dp.logits[0].cpu().numpy(), dm.logits[0].cpu().numpy()
        cache = sc.oracle_cache(j)
        hid = oracle.forward_request(shape, W32, cache, [tok], [c])
        ref = oracle.final_logits(W32, hid)[0]
        assert max_abs(gp, ref) <= TOL[dtype], (c, max_abs(gp, ref))
        assert max_abs(gp, gm) <= TOL[dtype], (c, max_abs(gp, gm))
        assert near_tie_ok(int(dp.tokens[0].item()), ref, TOL[dtype]), c
        assert int(dp.tokens[0].item()) == int(oracle.argmax_lowest(gp))
        # the new key and value the kernel stored at the slot (bf16) against the oracle's fp32 ones:
        # within 3e-2 relative above magnitude 1 (a bf16 ulp is 2^-7 relative, so this allows the
        # storage rounding plus a few ulps of upstream rounding order); the multi-kernel step's
        # stored values obey the same bound, so the two differ by at most twice it
        b, o = slot // 16, slot % 16
        for l in range(shape.layers):
            kp, km = dp.k_pool[l][b, :, o, :].float().cpu().numpy(), dm.k_pool[l][b, :, o, :].float().cpu().numpy()
            vp, vm = dp.v_pool[l][b, :, :, o].float().cpu().numpy(), dm.v_pool[l][b, :, :, o].float().cpu().numpy()
            kr, vr = cache.k[l][c], cache.v[l][c]
            for got, want, k in ((kp, kr, 1), (vp, vr, 1), (kp, km, 2), (vp, vm, 2)):
                lim = k * 3e-2 * np.maximum(1.0, np.abs(want))
                assert np.all(np.abs(got - want) <= lim), (c, l, k, float(np.max(np.abs(got - want) / lim)))
            assert float(np.abs(kr).max()) > 0
    # continue on the device from the last request: tokens, positions and slots advance in place
    for i in range(3):
        dp.decode_continue()
        dm.decode_continue()
        torch.cuda.synchronize()
        dp.device_status()
        gp, gm = dp.logits[0].cpu().numpy(), dm.logits[0].cpu().numpy()
        tp, tm = int(dp.tokens[0].item()), int(dm.tokens[0].item())
        if tp != tm:   # allowed only at a near tie; the steps then diverge, so stop comparing
            assert near_tie_ok(tp, gm, TOL[dtype]), i
            break
        assert max_abs(gp, gm) <= TOL[dtype], (i, max_abs(gp, gm))
    assert dp.kernels_per_decode(1) == 1   # the sampler runs inside the step kernel
    dp.close()
    dm.close()


def test_persistent_graph_equals_eager_bitwise_and_gumbel(torch_cuda):
    """The persistent step replayed from its graph gives the same bits as the eager launch, and
    repeating a host-fed step gives the same bits again (the kernel's reductions have a fixed
    order); Gumbel-max tokens equal the argmax of the scores over the GPU's own logits."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=3, vocab=4096)
    W = synth.make_weights(shape, 0)
    sc = Scenario(shape, W, [700], steps=3, seed=1102)
    kw = dict(num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=1024, max_batch=1, buckets=[1],
              persistent_decode=True)
    dg = _decoder(shape, W, use_graphs=True, **kw)
    de = _decoder(shape, W, use_graphs=False, **kw)
    sc.inject(dg)
    sc.inject(de)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    seed = 0x5EED_1102
    out = []
    for d in (dg, de, dg, de):   # both contexts take two host-fed steps (same Philox step counters)
        d.decode(toks, pos, lens, slots, bt, temperature=np.ones(1, np.float32), seed=seed)
        torch.cuda.synchronize()
        d.device_status()
        out.append((d.logits[0].cpu().numpy().copy(), int(d.tokens[0].item())))
    assert np.array_equal(out[0][0], out[1][0])
    assert np.array_equal(out[0][0], out[2][0])
    assert np.array_equal(out[1][0], out[3][0])
    assert out[0][1] == out[1][1]
    u = oracle.philox_uniforms(seed, 0, 1, shape.vocab)[0]
    s = oracle.gumbel_scores(out[1][0], 1.0, u)
    top = np.sort(s)[-2:]
    assert int(np.argmax(s)) == out[1][1] or top[1] - top[0] < 1e-5 * max(1.0, abs(top[1]))
    for _ in range(2):
        dg.decode_continue()
        de.decode_continue()
    torch.cuda.synchronize()
    dg.device_status()
    assert int(dg.tokens[0].item()) == int(de.tokens[0].item())
    assert np.array_equal(dg.logits[0].cpu().numpy(), de.logits[0].cpu().numpy())
    dg.close()
    de.close()


def test_persistent_bs1_workload_prefill_then_graph_greedy_loop(torch_cuda):
    """The batch-1 workload through the persistent step: Qwen3-0.6B bf16, 1,024-token prompt
    prefilled through the packed path, then all 256 greedy graph replays continuing on the device.
    The logits of every step and every generated token against the oracle, teacher-forced on the
    GPU's tokens; phase stamps of a profiled step are ordered."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B
    W = synth.make_weights(shape, 0)
    W32 = fp32_weights(W)
    n, steps = 1024, 256
    prompt = synth.tokens(n, shape.vocab, 1002)
    table = synth.block_tables([n + steps + 2], -(-(n + steps + 2) // 16) + 2, 1002, shuffled=True)[0]
    bt = np.asarray([table], np.int32)
    dec = _decoder(shape, W, num_blocks=len(table) + 2, max_blocks_per_seq=len(table), max_position=n + steps + 16,
                   max_batch=1, buckets=[1], max_tokens=n, max_reqs=1, max_logit_rows=1, history=True,
                   persistent_decode=True)
    pos = np.arange(n, dtype=np.int32)
    slots = np.array([oracle.slot_of(table, int(p), 16) for p in pos], np.int32)
    log("gpu prefill")
    dec.mixed([0, n], [n], prompt, pos, slots, bt, [n - 1], num_prefill_reqs=1)
    torch.cuda.synchronize()
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
    dec.device_status()
    hist = dec.history[0, n:n + steps].cpu().numpy()
    prof = dec.profile_decode()
    assert [k for k, _ in prof] == ["decode_step_persistent"]
    st = dec.phase_stamps()
    dec.device_status()
    dec.close()
    assert st is not None
    marks = [st[0]] + [st[8 * l + k] for l in range(shape.layers) for k in (1, 2, 3, 4, 5, 6)] + \
        [st[8 * shape.layers + 1], st[8 * shape.layers + 2]]
    assert all(m >= 0 for m in marks) and all(b >= a for a, b in zip(marks, marks[1:])), marks
    log("oracle prefill + decode")
    cache = oracle.RequestCache(shape.layers)
    oracle.forward_request(shape, W32, cache, prompt, list(range(n)))
    inputs = [first] + hist[:-1].tolist()
    hid = oracle.forward_request(shape, W32, cache, inputs, list(range(n, n + steps)))
    ref = oracle.final_logits(W32, hid)
    for i, lg in enumerate(step_logits):
        assert max_abs(lg, ref[i]) <= TOL["bf16"], (i, max_abs(lg, ref[i]))
    bad = [i for i in range(steps) if not near_tie_ok(int(hist[i]), ref[i], TOL["bf16"])]
    assert not bad, bad


def test_persistent_fused_sampling_equals_separate_sampler(torch_cuda):
    """The sampler fused into the persistent step's LM head against the separate sampling kernels
    behind the same step kernel (sampling_filters = 1 with the filters off), at temperature 0.8 over
    the full 151,936-token vocabulary (74 or 75 rows per LM-head wave): the same logits bitwise, the
    same token, history and continued state at every step (bit-exact); each token also equals
    step_sample's draw from the kernel's own logits at the step's Philox counter, and at temperature
    0 the lowest-index argmax."""
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2)
    W = synth.make_weights(shape, 0)
    n = 300
    sc = Scenario(shape, W, [n], steps=8, seed=1103)
    table, bt = sc.tables[0], sc.table_array()
    kw = dict(num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=n + 32, max_batch=1,
              buckets=[1], history=True, persistent_decode=True)
    df = _decoder(shape, W, **kw)
    ds = _decoder(shape, W, sampling_filters=True, **kw)
    for d in (df, ds):
        sc.inject(d)
    seed = 0x5EED_1103
    for temp in (0.8, 0.0):
        log("fused sampling, temperature", temp)
        tok = int(sc.tokens[0])
        args = ([tok], [n], [n + 1], [oracle.slot_of(table, n, 16)], bt)
        toks = {}
        for name, d in (("fused", df), ("separate", ds)):
            d.decode(*args, temperature=np.full(1, temp, np.float32), seed=seed)
            torch.cuda.synchronize()
            d.device_status()
            out = []
            for i in range(4):
                if i:
                    d.decode_continue()
                    torch.cuda.synchronize()
                    d.device_status()
                lg = d.logits[0:1].clone()
                t = int(d.tokens[0].item())
                out.append((lg.cpu().numpy()[0], t))
                if name == "fused":
                    # the step counter of host-fed step k is k (0 first), moved on by one per step
                    c = (0 if temp > 0 else 4) + i
                    want = int(d.sample(lg, temperature=np.full(1, temp, np.float32), seed=seed, counter=c)[0].item())
                    assert t == want, (temp, i, t, want)
                    if temp == 0:
                        assert t == int(oracle.argmax_lowest(out[-1][0])), i
            toks[name] = (out, d.history[0, n:n + 4].cpu().numpy().copy())
        (of, hf), (os_, hs) = toks["fused"], toks["separate"]
        for i in range(4):
            assert np.array_equal(of[i][0], os_[i][0]), (temp, i)
            assert of[i][1] == os_[i][1], (temp, i)
        assert np.array_equal(hf, hs), (hf, hs)
        assert hf.tolist() == [t for _, t in of]
    assert df.kernels_per_decode(1) == 1
    assert ds.kernels_per_decode(1) == 3   # step kernel, filter, sampler
    df.close()
    ds.close()


@pytest.mark.parametrize("filters", [False, True])
def test_persistent_given_up_wait_poisons_outputs_and_stops_advance(torch_cuda, filters):
    """The failure contract of the persistent step, forced from the host: with the give-up flag set
    (as a wait that gave up would set it) every bounded wait ends at once and every kernel exits
    normally; each step then writes NaN logits and token -1 and does not advance the row (graph
    replays included), with the sampler fused into the kernel and with the separate sampler behind
    it. step_device_status reports and clears the flag, and the next step continues exactly where
    the last good step left off: its logits and token equal, bit for bit, those of an identical
    decoder that never failed."""
    import graph_replay_amd as g
    torch = torch_cuda
    shape = synth.QWEN3_0_6B.replace(layers=2, vocab=4096)
    W = synth.make_weights(shape, 0)
    n = 200
    sc = Scenario(shape, W, [n], steps=8, seed=1104)
    table, bt = sc.tables[0], sc.table_array()
    kw = dict(num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=n + 32, max_batch=1,
              buckets=[1], history=True, persistent_decode=True, sampling_filters=filters)
    df = _decoder(shape, W, **kw)     # fails twice in the middle
    dr = _decoder(shape, W, **kw)     # reference: never fails
    for d in (df, dr):
        sc.inject(d)
    args = ([int(sc.tokens[0])], [n], [n + 1], [oracle.slot_of(table, n, 16)], bt)
    temp = np.full(1, 0.9, np.float32)
    for d in (df, dr):
        d.decode(*args, temperature=temp, seed=77)
        d.decode_continue()
    torch.cuda.synchronize()
    df.device_status()
    good_hist = df.history[0].cpu().numpy().copy()
    log("forcing the give-up flag, filters", filters)
    df.set_device_status(5)
    for _ in range(2):
        df.decode_continue()       # graph replays with every wait giving up at once
        torch.cuda.synchronize()
        assert int(df.tokens[0].item()) == -1
        assert bool(torch.isnan(df.logits[0]).all().item())
        assert np.array_equal(df.history[0].cpu().numpy(), good_hist)   # no advance
    with pytest.raises(g.StepError, match="site 5"):
        df.device_status()
    df.device_status()             # cleared
    for i in range(3):
        df.decode_continue()
        dr.decode_continue()
        torch.cuda.synchronize()
        df.device_status()
        assert np.array_equal(df.logits[0].cpu().numpy(), dr.logits[0].cpu().numpy()), i
        assert int(df.tokens[0].item()) == int(dr.tokens[0].item()) >= 0, i
    assert np.array_equal(df.history[0].cpu().numpy(), dr.history[0].cpu().numpy())
    df.close()
    dr.close()
