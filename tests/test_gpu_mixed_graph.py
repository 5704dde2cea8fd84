"""GPU: mixed (prefill chunks + decode rows) steps padded to token-count buckets and replayed as
hipGraphs. The bucketed plan must give bit-identical results with and without graphs, match the
exact-size plan and the oracle within tolerance, and fall back to the exact-size plan for steps
larger than the largest bucket or with per-row prefill attention."""
import numpy as np
import pytest

import synth
from harness import TOL, fp32_weights, log, max_abs, near_tie_ok
from test_gpu_configs import MixedCase, _decoder

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _mixed_run(case, W, torch, *, mixed_buckets, use_graphs, max_tokens, mode=0, repeat=1):
    """One decoder, `repeat` identical mixed steps; returns logits, tokens of the last and the bucket."""
    nreq = len(case.prefill_lens) + len(case.decode_ctx)
    dec = _decoder(case.shape, W, num_blocks=case.num_blocks, max_blocks_per_seq=case.width,
                   max_position=max(case.decode_ctx + case.prefill_lens) + 16, max_batch=1, buckets=[1],
                   max_tokens=max_tokens, max_reqs=nreq + 2, max_logit_rows=nreq + 3, use_graphs=use_graphs,
                   mixed_buckets=mixed_buckets)
    case.inject(dec)
    outs = []
    for _ in range(repeat):
        dec.mixed(**case.packed(), prefill_attention=mode)
        torch.cuda.synchronize()
        outs.append((dec.logits[:nreq].cpu().numpy().copy(), dec.tokens[:nreq].cpu().numpy().copy()))
    bucket = dec.last_mixed_bucket()
    # rows past num_logits are not sampled: their token slots keep their previous contents (zero)
    spare = dec.tokens[nreq:nreq + 3].cpu().numpy().copy()
    dec.close()
    return outs, bucket, spare


def _check_case(case, W, torch, buckets, expect_bucket, max_tokens, tol, oracle_check):
    g_outs, gb, spare = _mixed_run(case, W, torch, mixed_buckets=buckets, use_graphs=True, max_tokens=max_tokens,
                                   repeat=2)
    assert gb == expect_bucket, (gb, expect_bucket)
    assert np.all(spare == 0), spare
    (lg, tg), (lg2, tg2) = g_outs
    assert np.array_equal(lg, lg2) and np.array_equal(tg, tg2), "graph replays differ"
    e_outs, eb, _ = _mixed_run(case, W, torch, mixed_buckets=buckets, use_graphs=False, max_tokens=max_tokens)
    assert eb == expect_bucket
    le, te = e_outs[0]
    assert np.array_equal(lg, le), max_abs(lg, le)
    assert np.array_equal(tg, te)
    x_outs, xb, _ = _mixed_run(case, W, torch, mixed_buckets=None, use_graphs=True, max_tokens=max_tokens)
    assert xb == 0
    lx, _ = x_outs[0]
    assert max_abs(lg, lx) <= tol, max_abs(lg, lx)
    if oracle_check:
        log("oracle")
        ref = case.oracle_logits(fp32_weights(W))
        for r in range(ref.shape[0]):
            assert max_abs(lg[r], ref[r]) <= tol, (r, max_abs(lg[r], ref[r]))
            assert near_tie_ok(int(tg[r]), ref[r], tol), r


def test_qwen25_mixed_step_bucketed_graph(torch_cuda):
    """Qwen2.5-1.5B shape fp16, 2 layers: the 544-token mixed step (prefill 16/240/256 + 32 decode rows)
    padded to the 576 bucket, and a 59-token step padded to 64, each replayed twice as a graph."""
    torch = torch_cuda
    wl = synth.workload_q25_mixed()
    shape = wl.shape.replace(layers=2)
    W = synth.make_weights(shape, 0)
    buckets = [64, 128, 576, 1024]
    log("q25 mixed 544 tokens")
    case = MixedCase(shape, wl.prefill_lens, wl.decode_contexts, wl.input_seed)
    _check_case(case, W, torch, buckets, 576, 1024, TOL["f16"], oracle_check=True)
    log("q25 mixed 59 tokens")
    small = MixedCase(shape, [16, 40], [64, 1024, 16], wl.input_seed + 7)
    _check_case(small, W, torch, buckets, 64, 1024, TOL["f16"], oracle_check=True)


def test_tiny_f32_mixed_step_bucketed_graph(torch_cuda):
    """Tiny fp32 shape: the bucketed plan with per-row attention for every token, graph == eager
    bitwise and == the oracle at 1e-4."""
    torch = torch_cuda
    shape = synth.TINY
    W = synth.make_weights(shape, 0)
    case = MixedCase(shape, [16, 33], [5, 40], 4242)
    _check_case(case, W, torch, [32, 64, 128], 64, 128, TOL["f32"], oracle_check=True)


def test_mixed_step_outside_buckets_runs_exact_plan(torch_cuda):
    """A step larger than the largest bucket, and a step asking for per-row prefill attention, run the
    exact-size plan (bucket 0) and still match the bucketed result."""
    torch = torch_cuda
    shape = synth.QWEN2_5_1_5B.replace(layers=2)
    W = synth.make_weights(shape, 0)
    case = MixedCase(shape, [16, 40], [64, 1024, 16], 5151)
    big, bb, _ = _mixed_run(case, W, torch, mixed_buckets=[32], use_graphs=True, max_tokens=128)
    assert bb == 0
    rows, rb, _ = _mixed_run(case, W, torch, mixed_buckets=[64], use_graphs=True, max_tokens=128, mode=1)
    assert rb == 0
    fit, fb, _ = _mixed_run(case, W, torch, mixed_buckets=[64], use_graphs=True, max_tokens=128)
    assert fb == 64
    assert max_abs(big[0][0], fit[0][0]) <= TOL["f16"]
    assert max_abs(rows[0][0], fit[0][0]) <= TOL["f16"]
