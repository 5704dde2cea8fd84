"""GPU: top-k / top-p filters before the Gumbel-max argmax ("Fast decode: syncs, CUDA graphs and
compilation", section "Sampling without the CPU"). The device's token must be the Gumbel argmax over
the oracle's kept set (same fp32 z, same uniforms). Top-k is an exact integer decision on both
sides. Top-p compares fp32 / fixed-point sums on the device with fp64 sums in the oracle, so a row
whose cut lies within 2e-4 of p may keep a slightly different set: there the token is checked
against the sets kept at p -/+ 2e-4."""
import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from harness import Scenario, log

pytestmark = pytest.mark.gpu
F32 = np.float32
EPS_P = 2e-4


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _decoder(shape, weights, **kw):
    import graph_replay_amd as g
    return g.Decoder(shape, weights, **kw)


def _check(got: int, z: np.ndarray, T: float, u: np.ndarray, k: int, p: float) -> bool:
    """True if `got` is exactly the oracle's filtered Gumbel-max token; asserts the relaxed rule
    (top-p boundary within EPS_P, or a near tie of the scores) otherwise and returns False."""
    z = z.astype(F32)
    if T == 0:
        exp = int(oracle.argmax_lowest(z))
        if got == exp:
            return True
        top = np.sort(z)[-2:]
        assert top[1] - top[0] < 1e-5 * max(1.0, abs(float(top[1]))), (got, exp)
        return False
    zs = z / F32(T)
    sc = oracle.gumbel_scores(z, T, u)
    keep = oracle.topk_topp_keep(zs, k, p)
    exp = int(np.argmax(np.where(keep, sc, -np.inf)))
    if got == exp:
        return True
    lo = oracle.topk_topp_keep(zs, k, max(p - EPS_P, 1e-9)) if p < 1 else keep
    hi = oracle.topk_topp_keep(zs, k, p + EPS_P) if p < 1 else keep
    assert hi[got], (got, exp, "token outside every admissible kept set")
    best_lo = float(np.max(np.where(lo, sc, -np.inf)))
    assert sc[got] >= best_lo - 1e-5 * max(1.0, abs(best_lo)), (got, exp)
    return False


def _rows(V: int, rng):
    """(logits, T, top_k, top_p) cases: plain, ties, a flat row, a peaked row, every filter edge."""
    n = rng.standard_normal
    cases = [
        (n(V) * 2, 0.0, 5, 0.5),                      # greedy: filters ignored
        (n(V) * 2, 1.0, 1, 1.0),                      # top-1
        (n(V) * 2, 0.7, 50, 1.0),
        (n(V) * 2, 1.0, 0, 0.9),
        (n(V) * 2, 0.8, 1000, 0.95),
        (n(V) * 2, 1.3, 20000, 0.5),
        (np.round(n(V) * 4) / 4, 1.0, 300, 1.0),      # exact ties at the k-th value
        (np.round(n(V) * 4) / 4, 1.0, 0, 0.6),        # ties around the top-p cut
        (np.zeros(V), 1.0, 0, 0.3),                   # one key value for every token
        (np.zeros(V), 1.0, 100, 1.0),                 # top-k over all-equal logits: all kept
        (np.concatenate([[20.0], n(V - 1)]), 1.0, 0, 0.5),   # one dominant token
        (n(V) * 2, 1.0, V, 1.0),                      # both filters off
        (n(V) * 2, 2.0, 5, 0.99),
        (n(V) * 0.1, 1.0, 0, 0.9),                    # flat row: the cut is deep in the vocabulary
        (n(V) * 2, 1.0, 0, 1e-6),                     # the top token only
        (n(V) * 3, 0.6, 7, 0.2),
    ]
    z = np.stack([c[0] for c in cases]).astype(F32)
    T = np.array([c[1] for c in cases], F32)
    k = np.array([c[2] for c in cases], np.int32)
    p = np.array([c[3] for c in cases], F32)
    return z, T, k, p


def test_step_sample_filters_match_oracle(torch_cuda):
    torch = torch_cuda
    shape = synth.TINY.replace(dtype="bf16", vocab=151936, layers=1)
    W = synth.make_weights(shape.replace(vocab=1024), 0)
    W["embed"] = torch.zeros(shape.vocab, shape.hidden, dtype=torch.bfloat16)
    W["lm_head"] = W["embed"]
    dec = _decoder(shape, W, num_blocks=4, max_blocks_per_seq=2, max_position=32, max_batch=16, buckets=[16],
                   use_graphs=False)
    z, T, k, p = _rows(shape.vocab, np.random.default_rng(9))
    rows = z.shape[0]
    zt = torch.as_tensor(z, device=dec.device)
    u = synth.uniforms(rows, shape.vocab, 33)
    exact = 0
    for rep, (uu, kw) in enumerate([(u, dict(uniforms=torch.as_tensor(u, device=dec.device))),
                                    (oracle.philox_uniforms(91, 4, rows, shape.vocab), dict(seed=91, counter=4))]):
        got = dec.sample(zt, temperature=T, top_k=k, top_p=p, **kw).cpu().numpy()
        for i in range(rows):
            log("rep", rep, "row", i, "T", float(T[i]), "k", int(k[i]), "p", float(p[i]), "token", int(got[i]))
            exact += _check(int(got[i]), z[i], float(T[i]), uu[i], int(k[i]), float(p[i]))
    assert exact >= 2 * rows - 2, exact
    dec.close()


def test_filtered_frequencies_match_filtered_softmax(torch_cuda):
    """The pages' milestone check with filters: 20,480 device draws (256 rows x 80 Philox steps of one
    logits row) against softmax(z / T) renormalised over the kept set."""
    torch = torch_cuda
    shape = synth.TINY.replace(dtype="bf16", vocab=1024, layers=1)
    W = synth.make_weights(shape, 0)
    dec = _decoder(shape, W, num_blocks=4, max_blocks_per_seq=2, max_position=32, max_batch=256, buckets=[256],
                   use_graphs=False)
    rng = np.random.default_rng(17)
    V, T, k, p = 128, 0.9, 40, 0.8
    row = (rng.standard_normal(V) * 1.5).astype(F32)
    zs = row / F32(T)
    keep = oracle.topk_topp_keep(zs, k, p)
    # the cut must not sit on a rounding boundary for this check
    assert np.array_equal(keep, oracle.topk_topp_keep(zs, k, p - 1e-3))
    assert np.array_equal(keep, oracle.topk_topp_keep(zs, k, p + 1e-3))
    zt = torch.as_tensor(np.repeat(row[None, :], 256, 0), device=dec.device)
    temps = np.full(256, T, F32)
    ks = np.full(256, k, np.int32)
    ps = np.full(256, p, F32)
    draws = []
    for step in range(80):
        draws.append(dec.sample(zt, temperature=temps, top_k=ks, top_p=ps, seed=5, counter=step).cpu().numpy())
    draws = np.concatenate(draws)
    assert keep[draws].all()
    w = np.where(keep, np.exp(zs.astype(np.float64) - zs.max()), 0.0)
    expected = w / w.sum() * draws.size
    counts = np.bincount(draws, minlength=V)
    idx = np.nonzero(keep)[0]
    chi2 = float(((counts[idx] - expected[idx]) ** 2 / expected[idx]).sum())
    assert chi2 < stats.chi2.ppf(0.999, len(idx) - 1), chi2
    dec.close()


def test_decode_steps_apply_filters_and_keep_them_across_replays(torch_cuda):
    """Tiny fp32 model, 4 rows: the decode step (a captured graph) samples with per-row top-k / top-p,
    and continued steps keep the filters; each step's tokens are the filtered Gumbel argmax over that
    step's logits with the Philox stream of that step."""
    torch = torch_cuda
    shape = synth.TINY
    W = synth.make_weights(shape, 0)
    sc = Scenario(shape, W, [5, 17, 30, 2], steps=4, seed=77)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=64, max_batch=4,
                   buckets=[1, 2, 4], sampling_filters=True)
    sc.inject(dec)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    T = np.array([1.0, 0.8, 0.0, 1.2], F32)
    k = np.array([5, 0, 3, 50], np.int32)
    p = np.array([1.0, 0.7, 0.5, 0.9], F32)
    seed = 0xABCDEF
    dec.decode(toks, pos, lens, slots, bt, temperature=T, seed=seed, top_k=k, top_p=p)
    exact = 0
    for step in range(3):
        if step:
            dec.decode_continue()
        torch.cuda.synchronize()
        z = dec.logits[:4].cpu().numpy()
        got = dec.tokens[:4].cpu().numpy()
        u = oracle.philox_uniforms(seed, step, 4, shape.vocab)
        for i in range(4):
            exact += _check(int(got[i]), z[i], float(T[i]), u[i], int(k[i]), float(p[i]))
    assert exact >= 11, exact
    dec.close()


def test_filters_need_the_config_flag(torch_cuda):
    shape = synth.TINY
    W = synth.make_weights(shape, 0)
    sc = Scenario(shape, W, [3], steps=1, seed=5)
    dec = _decoder(shape, W, num_blocks=sc.num_blocks, max_blocks_per_seq=sc.width, max_position=16, max_batch=1,
                   buckets=[1])
    sc.inject(dec)
    toks, pos, lens, slots, bt = sc.step_inputs(sc.tokens, sc.contexts)
    with pytest.raises(ValueError, match="sampling_filters"):
        dec.decode(toks, pos, lens, slots, bt, temperature=np.ones(1, F32), top_k=np.array([3], np.int32))
    dec.close()
