"""Pins of the CPU oracle against things other than itself: closed forms, brute force on tiny
inputs, published known-answer vectors, and the pages' own worked examples."""
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from conftest import oracle_weights

F32 = np.float32


# ---------------------------------------------------------------- linear / norm / silu / rope

def test_linear_matches_explicit_loops():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5)).astype(F32)
    w = rng.standard_normal((4, 5)).astype(F32)     # [out, in], deliberately non-square
    b = rng.standard_normal(4).astype(F32)
    y = oracle.linear(x, w, b)
    for r in range(3):
        for i in range(4):
            ref = sum(float(x[r, k]) * float(w[i, k]) for k in range(5)) + float(b[i])
            assert abs(y[r, i] - ref) < 1e-5


def test_rmsnorm_closed_forms():
    # hand example: x = [3, 4]: mean square 12.5, rms = sqrt(12.5)
    y = oracle.rmsnorm(np.array([3.0, 4.0], F32), np.array([1.0, 2.0], F32), 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], rtol=1e-6)
    # constant vector c: y = c / sqrt(c^2 + eps) * w
    for c in (-2.5, 0.3, 7.0):
        w = np.linspace(0.5, 1.5, 16).astype(F32)
        y = oracle.rmsnorm(np.full(16, c, F32), w, 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6) * w, rtol=1e-6)
    # scale invariance (eps small relative to the mean square)
    x = np.random.default_rng(1).standard_normal((2, 64)).astype(F32)
    w = np.ones(64, F32)
    assert np.allclose(oracle.rmsnorm(x, w, 1e-6), oracle.rmsnorm(5.0 * x, w, 1e-6), atol=1e-5)
    # eps enters under the root: x = 0 gives 0, and x tiny is damped
    assert np.all(oracle.rmsnorm(np.zeros(8, F32), np.ones(8, F32), 1e-6) == 0)


def test_silu_mul_closed_forms():
    g = np.array([0.0, 1.0, 30.0, -30.0], F32)
    u = np.array([5.0, 2.0, 1.0, 1.0], F32)
    y = oracle.silu_mul(g, u)
    assert y[0] == 0.0
    assert abs(y[1] - 2.0 / (1.0 + math.exp(-1.0))) < 1e-6
    assert abs(y[2] - 30.0) < 1e-5          # silu(x) -> x for large x
    assert abs(y[3]) < 1e-11 * 1e4          # silu(x) -> 0 for very negative x


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(2).standard_normal((3, 4, 64)).astype(F32)
    assert np.array_equal(oracle.rope(x, [0, 0, 0], 1e6), x)


def test_rope_hand_cases_pin_pairing_and_frequency():
    # d = 2: the single pair rotates by angle pos * theta^0 = pos.
    e0 = np.array([[[1.0, 0.0]]], F32)
    e1 = np.array([[[0.0, 1.0]]], F32)
    assert np.allclose(oracle.rope(e0, [1], 1e6)[0, 0], [math.cos(1), math.sin(1)], atol=1e-6)
    assert np.allclose(oracle.rope(e1, [1], 1e6)[0, 0], [-math.sin(1), math.cos(1)], atol=1e-6)
    # d = 4, theta = 100: index 1 pairs with index 3 (rotate-half), frequency 100^(-2/4) = 0.1.
    x = np.zeros((1, 1, 4), F32)
    x[0, 0, 1] = 1.0
    y = oracle.rope(x, [2], 100.0)[0, 0]
    assert np.allclose(y, [0.0, math.cos(0.2), 0.0, math.sin(0.2)], atol=1e-6)


def test_rope_preserves_norm_and_relative_position():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 128)).astype(F32)
    k = rng.standard_normal((1, 1, 128)).astype(F32)
    for p in (1, 77, 4000):
        assert abs(np.linalg.norm(oracle.rope(q, [p], 1e6)) - np.linalg.norm(q)) < 1e-3
    dots = []
    for m, n in ((10, 3), (107, 100), (2007, 2000)):
        dots.append(float(np.sum(oracle.rope(q, [m], 1e6) * oracle.rope(k, [n], 1e6))))
    assert max(dots) - min(dots) < 2e-3


# ---------------------------------------------------------------- attention

def _attention_brute(q, k, v, q_pos):
    n, nq, d = q.shape
    L, nkv, _ = k.shape
    out = np.zeros((n, nq, d))
    for i in range(n):
        for h in range(nq):
            g = h // (nq // nkv)
            keys = [j for j in range(L) if j <= q_pos[i]]
            if not keys:
                continue
            s = [sum(float(q[i, h, t]) * float(k[j, g, t]) for t in range(d)) / math.sqrt(d) for j in keys]
            e = [math.exp(x) for x in s]
            z = sum(e)
            for jj, j in enumerate(keys):
                out[i, h] += e[jj] / z * v[j, g].astype(np.float64)
    return out


def test_attention_matches_brute_force_with_gqa_and_causal_mask():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 4, 8)).astype(F32)
    k = rng.standard_normal((6, 2, 8)).astype(F32)
    v = rng.standard_normal((6, 2, 8)).astype(F32)
    pos = [2, 4, 5]
    assert np.allclose(oracle.attend(q, k, v, pos), _attention_brute(q, k, v, pos), atol=2e-6)


def test_attention_single_key_and_equal_keys_and_empty():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 8)).astype(F32)
    k = rng.standard_normal((4, 1, 8)).astype(F32)
    v = rng.standard_normal((4, 1, 8)).astype(F32)
    assert np.allclose(oracle.attend(q, k, v, [0])[0, 1], v[0, 0], atol=1e-7)     # one visible key: o = v
    k_eq = np.repeat(k[:1], 4, axis=0)
    assert np.allclose(oracle.attend(q, k_eq, v, [3])[0, 0], v[:, 0].mean(0), atol=1e-6)   # equal keys: mean
    assert np.all(oracle.attend(q, k, v, [-1]) == 0)                                 # no key: zeros


# ---------------------------------------------------------------- sampling

def test_argmax_ties_go_to_lowest_index():
    assert oracle.argmax_lowest(np.array([1.0, 3.0, 3.0, 2.0], F32)) == 1
    assert list(oracle.sample(np.array([[0, 5, 5], [9, 9, 1]], F32), 0.0)) == [1, 0]


def test_philox_known_answer_vectors(golden_dir):
    rows = [l.split() for l in open(os.path.join(golden_dir, "philox4x32_10_kat.txt")) if not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        vals = [int(x, 16) for x in r]
        out = oracle.philox4x32_10(vals[0:4], vals[4:6])
        assert [int(o) for o in out] == vals[6:10]


def test_philox_uniforms_are_uniform_and_in_range():
    u = oracle.philox_uniforms(seed=1234, step=0, rows=64, cols=4096).ravel()
    assert u.min() >= 1e-10 and u.max() < 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    # different steps and rows give different streams
    a = oracle.philox_uniforms(1234, 0, 2, 8)
    b = oracle.philox_uniforms(1234, 1, 2, 8)
    assert not np.array_equal(a, b) and not np.array_equal(a[0], a[1])


@pytest.mark.parametrize("temperature", [0.7, 1.0])
def test_gumbel_max_frequencies_match_softmax(temperature):
    """Fast decode, section "Sampling without the CPU": 20,000 draws against softmax(z / T)."""
    z = np.linspace(-2.0, 1.5, 16).astype(F32)
    n = 20000
    u = oracle.philox_uniforms(seed=99, step=0, rows=n, cols=16)
    draws = oracle.sample(np.broadcast_to(z, (n, 16)), temperature, u)
    p = np.exp(z / temperature - np.max(z / temperature))
    p = p / p.sum()
    counts = np.bincount(draws, minlength=16)
    sigma = np.sqrt(n * p * (1 - p))
    assert np.all(np.abs(counts - n * p) < 5 * sigma + 1)
    assert stats.chisquare(counts, n * p).pvalue > 1e-3


def test_gumbel_limits():
    n = 20000
    u = oracle.philox_uniforms(seed=7, step=3, rows=n, cols=8)
    z = np.array([0, 0, 0, 40, 0, 0, 0, 0], F32)
    assert np.all(oracle.sample(np.broadcast_to(z, (n, 8)), 1.0, u) == 3)      # dominant logit wins
    z = np.linspace(0, 1, 8).astype(F32)
    counts = np.bincount(oracle.sample(np.broadcast_to(z, (n, 8)), 1e4, u), minlength=8)
    assert stats.chisquare(counts).pvalue > 1e-3                                  # huge T: uniform


# ---------------------------------------------------------------- top-k / top-p filters

def _keep_brute(z32, k, p):
    """Independent statement of the kept set: sort the (value, index) pairs, cut top-k by count with
    ties at the k-th value kept, then grow a prefix one token at a time until its mass reaches p."""
    V = len(z32)
    pairs = sorted(((-float(z32[i]), i) for i in range(V)))
    cand = [i for _, i in pairs]
    if 0 < k < V:
        kth = float(z32[cand[k - 1]])
        cand = [i for i in cand if float(z32[i]) >= kth]
    if p < 1.0:
        zmax = max(float(z32[i]) for i in cand)
        w = {i: math.exp(float(z32[i]) - zmax) for i in cand}
        tot = sum(w.values())
        chosen, acc = [], 0.0
        for i in cand:
            chosen.append(i)
            acc += w[i] / tot
            if acc >= p:
                break
        cand = chosen
    out = np.zeros(V, dtype=bool)
    out[cand] = True
    return out


def test_filters_off_keep_everything():
    z = np.random.default_rng(5).normal(size=50).astype(F32)
    for k, p in [(0, 1.0), (50, 1.0), (80, 1.0), (-3, 1.0), (0, 1.5)]:
        assert oracle.topk_topp_keep(z, k, p).all()


def test_top1_keeps_the_argmax_and_its_ties():
    z = np.array([0.5, 2.0, -1.0, 2.0, 1.0], dtype=F32)
    assert oracle.topk_topp_keep(z, 1, 1.0).tolist() == [False, True, False, True, False]
    assert oracle.topk_topp_keep(z, 3, 1.0).tolist() == [False, True, False, True, True]


def test_top_p_hand_computed_masses():
    # probabilities 0.4, 0.3, 0.2, 0.1 placed at shuffled indices
    z = np.log(np.array([0.2, 0.4, 0.1, 0.3])).astype(F32)
    keep = lambda k, p: np.nonzero(oracle.topk_topp_keep(z, k, p))[0].tolist()
    assert keep(0, 0.39) == [1]            # the second token starts at mass 0.4 >= 0.39
    assert keep(0, 0.41) == [1, 3]
    assert keep(0, 0.5) == [1, 3]
    assert keep(0, 0.75) == [0, 1, 3]
    assert keep(0, 0.95) == [0, 1, 2, 3]
    # top-k first: {0.4, 0.3} renormalised to 4/7, 3/7
    assert keep(2, 0.5) == [1]
    assert keep(2, 0.6) == [1, 3]
    assert keep(3, 0.85) == [0, 1, 3]      # 4/9 + 3/9 = 7/9 < 0.85: the third one is needed


def test_top_p_uniform_logits_keep_lowest_indices():
    z = np.zeros(10, dtype=F32)
    assert np.nonzero(oracle.topk_topp_keep(z, 0, 0.35))[0].tolist() == [0, 1, 2, 3]
    assert np.nonzero(oracle.topk_topp_keep(z, 0, 0.05))[0].tolist() == [0]


@pytest.mark.parametrize("seed", range(6))
def test_filters_match_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    V = 12
    z = np.round(rng.normal(size=V) * 2, 1).astype(F32)      # rounded: some exact ties
    for k in [0, 1, 2, 5, 11, 12]:
        for p in [1.0, 0.97, 0.8, 0.5, 0.2, 0.01]:
            got = oracle.topk_topp_keep(z, k, p)
            assert np.array_equal(got, _keep_brute(z, k, p)), (k, p)


def test_filtered_gumbel_max_frequencies_match_filtered_softmax():
    """The pages' milestone check, with filters: 20,000 Gumbel-max draws with Philox uniforms land
    on the kept tokens with frequencies softmax(z / T) renormalised over the kept set."""
    rng = np.random.default_rng(11)
    V, T, k, p, n = 16, 0.8, 10, 0.9, 20000
    logits = rng.normal(size=V).astype(F32) * F32(1.5)
    u = oracle.philox_uniforms(seed=4321, step=0, rows=n, cols=V)
    draws = oracle.sample(np.repeat(logits[None, :], n, 0), T, u, top_k=k, top_p=p)
    keep = oracle.topk_topp_keep(logits / F32(T), k, p)
    assert keep[draws].all()
    zz = logits.astype(np.float64) / T
    w = np.where(keep, np.exp(zz - zz.max()), 0.0)
    expected = w / w.sum() * n
    counts = np.bincount(draws, minlength=V)
    idx = np.nonzero(keep)[0]
    chi2 = float(((counts[idx] - expected[idx]) ** 2 / expected[idx]).sum())
    assert chi2 < stats.chi2.ppf(0.999, len(idx) - 1), chi2


# ---------------------------------------------------------------- paging and buckets

def test_bucket_choice_matches_page_example(golden_dir):
    for line in open(os.path.join(golden_dir, "bucket_example.txt")):
        if line.startswith("#") or not line.strip():
            continue
        b, r, want, pad = [x.strip() for x in line.split(";")]
        buckets = [int(x) for x in b.split()]
        got = oracle.bucket_for(int(r), buckets)
        assert got == int(want)
        assert len(oracle.pad_rows(int(r), got, 4)) == int(pad)
    with pytest.raises(ValueError):
        oracle.bucket_for(41, [1, 2, 4, 8, 16, 24, 32, 40])


def test_slot_arithmetic_brute_force():
    table = [7, 3, 11]
    slots = [oracle.slot_of(table, p, 16) for p in range(48)]
    want = [b * 16 + o for b in table for o in range(16)]
    assert slots == want
    assert all(r[2] == -1 and r[3] == 0 for r in oracle.pad_rows(13, 16, 5))


def test_weight_bytes_match_pages(golden_dir):
    shapes = {"qwen3-0.6b": synth.QWEN3_0_6B, "qwen2.5-1.5b": synth.QWEN2_5_1_5B}
    for line in open(os.path.join(golden_dir, "weight_bytes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, eb, gb, tol = [x.strip() for x in line.split(";")]
        got = synth.num_params(shapes[name]) * int(eb) / 1e9
        assert abs(got - float(gb)) / float(gb) < float(tol)


# ---------------------------------------------------------------- whole-model invariants

MICRO = synth.Shape("micro", 1, 8, 2, 1, 4, 6, 10, qk_norm=True, qkv_bias=True, tied=True, dtype="f32")


def _fp32_weights(shape, seed=0):
    return oracle_weights(synth.make_weights(shape, seed))


def test_zero_layer_contribution_gives_closed_form_logits():
    """With W_o = W_down = 0 the residual stays the embedding: logits = rmsnorm(E[t]) * g . E^T."""
    w = _fp32_weights(MICRO)
    for l in w["layers"]:
        l["wo"] = np.zeros_like(l["wo"])
        l["wd"] = np.zeros_like(l["wd"])
    t = 6
    hid = oracle.forward_request(MICRO, w, oracle.RequestCache(1), [t], [0])
    logits = oracle.final_logits(w, hid)[0]
    e = w["embed"][t].astype(np.float64)
    rms = math.sqrt(sum(x * x for x in e) / len(e) + 1e-6)
    for vid in range(MICRO.vocab):
        ref = sum(e[i] / rms * w["final_norm"][i] * w["embed"][vid, i] for i in range(MICRO.hidden))
        assert abs(logits[vid] - ref) < 1e-5


def test_single_token_layer_closed_form():
    """One token at position 0 sees one key, so each head's attention output is its KV head's v
    (RoPE at 0 is the identity and the scores do not matter). Written out with explicit loops."""
    s = MICRO.replace(q_heads=4, kv_heads=2, hidden=8, head_dim=2)
    w = _fp32_weights(s, seed=3)
    t = 4
    hid = oracle.forward_request(s, w, oracle.RequestCache(1), [t], [0])
    L = w["layers"][0]
    H, d, nq, nkv, I = s.hidden, s.head_dim, s.q_heads, s.kv_heads, s.intermediate

    def norm(x, g):
        rms = math.sqrt(sum(a * a for a in x) / len(x) + 1e-6)
        return [x[i] / rms * g[i] for i in range(len(x))]

    def mv(W, x, b=None):
        return [sum(W[i][k] * x[k] for k in range(len(x))) + (b[i] if b is not None else 0.0)
                for i in range(len(W))]

    r = [float(a) for a in w["embed"][t]]
    h = norm(r, L["in_norm"])
    v = mv(L["wv"], h, L["bv"])
    o = []
    for head in range(nq):
        g = head // (nq // nkv)
        o += v[g * d:(g + 1) * d]
    y = mv(L["wo"], o)
    r = [r[i] + y[i] for i in range(H)]
    h2 = norm(r, L["post_norm"])
    gate, up = mv(L["wg"], h2), mv(L["wu"], h2)
    a = [gate[i] / (1 + math.exp(-gate[i])) * up[i] for i in range(I)]
    x = mv(L["wd"], a)
    r = [r[i] + x[i] for i in range(H)]
    want = norm(r, w["final_norm"])
    assert np.allclose(hid[0], want, atol=1e-5)


def _layer_by_loops(s, w, toks, positions, qk_norm_order="before_rope", qk_norm_span="head"):
    """One layer, every token of one request, written out with scalar loops in fp64 in the order
    the per-layer operations are listed for Qwen3-0.6B (Fast decode: syncs, CUDA graphs and
    compilation, section "Where the time goes"): RMSNorm, Q/K/V, the two QK-norms, RoPE, cache
    write, causal attention, O projection + residual, RMSNorm, gate/up, SiLU * up, down +
    residual. Then the final RMSNorm. The two keyword arguments build the wrong variants the test
    must tell apart: the QK-norm after RoPE, and the QK-norm over all heads of a token at once."""
    H, d, nq, nkv, I = s.hidden, s.head_dim, s.q_heads, s.kv_heads, s.intermediate
    L = w["layers"][0]
    half = d // 2

    def norm(x, g):
        rms = math.sqrt(sum(a * a for a in x) / len(x) + s.eps)
        return [x[i] / rms * float(g[i % len(g)]) for i in range(len(x))]

    def mv(W, x, b=None):
        return [sum(float(W[i][k]) * x[k] for k in range(len(x))) + (float(b[i]) if b is not None else 0.0)
                for i in range(len(W))]

    def rot(x, pos):                      # rotate-half on one head
        y = list(x)
        for i in range(half):
            a = pos * s.theta ** (-2.0 * i / d)
            y[i] = x[i] * math.cos(a) - x[i + half] * math.sin(a)
            y[i + half] = x[i + half] * math.cos(a) + x[i] * math.sin(a)
        return y

    def heads(x, n):
        return [x[j * d:(j + 1) * d] for j in range(n)]

    def qk(x, n, g, pos):
        hs = heads(x, n)
        if qk_norm_order == "after_rope":
            hs = [rot(hh, pos) for hh in hs]
        if qk_norm_span == "head":
            hs = [norm(hh, g) for hh in hs]
        else:
            flat = norm([a for hh in hs for a in hh], g)
            hs = heads(flat, n)
        if qk_norm_order == "before_rope":
            hs = [rot(hh, pos) for hh in hs]
        return hs

    K, V, res, out = [], [], [], []
    for t, pos in zip(toks, positions):
        r = [float(a) for a in w["embed"][t]]
        h = norm(r, L["in_norm"])
        K.append(qk(mv(L["wk"], h, L["bk"]), nkv, L["k_norm"], pos))
        V.append(heads(mv(L["wv"], h, L["bv"]), nkv))
        res.append((r, qk(mv(L["wq"], h, L["bq"]), nq, L["q_norm"], pos)))
    for i, (r, q) in enumerate(res):
        o = []
        for head in range(nq):
            g = head // (nq // nkv)
            sc = [sum(q[head][c] * K[j][g][c] for c in range(d)) / math.sqrt(d)
                  for j in range(len(toks)) if positions[j] <= positions[i]]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            z = sum(e)
            o += [sum(e[j] / z * V[j][g][c] for j in range(len(e))) for c in range(d)]
        y = mv(L["wo"], o)
        r = [r[c] + y[c] for c in range(H)]
        h2 = norm(r, L["post_norm"])
        gate, up = mv(L["wg"], h2), mv(L["wu"], h2)
        a = [gate[c] / (1 + math.exp(-gate[c])) * up[c] for c in range(I)]
        x = mv(L["wd"], a)
        out.append(norm([r[c] + x[c] for c in range(H)], w["final_norm"]))
    return np.asarray(out)


def test_qk_norm_per_head_before_rope_closed_form():
    """Pins where the QK-norm acts and over what: per head, with one gain [d] shared by the heads,
    before RoPE. Three tokens at positions 0, 1, 2 see 1, 2 and 3 keys, so the scores matter; the
    gains differ inside every RoPE pair (norm-then-rotate differs from rotate-then-norm only
    then) and the heads of a token differ in scale (a norm over all heads differs only then)."""
    s = MICRO.replace(q_heads=4, kv_heads=2, hidden=8, head_dim=4, intermediate=6)
    w = _fp32_weights(s, seed=4)
    rng = np.random.default_rng(44)
    L = w["layers"][0]
    L["q_norm"] = rng.uniform(0.3, 2.5, s.head_dim).astype(F32)
    L["k_norm"] = rng.uniform(0.3, 2.5, s.head_dim).astype(F32)
    # head-dependent scale in the Q and K projections, so per-head and all-head norms differ
    L["wq"] = (L["wq"] * np.repeat(np.array([1.0, 4.0, 0.5, 2.0], F32), s.head_dim)[:, None] * 40).astype(F32)
    L["wk"] = (L["wk"] * np.repeat(np.array([3.0, 0.4], F32), s.head_dim)[:, None] * 40).astype(F32)
    L["wv"] = (L["wv"] * 40).astype(F32)
    L["wo"] = (L["wo"] * 40).astype(F32)
    toks, pos = [3, 7, 1], [0, 1, 2]
    got = oracle.forward_request(s, w, oracle.RequestCache(1), toks, pos)
    want = _layer_by_loops(s, w, toks, pos)
    assert np.allclose(got, want, atol=2e-5), np.abs(got - want).max()
    # the closed form tells the right order and span from the two plausible wrong ones
    for kw in ({"qk_norm_order": "after_rope"}, {"qk_norm_span": "all_heads"}):
        wrong = _layer_by_loops(s, w, toks, pos, **kw)
        assert np.abs(wrong[1:] - want[1:]).max() > 100 * 2e-5, kw


def test_incremental_decode_equals_full_sequence_prefill():
    s = synth.TINY
    w = _fp32_weights(s)
    toks = synth.tokens(12, s.vocab, 5)
    full = oracle.forward_request(s, w, oracle.RequestCache(s.layers), toks, list(range(12)))
    cache = oracle.RequestCache(s.layers)
    part = oracle.forward_request(s, w, cache, toks[:5], list(range(5)))
    rows = [part]
    for p in range(5, 12):
        rows.append(oracle.forward_request(s, w, cache, toks[p:p + 1], [p]))
    assert np.allclose(np.concatenate(rows), full, atol=2e-5)


def test_causality_future_tokens_do_not_change_the_past():
    s = synth.TINY_BIAS
    w = _fp32_weights(s)
    a = oracle.forward_request(s, w, oracle.RequestCache(s.layers), [5, 9, 100, 7], [0, 1, 2, 3])
    b = oracle.forward_request(s, w, oracle.RequestCache(s.layers), [5, 9, 100, 900], [0, 1, 2, 3])
    assert np.array_equal(a[:3], b[:3]) and not np.allclose(a[3], b[3])


def test_gqa_equals_mha_with_duplicated_kv_heads():
    g = synth.TINY                       # 4 query heads over 2 KV heads
    m = g.replace(kv_heads=4)
    wg = _fp32_weights(g)
    wm = _fp32_weights(g)
    d = g.head_dim
    for lg, lm in zip(wg["layers"], wm["layers"]):
        for name in ("wk", "wv"):
            heads = lg[name].reshape(g.kv_heads, d, g.hidden)
            lm[name] = np.repeat(heads, 2, axis=0).reshape(4 * d, g.hidden)
    toks = synth.tokens(6, g.vocab, 9)
    a = oracle.forward_request(g, wg, oracle.RequestCache(g.layers), toks, list(range(6)))
    b = oracle.forward_request(m, wm, oracle.RequestCache(m.layers), toks, list(range(6)))
    assert np.allclose(a, b, atol=2e-5)
