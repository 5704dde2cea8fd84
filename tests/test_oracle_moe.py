"""Pins of the MoE oracle (oracle/moe.py) against things other than itself: the grouping worked
by hand from the definition in "Removing overhead: fusion, graphs and async scheduling" (section
"A MoE layer that never asks the host"), a second grouping by scalar counting loops, the
grouping's invariants, brute-force loops, the dense SwiGLU MLP that one expert reduces to, and
the symmetries of the layer."""
import os

import numpy as np
import pytest

import oracle
from oracle import moe

F64 = np.float64


def _read_golden(golden_dir, name):
    out = {}
    for line in open(os.path.join(golden_dir, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = (s.strip() for s in line.split(":"))
        out[k] = [int(t) for t in v.split()]
    return out


def test_align_worked_example(golden_dir):
    g = _read_golden(golden_dir, "moe_align_example.txt")
    ids = np.asarray(g["expert_ids"], np.int64).reshape(g["tokens"][0], g["top_k"][0])
    s, be, npad = moe.moe_align(ids, g["num_experts"][0], g["block_m"][0])
    assert s.tolist() == g["sorted_ids"]
    assert be.tolist() == g["block_expert"]
    assert npad == g["num_padded"][0]


def _align_by_counting(flat, E, bm):
    """The grouping contract checked with scalar loops, one assignment at a time: count each
    expert's assignments, lay the groups out in expert order with each group's length rounded up
    to whole blocks, then place assignment i at its group's first row plus the number of earlier
    assignments of the same expert. Ids outside [0, E) get no row."""
    total = len(flat)
    m_max = -(-(total + E * (bm - 1)) // bm) * bm
    count = [0] * E
    for e in flat:
        if 0 <= e < E:
            count[e] += 1
    first_row, row = [0] * E, 0
    for e in range(E):
        first_row[e] = row
        row += -(-count[e] // bm) * bm
    sorted_ids = [total] * m_max
    seen = [0] * E
    for i, e in enumerate(flat):
        if 0 <= e < E:
            sorted_ids[first_row[e] + seen[e]] = i
            seen[e] += 1
    block_expert = [E - 1] * (m_max // bm)
    for e in range(E):
        for r in range(first_row[e], first_row[e] + -(-count[e] // bm) * bm, bm):
            block_expert[r // bm] = e
    return np.asarray(sorted_ids), np.asarray(block_expert), row


@pytest.mark.parametrize("E,n,k,bm", [(4, 3, 2, 4), (8, 1, 1, 16), (16, 37, 4, 16), (128, 32, 8, 16),
                                      (5, 50, 3, 1), (3, 20, 2, 64), (64, 9, 6, 7), (1, 10, 1, 16)])
def test_align_equals_counting_loops_and_invariants(E, n, k, bm):
    rng = np.random.default_rng(E * 1000 + n * 10 + k)
    ids = rng.integers(0, E, size=(n, k))
    if E > 4:
        ids[ids == 2] = 3          # an expert with no assignment
    flat = ids.reshape(-1)
    total = flat.size
    s, be, npad = moe.moe_align(ids, E, bm)
    s2, be2, npad2 = _align_by_counting(flat.tolist(), E, bm)
    assert np.array_equal(s, s2) and np.array_equal(be, be2) and npad == npad2
    m_max = moe.align_rows(total, E, bm)
    assert s.size == m_max and m_max % bm == 0 and be.size == m_max // bm
    real = s[s < total]
    assert sorted(real.tolist()) == list(range(total))           # every assignment exactly once
    assert np.all(s[npad:] == total) and npad % bm == 0
    for b in range(npad // bm):
        blk = s[b * bm:(b + 1) * bm]
        live = blk[blk < total]
        assert live.size > 0                                     # no block is all padding
        assert np.all(flat[live] == be[b])                       # one expert per block
        assert np.all(np.diff(live) > 0)                         # assignment order inside
        assert np.all(blk[:live.size] == live)                   # padding only at the end
    assert np.all(np.diff(be[:npad // bm]) >= 0)                 # groups in expert order
    assert np.all(be[npad // bm:] == E - 1)


def test_align_skips_out_of_range_ids():
    ids = np.array([[0, 7], [-1, 1], [1, 0]])
    s, be, npad = moe.moe_align(ids, 2, 2)
    assert s[:npad].tolist() == [0, 5, 3, 4]
    assert be[:2].tolist() == [0, 1] and npad == 4
    assert 1 not in s.tolist() and 2 not in s.tolist()


def _tiny_layer(E=3, k=2, D=4, inter=3, n=3, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D))
    gu = rng.standard_normal((E, 2 * inter, D)) * 0.5
    dn = rng.standard_normal((E, D, inter)) * 0.5
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)])
    w = rng.uniform(0.1, 1.0, size=(n, k))
    return x, gu, dn, w, ids


def test_layer_matches_scalar_loops():
    x, gu, dn, w, ids = _tiny_layer()
    n, k = ids.shape
    E, two_i, D = gu.shape
    inter = two_i // 2
    got = moe.moe_layer(x, gu, dn, w, ids)
    for t in range(n):
        for d in range(D):
            acc = 0.0
            for j in range(k):
                e = ids[t, j]
                a = []
                for i in range(inter):
                    g = sum(gu[e, i, c] * x[t, c] for c in range(D))
                    u = sum(gu[e, inter + i, c] * x[t, c] for c in range(D))
                    a.append(g / (1.0 + np.exp(-g)) * u)
                acc += w[t, j] * sum(dn[e, d, i] * a[i] for i in range(inter))
            assert abs(got[t, d] - acc) < 1e-12


def test_one_expert_is_the_dense_swiglu_mlp():
    """E = 1, k = 1, weight 1: the layer is the dense MLP down(silu(gate x) * up x), here from the
    decoder oracle's separately pinned linear and silu_mul (gate and up as separate matrices)."""
    rng = np.random.default_rng(5)
    D, inter, n = 32, 24, 6
    x = rng.standard_normal((n, D)).astype(np.float32)
    wg = (rng.standard_normal((inter, D)) * 0.1).astype(np.float32)
    wu = (rng.standard_normal((inter, D)) * 0.1).astype(np.float32)
    wd = (rng.standard_normal((D, inter)) * 0.1).astype(np.float32)
    dense = oracle.linear(oracle.silu_mul(oracle.linear(x, wg), oracle.linear(x, wu)), wd)
    got = moe.moe_layer(x, np.concatenate([wg, wu])[None], wd[None], np.ones((n, 1)), np.zeros((n, 1), np.int64))
    assert np.allclose(got, dense, rtol=1e-5, atol=1e-6)


def test_layer_symmetries():
    x, gu, dn, w, ids = _tiny_layer(E=6, k=3, D=8, inter=5, n=7, seed=3)
    base = moe.moe_layer(x, gu, dn, w, ids)
    # linear in the router weights
    assert np.allclose(moe.moe_layer(x, gu, dn, 2.5 * w, ids), 2.5 * base, rtol=1e-12, atol=1e-14)
    w1 = w * np.random.default_rng(1).uniform(0, 1, size=w.shape)
    assert np.allclose(moe.moe_layer(x, gu, dn, w1, ids) + moe.moe_layer(x, gu, dn, w - w1, ids), base,
                       rtol=1e-12, atol=1e-14)
    # relabelled experts (weights permuted to match)
    perm = np.random.default_rng(2).permutation(6)
    inv = np.argsort(perm)
    assert np.allclose(moe.moe_layer(x, gu[perm], dn[perm], w, inv[ids]), base, rtol=1e-12, atol=1e-14)
    # a token's slots in another order
    sp = np.array([2, 0, 1])
    assert np.allclose(moe.moe_layer(x, gu, dn, w[:, sp], ids[:, sp]), base, rtol=1e-12, atol=1e-14)
    # the same expert in two slots adds its weights
    ids2 = ids.copy()
    ids2[:, 1] = ids2[:, 0]
    merged = moe.moe_layer(x, gu, dn, np.stack([w[:, 0] + w[:, 1], w[:, 2]], 1), ids2[:, [0, 2]])
    assert np.allclose(moe.moe_layer(x, gu, dn, w, ids2), merged, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bm", [1, 4, 16, 64])
def test_grouped_route_equals_definition(bm):
    x, gu, dn, w, ids = _tiny_layer(E=9, k=3, D=16, inter=8, n=23, seed=bm)
    ids[4, 1] = 9          # out of range: contributes nothing
    ids[7, :] = -1         # a token with no valid expert: zeros
    got = moe.moe_grouped(x, gu, dn, w, ids, bm)
    ref = moe.moe_layer(x, gu, dn, w, ids)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    assert np.all(ref[7] == 0)
