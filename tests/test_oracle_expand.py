"""Pins of the oracle's expansion, rerank and flattening.

What fixes them (EAGLE-2 notes, "Expanding the Draft Tree" and "Rerank draft
tokens"; EAGLE-1 notes, appendix A.1): top-k children; the value equation
V = prod of confidences on the root path; the frontier is the current layer's
top-k by value; the reranked top-m keeps the highest values, prefers shallower
nodes at equal value, and is connected; values never increase along a path.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import stats as sstats

from oracle import enumerate as en
from oracle import expand


def test_softmax_closed_forms():
    z = np.zeros(7, np.float32)
    M, S = expand.softmax_stats(z, 1.0)
    assert M == 0.0 and S == 7.0
    z = np.array([np.log(3.0), 0.0], np.float32)
    p = expand.softmax(z, 1.0)
    assert np.allclose(p, [0.75, 0.25], rtol=1e-7)
    # temperature 2 on logits 2*log(3), 0 gives the same law
    p2 = expand.softmax(np.array([2 * np.log(3.0), 0.0], np.float32), 2.0)
    assert np.allclose(p2, [0.75, 0.25], rtol=1e-6)
    # shift invariance and normalisation
    r = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.allclose(expand.softmax(r, 1.0), expand.softmax(r + np.float32(3.0), 1.0), rtol=1e-5)
    assert abs(expand.softmax(r, 0.7).sum() - 1.0) < 1e-12
    # greedy uses T' = 1
    assert np.allclose(expand.softmax(r, 0.0), expand.softmax(r, 1.0))


def test_greedy_children_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for trial in range(50):
        V = int(rng.integers(3, 40))
        k = int(rng.integers(1, V + 1))
        z = rng.integers(-3, 4, size=V).astype(np.float32)  # many exact ties
        toks, q, M, S, _ = expand.children_of_row(z, 0.0, k)
        brute = sorted(range(V), key=lambda v: (-float(z[v]), v))[:k]
        assert list(toks) == brute
        assert np.allclose(q, np.exp(z[brute].astype(np.float64) - z.max()) / np.exp(z - z.max()).sum())


def test_gumbel_children_distinct_and_deterministic():
    z = np.random.default_rng(2).standard_normal(1000).astype(np.float32)
    a = expand.children_of_row(z, 1.0, 10, seed=77, slot=3, req=1, round_id=5)[0]
    b = expand.children_of_row(z, 1.0, 10, seed=77, slot=3, req=1, round_id=5)[0]
    c = expand.children_of_row(z, 1.0, 10, seed=77, slot=4, req=1, round_id=5)[0]
    assert list(a) == list(b)
    assert len(set(a)) == 10
    assert list(a) != list(c)


def test_gumbel_order_follows_plackett_luce():
    """Ordered first-two draws match sequential sampling without replacement (chi^2)."""
    z = np.log(np.array([0.4, 0.3, 0.2, 0.1], np.float64)).astype(np.float32)
    q = expand.softmax(z, 1.0)
    counts = {}
    n = 12000
    for r in range(n):
        toks = tuple(int(t) for t in expand.children_of_row(z, 1.0, 2, seed=12345, slot=r % 7,
                                                             req=r // 7, round_id=9)[0])
        counts[toks] = counts.get(toks, 0) + 1
    pairs = list(itertools.permutations(range(4), 2))
    obs = np.array([counts.get(p, 0) for p in pairs], float)
    exp = np.array([en.pl_prob(q, p) for p in pairs]) * n
    chi2, pval = sstats.chisquare(obs, exp)
    assert pval > 1e-3, (chi2, pval)


def test_gumbel_order_temperature():
    """At T = 0.5 the first draw follows softmax(z / 0.5)."""
    z = np.array([0.3, 0.0, -0.4], np.float32)
    q = expand.softmax(z, 0.5)
    n = 9000
    first = np.zeros(3)
    for r in range(n):
        first[expand.children_of_row(z, 0.5, 1, seed=99, slot=r, req=0, round_id=1)[0][0]] += 1
    chi2, pval = sstats.chisquare(first, q * n)
    assert pval > 1e-3


def _random_children_fn(rng, V, k, tie_mode):
    def fn(s, path):
        toks = rng.choice(V, size=k, replace=False)
        if tie_mode == "equal":
            q = np.full(k, np.float32(0.5) ** int(rng.integers(1, 4)), np.float32)
        elif tie_mode == "zero":
            q = rng.choice(np.array([0.0, 1e-30, 0.25, 0.5, 1.0], np.float32), size=k)
        elif tie_mode == "tiny":
            q = (rng.random(k) * 1e-12).astype(np.float32)
        else:
            q = rng.dirichlet(np.ones(V))[toks].astype(np.float32)
        return toks, q
    return fn


def _check_tree_properties(t, k, D, m):
    S = 1 + (D - 1) * k
    N = m + 1
    par, dep, val = t["node_parent"], t["node_depth"], t["node_value"]
    assert len(par) == N and par[0] == -1 and dep[0] == 0
    # parents precede children, depth increases by one, BFS order
    for i in range(1, N):
        assert 0 <= par[i] < i
        assert dep[i] == dep[par[i]] + 1
        assert dep[i] >= dep[i - 1]
    # siblings contiguous and in sampling order
    for i in range(2, N):
        if par[i] == par[i - 1]:
            assert t["node_sib"][i] > t["node_sib"][i - 1]
        else:
            assert par[i] > par[i - 1]
    # values never increase along a path; value equals the product of confidences
    for i in range(1, N):
        assert val[i] <= val[par[i]]
        chain = []
        j = i
        while j > 0:
            chain.append(t["node_q"][j])
            j = par[j]
        v = np.float32(1.0)
        for qq in chain[::-1]:
            v = np.float32(v * qq)
        assert v == val[i]
    # top-m: every kept node's value >= every dropped pool node's value;
    # at equal value a kept node is never deeper than a dropped one.
    kept = set(int(e) for e in t["node_pool"][1:])
    pv, pd = t["pool_val"].reshape(-1), t["pool_depth"].reshape(-1)
    dropped = [e for e in range(S * k) if e not in kept]
    if dropped:
        vmin = min(pv[e] for e in kept)
        vmax = max(pv[e] for e in dropped)
        assert vmin >= vmax
        for e in kept:
            for f in dropped:
                if pv[e] == pv[f]:
                    assert pd[e] <= pd[f]
    # frontier: expanded nodes of layer d hold the layer's k best values
    for s in range(1, S):
        e = int(t["slot_src"][s])
        d = int(pd[e])
        layer = [f for f in range(S * k) if pd[f] == d]
        expanded = set(int(t["slot_src"][x]) for x in range(1, S) if pd[int(t["slot_src"][x])] == d)
        assert len(expanded) == min(k, len(layer))
        others = [f for f in layer if f not in expanded]
        if others:
            assert min(pv[x] for x in expanded) >= max(pv[x] for x in others)
    # pool index order equals (depth, cidx) order
    keys = [(int(pd[e]), int(t["pool_cidx"].reshape(-1)[e])) for e in range(S * k)]
    assert keys == sorted(keys)
    # pool_flat is the inverse of node_pool
    pf = t["pool_flat"].reshape(-1)
    for f in range(1, N):
        assert pf[t["node_pool"][f]] == f
    assert (pf >= 0).sum() == m


@settings(max_examples=150, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), k=st.integers(1, 4), D=st.integers(1, 4),
       mfrac=st.floats(0.0, 1.0), tie_mode=st.sampled_from(["none", "equal", "zero", "tiny"]))
def test_tree_invariants(seed, k, D, mfrac, tie_mode):
    rng = np.random.default_rng(seed)
    V = max(k + 1, 6)
    P = k + (D - 1) * k * k
    m = max(1, int(round(mfrac * P)))
    t = expand.build_tree(k, D, m, 0, _random_children_fn(rng, V, k, tie_mode))
    _check_tree_properties(t, k, D, m)


def test_rerank_prefers_shallower_on_exact_ties():
    # every confidence is 1: all values equal 1, so the top-m is the m shallowest
    def fn(s, path):
        return np.arange(3) + 10 * s, np.ones(3, np.float32)
    t = expand.build_tree(3, 3, 5, 0, fn)
    assert list(t["node_depth"]) == [0, 1, 1, 1, 2, 2]
    assert list(t["node_parent"]) == [-1, 0, 0, 0, 1, 1]


def test_expand_request_on_draft_rows():
    rng = np.random.default_rng(5)
    k, D, m, V = 3, 4, 12, 500
    S = 1 + (D - 1) * k
    rows = (2.0 * rng.standard_normal((S, V))).astype(np.float32)
    for T in (1.0, 0.0):
        out = expand.expand_request(rows, 7, T, k, D, m, seed=31, req=2, round_id=4)
        _check_tree_properties(out, k, D, m)
        # each slot's children are its own row's top keys
        for s in range(S):
            toks = expand.children_of_row(rows[s], T, k, 31, s, 2, 4)[0]
            assert list(out["pool_tok"][s]) == list(toks)
