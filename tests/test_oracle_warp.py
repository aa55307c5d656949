"""Pins of the sampling warps (oracle/warp.py) and of their use in a round.

hubwiz section 2: speculative decoding stays exact under top-k and nucleus
sampling when both distributions are adjusted the same way before the test.

* The kept set is checked against a brute-force sort of (t desc, id asc):
  top-k keeps exactly the first k; the nucleus keeps the shortest prefix whose
  mass reaches top_p (minimal and sufficient); at least min_keep tokens.
* Special cases: no warp is the plain softmax; top-k = 1 is the argmax (lowest
  id on ties).
* Children drawn from a warped row lie in its support and follow the warped
  law (chi-square on the first draw).
* A whole round with warped draft and target laws is lossless with respect to
  the warped target law (exact enumeration on a tiny vocabulary).
"""
import numpy as np
import pytest
from scipy import stats as sstats

from oracle import enumerate as en
from oracle import expand, warp


def _brute_order(t):
    return sorted(range(len(t)), key=lambda v: (-float(t[v]), v))


@pytest.mark.parametrize("seed", range(5))
def test_top_k_is_the_first_k_of_the_order(seed):
    rng = np.random.default_rng(seed)
    z = np.round(rng.standard_normal(200) * 2, 1).astype(np.float32)  # rounded: many exact ties
    for T in (1.0, 0.7):
        t = expand.scaled_logits(z, T)
        order = _brute_order(t)
        for k in (1, 5, 37, 200, 500):
            w = warp.warp_support(z, T, top_k=k)
            kept = set(order[:min(k, 200)])
            assert set(np.nonzero(w["mask"])[0]) == kept
            assert w["id_b"] == order[min(k, 200) - 1]
            # the boundary describes the set: t > t_b, or t == t_b and id <= id_b
            desc = {v for v in range(200) if t[v] > w["t_b"] or (t[v] == w["t_b"] and v <= w["id_b"])}
            assert desc == kept


@pytest.mark.parametrize("seed", range(5))
def test_nucleus_is_minimal_and_sufficient(seed):
    rng = np.random.default_rng(100 + seed)
    z = (rng.standard_normal(300) * 1.5).astype(np.float32)
    T = 1.0
    t = expand.scaled_logits(z, T).astype(np.float64)
    order = _brute_order(t.astype(np.float32))
    for top_k in (0, 120):
        base = order if top_k == 0 else order[:top_k]
        e = np.exp(t[base] - t.max())
        for top_p in (0.05, 0.5, 0.9, 0.99):
            w = warp.warp_support(z, T, top_k=top_k, top_p=top_p)
            n = w["n"]
            assert set(np.nonzero(w["mask"])[0]) == set(base[:n])
            mass = np.cumsum(e)
            assert mass[n - 1] >= top_p * e.sum() * (1 - 1e-12)
            if n > 1:
                assert mass[n - 2] < top_p * e.sum()
            np.testing.assert_allclose(w["S"], e[:n].sum(), rtol=1e-12)
    # at least min_keep tokens
    w = warp.warp_support(z, T, top_p=1e-6, min_keep=10)
    assert w["n"] == 10 and set(np.nonzero(w["mask"])[0]) == set(order[:10])


def test_special_cases():
    rng = np.random.default_rng(7)
    z = rng.standard_normal(50).astype(np.float32)
    np.testing.assert_allclose(warp.warped_softmax(z, 0.8), expand.softmax(z, 0.8), rtol=1e-14)
    z[[3, 17]] = z.max() + 1.0  # tie for the maximum
    p = warp.warped_softmax(z, 1.0, top_k=1)
    assert p[3] == 1.0 and p.sum() == 1.0
    # proportional to the softmax on the support, zero elsewhere
    p = warp.warped_softmax(z, 1.0, top_k=10, top_p=0.7)
    s = expand.softmax(z, 1.0)
    on = p > 0
    np.testing.assert_allclose(p[on] / s[on], (p[on] / s[on])[0], rtol=1e-12)
    assert abs(p.sum() - 1.0) < 1e-12


def test_warped_children_follow_the_warped_law():
    rng = np.random.default_rng(3)
    V, k = 40, 3
    z = rng.standard_normal(V).astype(np.float32)
    wp = (12, 0.8)
    q = warp.warped_softmax(z, 1.0, wp[0], wp[1], min_keep=k)
    sup = set(np.nonzero(q > 0)[0])
    n = 6000
    first = np.zeros(V)
    for r in range(n):
        toks, qs, M, S, _ = expand.children_of_row(z, 1.0, k, seed=4242, slot=r % 11, req=r // 11, warp=wp)
        assert set(int(t) for t in toks) <= sup and len(set(toks.tolist())) == k
        np.testing.assert_allclose(qs, q[toks].astype(np.float32), rtol=1e-6)
        first[toks[0]] += 1
    idx = sorted(sup)
    chi2, pval = sstats.chisquare(first[idx], q[idx] * n)
    assert pval > 1e-3, (chi2, pval)


def _warped_laws(V, seed, top_k, top_p, k):
    p, q = en.random_path_laws(V, seed, zero_frac=0.0)

    def w(f):
        def g(path):
            d = f(path)
            z = np.log(d).astype(np.float32)
            return warp.warped_softmax(z, 1.0, top_k, top_p, min_keep=k)
        return g
    return w(p), w(q)


@pytest.mark.parametrize("V,k,D,m,top_k,top_p", [(4, 2, 2, 3, 3, 1.0), (4, 2, 2, 6, 0, 0.6), (5, 1, 3, 3, 2, 0.9)])
def test_warped_round_is_lossless(V, k, D, m, top_k, top_p):
    pw, qw = _warped_laws(V, 5, top_k, top_p, k)
    law = en.round_law(V, k, D, m, 0, pw, qw)
    tgt = en.target_law(V, D, 0, pw)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    assert en.law_distance(law, tgt) < 1e-13
    # and the warp changed the law: it is not the unwarped target's
    p, _ = en.random_path_laws(V, 5, zero_frac=0.0)
    assert en.law_distance(tgt, en.target_law(V, D, 0, p)) > 1e-3
