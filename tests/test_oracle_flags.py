"""Pins of the oracle's near-tie flags.

Parity excludes a request only where the oracle flags a decision whose deciding
gap lies inside a stated window (acceptance draws with |u - min(1, ratio)| below
1e-6, inverse-CDF draws within 1e-6 of the total from a cumulative boundary,
child keys within KEY_TIE_REL, frontier and rerank values within
VALUE_TIE_REL).  Each test plants a decision on either side of its window, so a
flag that fires too often (hiding real disagreements) or never (turning a
rounding difference into a failure) breaks one of them.
"""
import warnings

import numpy as np
import pytest

from oracle import accept as oaccept
from oracle import expand
from oracle import warp as owarp


def test_rel_gap_special_values():
    inf = float("inf")
    assert expand._rel_gap(1.0, 1.0) == 0.0
    assert expand._rel_gap(-inf, -inf) == 0.0          # both dropped: equal keys
    assert expand._rel_gap(3.0, -inf) == inf            # a kept key beside a dropped one is decided
    assert expand._rel_gap(-inf, 3.0) == inf
    assert expand._rel_gap(0.0, 0.0) == 0.0
    assert expand._rel_gap(2.0, 1.0) == 0.5
    assert expand._rel_gap(-2.0, -1.0) == 0.5
    g = expand._rel_gap(1.0, 1.0 + 1e-13)
    assert 0 < g < expand.KEY_TIE_REL
    for a, b in [(1.0, -inf), (-inf, -inf), (inf, inf), (0.0, 1e-300)]:
        assert not np.isnan(expand._rel_gap(a, b))


def test_gumbel_children_warp_keeping_exactly_k_flags_nothing():
    """A warp that keeps exactly k tokens puts key k+1 at -inf: a decided cut, no flag, no NaN."""
    z = np.random.default_rng(3).standard_normal(500).astype(np.float32)
    k = 4
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        toks, q, M, S, ties = expand.children_of_row(z, 1.0, k, seed=9, warp=(k, 1.0))
    assert ties == 0
    order = np.lexsort((np.arange(z.size), -z))
    assert set(toks) == set(order[:k])


def test_gumbel_planted_key_tie_is_flagged():
    """Two logits of 1e20: their fp64 keys t + g are equal (the noise is below an ulp), a true tie."""
    z = np.random.default_rng(4).standard_normal(300).astype(np.float32)
    z[17] = z[230] = np.float32(1e20)
    toks, _, _, _, ties = expand.children_of_row(z, 1.0, 3, seed=5)
    assert ties >= 1
    assert list(toks[:2]) == [17, 230]   # equal keys: lower id first
    # the same row without the plant has clear gaps
    z2 = z.copy()
    z2[230] = np.float32(-1e20)
    assert expand.children_of_row(z2, 1.0, 3, seed=5)[4] == 0


def test_greedy_children_never_flag_key_ties():
    z = np.zeros(50, np.float32)     # every logit tied: the id order decides, exactly on both sides
    toks, _, _, _, ties = expand.children_of_row(z, 0.0, 5)
    assert ties == 0 and list(toks) == [0, 1, 2, 3, 4]


def _tree_with_q(k, D, m, qfn):
    """build_tree with children (token = slot * k + j) whose confidences come from qfn(slot)."""
    def children_fn(s, path):
        return np.arange(k) + 100 * s, np.asarray(qfn(s), np.float32)
    return expand.build_tree(k, D, m, 7, children_fn)


def test_frontier_flag_planted_values():
    k = 2
    # layer 1: q = (0.5, 0.5 * (1 - d)); children of different parents compete for the frontier at depth 2
    for d, want in [(1e-7, True), (1e-3, False)]:
        def qfn(s):
            if s == 0:
                return [0.6, 0.4]
            # slot 1 expands the first child (value 0.6), slot 2 the second (value 0.4)
            return [0.5, 0.1] if s == 1 else [0.75 * (1 - d), 0.1]
        t = _tree_with_q(k, 3, 4, qfn)
        # values: 0.6*0.5 = 0.3 and 0.4*0.75*(1-d) ~ 0.3: rank 0/1 of the depth-2 layer are near-tied
        assert (t["ties"]["frontier"] >= 1) == want, (d, t["ties"])


def test_frontier_same_q_siblings_are_exempt():
    """Siblings with equal q have bit-equal values on both sides; their order is the exact cidx: no flag."""
    k = 3
    # depth 1: three siblings with q = 0.25 compete for two frontier places (k = 3 > layer - 1)
    t = _tree_with_q(k, 2, 5, lambda s: [0.25, 0.25, 0.25] if s == 0 else [0.2, 0.1, 0.05])
    assert t["ties"]["frontier"] == 0
    assert list(t["slot_src"][1:]) == [0, 1, 2]     # cidx order decides
    # the same equal values from different parents are flagged
    t = _tree_with_q(2, 3, 4, lambda s: [0.5, 0.25] if s == 0 else ([0.25, 0.1] if s == 1 else [0.5, 0.1]))
    assert t["ties"]["frontier"] >= 1


def test_rerank_flag_planted_values():
    k = 2

    def qfn(s):
        return [0.5, 0.3] if s == 0 else [0.6, 0.2]
    # pool values: depth 1: 0.5, 0.3; depth 2 under 0.5: 0.3, 0.1; under 0.3: 0.18, 0.06
    # m = 2 cuts between 0.5 and the tied pair 0.3/0.3 of different depths: flagged
    t = _tree_with_q(k, 2, 2, qfn)
    assert t["ties"]["rerank"] == 1
    # the shallower node wins the exact tie
    assert 1 in set(t["pool_flat"][0]) or 2 in set(t["pool_flat"][0])
    sel_depths = sorted(t["node_depth"][1:])
    assert sel_depths == [1, 1]
    # m = 3 cuts between 0.3 and 0.18: clear
    assert _tree_with_q(k, 2, 3, qfn)["ties"]["rerank"] == 0
    # m = P keeps everything: nothing to decide
    assert _tree_with_q(k, 2, 6, qfn)["ties"]["rerank"] == 0


@pytest.mark.parametrize("offset,flag", [(0.0, True), (5e-7, True), (-5e-7, True), (2e-6, False), (-2e-6, False)])
def test_uniform_chooser_accept_window(offset, flag):
    U = np.full((1, 3), 0.4 + offset)
    ch = oaccept.UniformChooser(U, 2)
    acc = ch.accept(0, 0, 0.4)
    assert acc == (0.4 + offset < 0.4)
    assert (ch.ties == 1) == flag


@pytest.mark.parametrize("x,flag,token", [(0.25, True, 1), (0.25 + 2e-7, True, 1), (0.25 - 2e-7, True, 0),
                                          (0.26, False, 1), (0.24, False, 0), (0.999, False, 3)])
def test_uniform_chooser_draw_window(x, flag, token):
    """Inverse CDF over P = (1, 1, 1, 1) / 4 * 2 (total 2): boundaries at u = 0.25, 0.5, 0.75."""
    P = np.full(4, 0.5)
    U = np.array([[0.0, 0.0, x]])
    ch = oaccept.UniformChooser(U, 2)
    assert ch.draw(0, P) == token
    assert (ch.ties == 1) == flag


def test_nucleus_flag_window():
    """A nucleus target that lands on a cumulative mass boundary is flagged; one mid-token is not."""
    z = np.log(np.array([4.0, 3.0, 2.0, 1.0])).astype(np.float32)   # masses 0.4, 0.3, 0.2, 0.1 of 1
    t = owarp.scaled_logits(z, 1.0).astype(np.float64)
    e = np.exp(t - t.max())
    c = np.cumsum(e) / e.sum()
    w = owarp.warp_support(z, 1.0, 0, float(c[1]), 1)   # top_p exactly at the 2-token mass
    assert w["tie"] and w["n"] == 2
    w = owarp.warp_support(z, 1.0, 0, float(0.5 * (c[1] + c[2])), 1)
    assert not w["tie"] and w["n"] == 3
