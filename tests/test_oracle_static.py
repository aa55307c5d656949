"""Pins of the oracle's static (EAGLE-1) draft tree.

* Shape bookkeeping (EAGLE-1 notes, appendix A.1: k children per node read off
  a fixed shape, k = 4 at the root, 5 draft passes): the default shape has a
  4-child root and depth 5; slots are the nodes with children, in flat order.
* Losslessness (EAGLE-1 notes, background A3 and section 3.3; hubwiz section
  2): by exact enumeration on a tiny vocabulary, a round on a static shape,
  extended by target sampling, follows the target's own law.  A planted
  deterministic top-k child choice at T > 0 breaks it.
* A slot with k_s children takes the first k_s of the top-k_max order: the
  top-k_s keys are a prefix of the top-k_max keys (greedy and Gumbel alike).
* Greedy on a static tree is greedy decoding as far as the tree holds it.
"""
import numpy as np
import pytest

from oracle import accept, expand
from oracle import enumerate as en
from oracle import static_tree as st

SMALL_SHAPES = [
    st.parents_from_paths([(0,), (1,), (0, 0)]),             # root 2, first child 1
    st.parents_from_paths([(0,), (0, 0), (0, 1)]),           # root 1, its child 2
    st.parents_from_paths([(0,), (1,), (0, 0), (1, 0)]),     # root 2, each child 1
    st.parents_from_paths([(0,), (0, 0)]),                   # a chain of 2
]


def test_default_shape_bookkeeping():
    info = st.shape_info(st.DEFAULT_SHAPE)
    assert info["n"] == 1 + len(st.DEFAULT_PATHS)
    assert info["D"] == 5 and info["kmax"] == 4
    assert info["slot_k"][0] == 4 and info["slot_node"][0] == 0
    # depth of every node = length of its path; siblings ranked in flat order
    for i, p in enumerate(st.DEFAULT_PATHS, start=1):
        assert info["depth"][i] == len(p) and info["sib"][i] == p[-1]
    # slot s's children count = number of nodes whose parent is the slot's node
    par = st.DEFAULT_SHAPE
    for s, u in enumerate(info["slot_node"]):
        assert info["slot_k"][s] == int((par == u).sum())
        assert info["slot"][u] == s
    # the more probable branch is at least as deep and wide as its later siblings
    for u in range(info["n"]):
        kids = [c for c in range(info["n"]) if par[c] == u]
        widths = [int((par == c).sum()) for c in kids]
        assert widths == sorted(widths, reverse=True)


def test_bad_shapes_rejected():
    for bad in ([0], [-1, 1], [-1, 0, 2], [-1, -1]):
        with pytest.raises(ValueError):
            st.shape_info(np.array(bad))


@pytest.mark.parametrize("shape_i", range(len(SMALL_SHAPES)))
@pytest.mark.parametrize("V,seed", [(3, 5), (4, 7)])
def test_static_round_is_lossless(shape_i, V, seed):
    par = SMALL_SHAPES[shape_i]
    info = st.shape_info(par)
    p, q = en.random_path_laws(V, seed)
    law = en.round_law(V, info["kmax"], info["D"], info["n"] - 1, 0, p, q, static_parent=par)
    tgt = en.target_law(V, info["D"], 0, p)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    assert en.law_distance(law, tgt) < 1e-13


def test_planted_deterministic_children_break_static_losslessness(monkeypatch):
    par = SMALL_SHAPES[0]
    info = st.shape_info(par)
    p, q = en.random_path_laws(4, 3, zero_frac=0.0)

    def topk_only(qq, toks):
        best = tuple(sorted(range(len(qq)), key=lambda v: (-qq[v], v))[: len(toks)])
        return 1.0 if tuple(toks) == best else 0.0
    monkeypatch.setattr(en, "pl_prob", topk_only)
    law = en.round_law(4, info["kmax"], info["D"], info["n"] - 1, 0, p, q, static_parent=par)
    assert en.law_distance(law, en.target_law(4, info["D"], 0, p)) > 1e-3


@pytest.mark.parametrize("T", [1.0, 0.6, 0.0])
def test_slot_children_are_a_prefix_of_the_top_kmax(T):
    rng = np.random.default_rng(12)
    z = rng.standard_normal(700).astype(np.float32)
    if T == 0.0:
        z[::7] = z[0]  # exact ties decided by id
    full = expand.children_of_row(z, T, 4, seed=99, slot=3, req=1, round_id=2)[0]
    for kk in (1, 2, 3):
        part = expand.children_of_row(z, T, kk, seed=99, slot=3, req=1, round_id=2)[0]
        assert list(part) == list(full[:kk])


def test_static_tree_fill_and_pool():
    rng = np.random.default_rng(4)
    par = st.DEFAULT_SHAPE
    info = st.shape_info(par)
    rows = rng.standard_normal((info["S"], 300)).astype(np.float32)
    out = st.expand_static_request(rows, par, 17, 1.0, seed=5, req=0, round_id=1)
    for s, u in enumerate(info["slot_node"]):
        kk = int(info["slot_k"][s])
        toks = expand.children_of_row(rows[s], 1.0, kk, seed=5, slot=s, req=0, round_id=1)[0]
        assert list(out["pool_tok"][s, :kk]) == list(toks)
        assert (out["pool_tok"][s, kk:] == -1).all() and (out["pool_flat"][s, kk:] == -1).all()
        for j in range(kk):
            c = int(out["pool_flat"][s, j])
            assert par[c] == u and out["node_tok"][c] == toks[j] and out["node_sib"][c] == j
    # values: fp32 products along the path, never above the parent's
    for c in range(1, info["n"]):
        assert out["node_value"][c] == np.float32(out["node_value"][par[c]] * out["node_q"][c])
        assert out["node_value"][c] <= out["node_value"][par[c]]
    # slot_src: pool entry of the node each slot expands
    k = info["kmax"]
    for s, u in enumerate(info["slot_node"]):
        if u == 0:
            assert out["slot_src"][s] == -1
        else:
            e = int(out["slot_src"][s])
            assert out["pool_flat"][e // k, e % k] == u


def test_static_greedy_walk_is_greedy_decoding():
    V = 6
    par = st.DEFAULT_SHAPE
    info = st.shape_info(par)
    for trial in range(20):
        p, q = en.random_path_laws(V, 300 + trial, zero_frac=0.0)

        def fn(s, path, kk):
            qq = q(tuple(path))
            toks = np.array(sorted(range(V), key=lambda v: (-qq[v], v))[:kk])
            return toks, qq[toks].astype(np.float32)
        tree = st.build_static_tree(par, 0, fn)
        paths = en.node_paths(tree)
        path_set = set(paths)
        g, seq = [], (0,)
        for _ in range(info["D"] + 1):
            y = int(np.argmax(p(seq)))
            g.append(y)
            seq = seq + (y,)
        n_in = 0
        while n_in < info["D"] and (0,) + tuple(g[: n_in + 1]) in path_set:
            n_in += 1
        _, com = accept.walk_greedy(tree, lambda u: int(np.argmax(p(paths[u]))))
        assert com == g[: n_in + 1]
