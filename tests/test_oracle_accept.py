"""Pins of the oracle's acceptance walk.

* Losslessness (EAGLE-1 notes, background A3 and section 3.3; hubwiz section
  2): by exact enumeration on a tiny vocabulary, the committed tokens of a
  round, extended by target sampling, follow the target's own law.
* k = 1 chain: one-step acceptance probability is sum_x min(p, q) = 1 - TV.
* Greedy (EAGLE-1 notes, A.1): committed tokens are the target's greedy
  continuation, as far as the tree holds it, plus one.
* Commit bounds (hubwiz section 1): 1 <= committed <= accepted + 1 <= D + 1.
* Planted mistakes in the oracle (on the CPU) must break the losslessness pin.
"""
import numpy as np
import pytest

from oracle import accept, expand
from oracle import enumerate as en
from oracle import round as oround

CASES = [(4, 2, 2, 6), (4, 2, 2, 3), (4, 2, 2, 2), (4, 1, 3, 3), (3, 2, 3, 10), (3, 2, 3, 4), (3, 2, 3, 2)]


@pytest.mark.parametrize("V,k,D,m", CASES)
@pytest.mark.parametrize("seed", [3, 11])
def test_round_is_lossless(V, k, D, m, seed):
    p, q = en.random_path_laws(V, seed)
    law = en.round_law(V, k, D, m, 0, p, q)
    tgt = en.target_law(V, D, 0, p)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    assert en.law_distance(law, tgt) < 1e-13


def _lossless_error(monkeypatch_target=None, V=4, k=2, D=2, m=3, seed=3):
    p, q = en.random_path_laws(V, seed, zero_frac=0.0)
    return en.law_distance(en.round_law(V, k, D, m, 0, p, q), en.target_law(V, D, 0, p))


def test_planted_no_residual_breaks_losslessness(monkeypatch):
    monkeypatch.setattr(accept, "residual", lambda P, Q: P)
    assert _lossless_error() > 1e-3


def test_planted_with_replacement_breaks_losslessness(monkeypatch):
    monkeypatch.setattr(accept, "remove_candidate", lambda Q, x: Q)
    assert _lossless_error() > 1e-3


def test_planted_in_tree_only_candidates_breaks_losslessness(monkeypatch):
    orig = accept.candidates
    monkeypatch.setattr(accept, "candidates",
                        lambda pt, pf, s, k: [c for c in orig(pt, pf, s, k) if c[2] >= 0])
    assert _lossless_error(m=2) > 1e-3


def test_planted_deterministic_topk_children_breaks_losslessness(monkeypatch):
    orig = en.pl_prob

    def topk_only(q, toks):
        best = tuple(sorted(range(len(q)), key=lambda v: (-q[v], v))[: len(toks)])
        return 1.0 if tuple(toks) == best else 0.0
    monkeypatch.setattr(en, "pl_prob", topk_only)
    assert _lossless_error(m=6) > 1e-3
    monkeypatch.setattr(en, "pl_prob", orig)


@pytest.mark.parametrize("seed", range(6))
def test_single_candidate_acceptance_is_one_minus_tv(seed):
    V = 5
    p, q = en.random_path_laws(V, seed)
    acc = 0.0
    for pt, tree, spaths in en.enumerate_trees(V, 1, 1, 1, 0, q):
        npaths = en.node_paths(tree)
        for pw, com in en.enumerate_walk(tree, 1, lambda u: p(npaths[u]), lambda s: q(spaths[s])):
            if len(com) == 2 and tree["pool_flat"][0, 0] == 1 and com[0] == tree["node_tok"][1]:
                acc += pt * pw
    pr, qr = p((0,)), q((0,))
    tv = 0.5 * np.abs(pr - qr).sum()
    assert abs(acc - (1.0 - tv)) < 1e-14


def test_greedy_walk_is_greedy_decoding():
    rng = np.random.default_rng(7)
    V, k, D, m = 6, 2, 4, 12
    for trial in range(40):
        p, q = en.random_path_laws(V, 100 + trial, zero_frac=0.0)

        def fn(s, path):
            qq = q(tuple(path))
            toks = np.array(sorted(range(V), key=lambda v: (-qq[v], v))[:k])
            return toks, qq[toks].astype(np.float32)
        tree = expand.build_tree(k, D, m, 0, fn)
        paths = en.node_paths(tree)
        path_set = set(paths)
        # greedy decoding of the target from the root
        g, seq = [], (0,)
        for _ in range(D + 1):
            y = int(np.argmax(p(seq)))
            g.append(y)
            seq = seq + (y,)
        n_in_tree = 0
        while n_in_tree < D and (0,) + tuple(g[: n_in_tree + 1]) in path_set:
            n_in_tree += 1
        _, com = accept.walk_greedy(tree, lambda u: int(np.argmax(p(paths[u]))))
        assert com == g[: n_in_tree + 1]
        assert 1 <= len(com) <= D + 1


def test_inverse_cdf_draw():
    P = np.array([0.1, 0.0, 0.25, 0.65])
    for u, exp in [(0.0, 0), (0.09, 0), (0.1, 2), (0.2, 2), (0.35, 3), (0.999, 3)]:
        ch = accept.UniformChooser(np.array([[0.0, u]]), 1)
        assert ch.draw(0, P) == exp


def test_commit_bounds_on_generated_round():
    import synth
    c = synth.get_config("mid_bf16")
    inp = synth.make_inputs(c)
    for T in c.temps:
        r = oround.run_round(inp, T)
        for b, a in enumerate(r["accept"]):
            assert 1 <= a["n_committed"] == a["accept_len"] + 1 <= c.D + 1
            path = [x for x in a["accept_path"] if x >= 0]
            par = r["expand"]["node_parent"][b]
            prev = 0
            for f in path:          # accepted nodes form a root path
                assert par[f] == prev
                prev = f
            toks = r["expand"]["node_tok"][b]
            assert list(a["committed"][: len(path)]) == [int(toks[f]) for f in path]


def test_prepass_rows_are_target_logits_on_the_path():
    """A slot's draft row minus its noise equals its node's verify row (path equivalence)."""
    import synth
    c = synth.get_config("mid_f32")
    inp = synth.make_inputs(c)
    r = oround.run_round(inp, 1.0)
    ex = r["expand"]
    checked = 0
    for b in range(c.B):
        for f in range(c.N):
            s = int(ex["node_slot"][b, f])
            if s < 0:
                continue
            z = r["logits64"][b * c.N + f]
            rebuilt = (z + np.float64(inp.sigma[b]) * inp.eps[b, s].astype(np.float64)).astype(np.float32)
            assert np.max(np.abs(rebuilt.astype(np.float64) - r["rows"][b, s])) <= 1e-6 * (1 + np.abs(z).max())
            checked += 1
    assert checked >= c.B
