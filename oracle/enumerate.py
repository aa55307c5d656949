"""Exact enumeration of one round on a tiny vocabulary (losslessness check).

Every random choice of a round is replaced by exact branching with its
probability: the ordered k children of each expanded node are drawn without
replacement from the draft distribution (the Plackett-Luce law that the
Gumbel-top-k keys realise), each acceptance test branches on accept/reject,
and each resample or bonus draw branches over the tokens of its distribution.
The enumeration replays the oracle's own `build_tree` and `walk` with a
chooser that records the branch taken, so it checks exactly the code the
oracle runs.

Each committed sequence is then extended to D+1 tokens by sampling the target,
giving the round's joint law of the next D+1 tokens.  Speculative sampling
leaves the output distribution unchanged (EAGLE-1 notes, background section A3;
hubwiz section 2), so this joint must equal the target's own law
prod_i p(c_i | root, c_1..c_{i-1}).
"""
from __future__ import annotations

import itertools
from collections import defaultdict

import numpy as np

from .accept import walk
from .expand import build_tree


class _Need(Exception):
    pass


def pl_prob(q, toks):
    """Probability of drawing the ordered tuple `toks` without replacement from q."""
    p, rem = 1.0, 1.0
    for t in toks:
        if rem <= 0.0:
            return 0.0
        p *= q[t] / rem
        rem -= q[t]
    return p


def enumerate_trees(V, k, D, m, root, q_path):
    """All (probability, tree, slot_paths) outcomes of the expansion."""
    out = []

    def rec(choices):
        calls = []
        prob = [1.0]
        slot_paths = {}

        def children_fn(s, path):
            q = q_path(tuple(path))
            i = len(calls)
            if i >= len(choices):
                raise _Need(q)
            toks = choices[i]
            calls.append(toks)
            slot_paths[s] = tuple(path)
            prob[0] *= pl_prob(q, toks)
            return np.array(toks), np.asarray(q, np.float64)[list(toks)].astype(np.float32)

        try:
            tree = build_tree(k, D, m, root, children_fn)
        except _Need as e:
            q = e.args[0]
            for toks in itertools.permutations(range(V), k):
                if pl_prob(q, toks) > 0.0:
                    rec(choices + [toks])
            return
        out.append((prob[0], tree, dict(slot_paths)))

    rec([])
    return out


def enumerate_static_trees(V, parent, root, q_path):
    """All (probability, tree, slot_paths) outcomes of filling a static shape."""
    from .static_tree import build_static_tree
    out = []

    def rec(choices):
        calls = []
        prob = [1.0]
        slot_paths = {}

        def children_fn(s, path, kk):
            q = q_path(tuple(path))
            i = len(calls)
            if i >= len(choices):
                raise _Need((q, kk))
            toks = choices[i]
            calls.append(toks)
            slot_paths[s] = tuple(path)
            prob[0] *= pl_prob(q, toks)
            return np.array(toks), np.asarray(q, np.float64)[list(toks)].astype(np.float32)

        try:
            tree = build_static_tree(parent, root, children_fn)
        except _Need as e:
            q, kk = e.args[0]
            for toks in itertools.permutations(range(V), kk):
                if pl_prob(q, toks) > 0.0:
                    rec(choices + [toks])
            return
        out.append((prob[0], tree, dict(slot_paths)))

    rec([])
    return out


class _EnumChooser:
    def __init__(self, decisions):
        self.dec = decisions
        self.i = 0
        self.prob = 1.0

    def accept(self, u, j, prob):
        if self.i >= len(self.dec):
            raise _Need(("b", prob))
        d = self.dec[self.i]
        self.i += 1
        self.prob *= prob if d else (1.0 - prob)
        return d

    def draw(self, u, P):
        P = np.asarray(P, np.float64)
        if self.i >= len(self.dec):
            raise _Need(("c", P))
        y = self.dec[self.i]
        self.i += 1
        self.prob *= P[y] / P.sum()
        return y


def enumerate_walk(tree, k, p_fn, q_fn, walk_fn=walk):
    """All (probability, committed tokens) outcomes of the acceptance walk."""
    out = []

    def rec(dec):
        ch = _EnumChooser(dec)
        try:
            _, com = walk_fn(tree, k, p_fn, q_fn, ch)
        except _Need as e:
            kind, val = e.args[0]
            if kind == "b":
                if val > 0.0:
                    rec(dec + [True])
                if val < 1.0:
                    rec(dec + [False])
            else:
                for y in np.nonzero(val > 0.0)[0]:
                    rec(dec + [int(y)])
            return
        out.append((ch.prob, list(com)))

    rec([])
    return out


def node_paths(tree):
    """Token path (root first) of every flat node."""
    par, tok = tree["node_parent"], tree["node_tok"]
    paths = []
    for u in range(len(par)):
        seq = []
        j = u
        while j >= 0:
            seq.append(int(tok[j]))
            j = int(par[j])
        paths.append(tuple(seq[::-1]))
    return paths


def round_law(V, k, D, m, root, p_path, q_path, walk_fn=walk, static_parent=None):
    """Joint law of the next D+1 tokens produced by one round plus target sampling.

    static_parent: a static shape (oracle/static_tree.py) instead of the
    dynamic tree (then k is the shape's largest child count and D its depth)."""
    joint = defaultdict(float)

    def extend(seq, w):
        if len(seq) == D + 1:
            joint[tuple(seq)] += w
            return
        p = p_path((root,) + tuple(seq))
        for y in range(V):
            if p[y] > 0.0:
                extend(seq + [y], w * p[y])

    trees = (enumerate_trees(V, k, D, m, root, q_path) if static_parent is None
             else enumerate_static_trees(V, static_parent, root, q_path))
    for pt, tree, spaths in trees:
        npaths = node_paths(tree)
        for pw, com in enumerate_walk(tree, k, lambda u: p_path(npaths[u]),
                                      lambda s: q_path(spaths[s]), walk_fn):
            assert 1 <= len(com) <= D + 1
            extend(com, pt * pw)
    return dict(joint)


def target_law(V, D, root, p_path):
    """prod_i p(c_i | root, c_<i) over all sequences of D+1 tokens."""
    out = {}
    for seq in itertools.product(range(V), repeat=D + 1):
        w = 1.0
        for i in range(D + 1):
            w *= p_path((root,) + seq[:i])[seq[i]]
            if w == 0.0:
                break
        if w > 0.0:
            out[seq] = w
    return out


def law_distance(a, b):
    """max |a(s) - b(s)| over all sequences."""
    keys = set(a) | set(b)
    return max(abs(a.get(s, 0.0) - b.get(s, 0.0)) for s in keys)


def random_path_laws(V, seed, zero_frac=0.25):
    """Deterministic p_path / q_path functions of the token path, for tests.

    Each distribution is a Dirichlet(1) draw keyed by (seed, path); with
    probability zero_frac one entry is set to 0 (exercising p(x) = 0 and
    q(x) = 0 cases) and the rest renormalised.
    """
    cache = {}

    def law(which, path):
        key = (which, path)
        if key not in cache:
            ss = np.random.SeedSequence(entropy=seed, spawn_key=(which,) + tuple(int(t) + 1 for t in path))
            rng = np.random.default_rng(ss)
            d = rng.dirichlet(np.ones(V))
            if rng.random() < zero_frac:
                d[rng.integers(V)] = 0.0
                d = d / d.sum()
            cache[key] = d
        return cache[key]

    return (lambda path: law(0, path)), (lambda path: law(1, path))
