"""Pins of the post-accept commit oracle (oracle/commit.py).

* The committed context reproduces what the verify pass gave the accepted
  leaf: the leaf's attention over (prefix + tree under its ancestor mask)
  equals its attention over the committed prefix alone (hubwiz section 5:
  each root-to-leaf path is scored as an independent sequence, and the loop
  continues from the longer context).
* Closed-form invariants: rows before L and after L + a are untouched, the
  appended rows are the tree rows of the path, the length grows by a + 1.
"""
import numpy as np
import pytest

from oracle import attention, commit, mask


def _tree(rng, N, D):
    """A random flattened tree: parents precede children, depth <= D."""
    parent = [-1]
    depth = [0]
    for i in range(1, N):
        cands = [j for j in range(i) if depth[j] < D]
        p = int(rng.choice(cands))
        parent.append(p)
        depth.append(depth[p] + 1)
    return np.array(parent), np.array(depth)


def _path_to(parent, leaf):
    path = []
    u = leaf
    while u != 0:
        path.append(u)
        u = parent[u]
    return path[::-1]


@pytest.mark.parametrize("seed", range(6))
def test_committed_context_is_the_accepted_sequence(seed):
    """After the commit, the accepted path is an ordinary causal sequence: a
    textbook causal attention over (prefix + committed rows), with each
    committed row's query, reproduces the tree attention that the verify pass
    gave the path's nodes (every root-to-leaf path is scored as a sequence of
    its own).  Causality makes this order-sensitive, so a dropped root, a
    reversed path or a shifted slot fails it; the tree positions (prefix
    length + depth) of the committed nodes must also equal their cache slots."""
    rng = np.random.default_rng(100 + seed)
    N, D, hq, hkv, dh, L, Lmax = 12, 4, 4, 2, 8, 7, 40
    parent, depth = _tree(rng, N, D)
    leaf = int(rng.integers(0, N))
    path = _path_to(parent, leaf)
    a = len(path)
    acc_path = np.zeros(D, np.int32)
    acc_path[:a] = path
    kp = rng.standard_normal((hkv, Lmax, dh))
    vp = rng.standard_normal((hkv, Lmax, dh))
    kt = rng.standard_normal((N, hkv, dh))
    vt = rng.standard_normal((N, hkv, dh))
    x = rng.standard_normal((N, 16))
    q = rng.standard_normal((N, hq, dh))
    q_prefix = rng.standard_normal((L, hq, dh))
    scale = 0.3
    ref = attention.tree_attention(q, kp, vp, L, kt, vt, mask.ancestor_mask(parent), scale)
    kp2, vp2, L2, feat, flags = commit.commit(kp, vp, L, kt, vt, x, a, acc_path, D)
    assert not flags and L2 == L + a + 1
    rows = [0] + path
    np.testing.assert_array_equal(mask.positions(depth, L)[rows], np.arange(L, L2))
    G = hq // hkv
    for h in range(hq):
        qs = np.concatenate([q_prefix[:, h], q[rows, h]], axis=0)
        got = attention.causal_attention(qs, kp2[h // G, :L2], vp2[h // G, :L2], scale)
        np.testing.assert_allclose(got[L:], ref[rows, h], rtol=1e-12, atol=1e-12)
    # features: root then the path, zero after
    np.testing.assert_array_equal(feat[:a + 1], x[rows])
    assert not feat[a + 1:].any()


def test_commit_invariants():
    rng = np.random.default_rng(7)
    N, D, hkv, dh, L, Lmax = 9, 5, 3, 4, 10, 20
    kp = rng.standard_normal((hkv, Lmax, dh))
    vp = rng.standard_normal((hkv, Lmax, dh))
    kt = rng.standard_normal((N, hkv, dh))
    vt = rng.standard_normal((N, hkv, dh))
    x = rng.standard_normal((N, 6))
    path = np.array([3, 5, 8, 0, 0], np.int32)
    kp2, vp2, L2, feat, flags = commit.commit(kp, vp, L, kt, vt, x, 3, path, D)
    assert not flags and L2 == L + 4
    np.testing.assert_array_equal(kp2[:, :L], kp[:, :L])
    np.testing.assert_array_equal(kp2[:, L + 4:], kp[:, L + 4:])
    for r, node in enumerate([0, 3, 5, 8]):
        np.testing.assert_array_equal(kp2[:, L + r], kt[node])
        np.testing.assert_array_equal(vp2[:, L + r], vt[node])
    # nothing accepted: the root alone
    kp3, _, L3, feat3, _ = commit.commit(kp, vp, L, kt, vt, x, 0, path, D)
    assert L3 == L + 1 and np.array_equal(kp3[:, L], kt[0]) and not feat3[1:].any()


def test_commit_edge_cases():
    rng = np.random.default_rng(8)
    N, D, hkv, dh = 6, 3, 1, 2
    kp = rng.standard_normal((hkv, 5, dh))
    kt = rng.standard_normal((N, hkv, dh))
    x = rng.standard_normal((N, 3))
    path = np.array([1, 2, 3], np.int32)
    # no room for 4 more rows at L = 2 of 5: prefix kept, features still written
    kp2, _, L2, feat, flags = commit.commit(kp, kp, 2, kt, kt, x, 3, path, D)
    assert flags == {"cache_full"} and L2 == 2 and np.array_equal(kp2, kp) and np.array_equal(feat[3], x[3])
    # a node outside [1, N) or a length past depth commits nothing
    for a, p in ((2, np.array([1, 6, 0], np.int32)), (4, path), (-1, path), (1, np.array([0, 1, 2], np.int32))):
        kp2, _, L2, feat, flags = commit.commit(kp, kp, 0, kt, kt, x, a, p, D)
        assert flags == {"bad_path"} and L2 == 0 and np.array_equal(kp2, kp) and not feat.any()
