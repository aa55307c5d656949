"""Pins of the oracle's mask and tree attention.

EAGLE-2 notes, "Tree Attention Mask": a token sees only its ancestors (never a
sibling branch).  hubwiz section 5: one pass scores each root-to-leaf path as
if independent, i.e. tree attention on a path equals ordinary causal attention
on prefix + path as one linear sequence.
"""
import numpy as np

from oracle import attention, expand, mask


def _random_tree(rng, k=3, D=4, m=20):
    def fn(s, path):
        return rng.choice(50, size=k, replace=False), rng.dirichlet(np.ones(50))[:k].astype(np.float32)
    return expand.build_tree(k, D, m, 1, fn)


def test_mask_is_transitive_closure_of_parent():
    rng = np.random.default_rng(0)
    for _ in range(20):
        t = _random_tree(rng)
        par = t["node_parent"]
        N = len(par)
        A = np.zeros((N, N), np.int64)
        for i in range(1, N):
            A[i, par[i]] = 1
        # reachability by repeated boolean products: I + A + A^2 + ...
        R = np.eye(N, dtype=np.int64)
        P = np.eye(N, dtype=np.int64)
        for _ in range(N):
            P = (P @ A > 0).astype(np.int64)
            R = R | P
        mb = mask.ancestor_mask(par)
        assert (mb == R.astype(bool)).all()
        # siblings never visible to each other
        for i in range(1, N):
            for j in range(1, N):
                if i != j and par[i] == par[j]:
                    assert not mb[i, j]


def test_pack_bits_round_trip():
    rng = np.random.default_rng(1)
    for N in (1, 5, 63, 64, 65, 130):
        mb = rng.random((N, N)) < 0.3
        w = mask.pack_bits(mb)
        assert w.shape == (N, (N + 63) // 64)
        back = np.zeros_like(mb)
        for i in range(N):
            for j in range(N):
                back[i, j] = (int(w[i, j // 64]) >> (j % 64)) & 1
        assert (back == mb).all()


def test_positions():
    assert list(mask.positions([0, 1, 1, 2], 100)) == [100, 101, 101, 102]


def test_tree_attention_equals_causal_attention_on_every_path():
    rng = np.random.default_rng(2)
    hq, hkv, dh, L = 4, 2, 8, 13
    t = _random_tree(rng, k=2, D=4, m=11)
    par = t["node_parent"]
    N = len(par)
    q = rng.standard_normal((N, hq, dh))
    kt = rng.standard_normal((N, hkv, dh))
    vt = rng.standard_normal((N, hkv, dh))
    kp = rng.standard_normal((hkv, L + 5, dh))
    vp = rng.standard_normal((hkv, L + 5, dh))
    scale = 0.37
    out = attention.tree_attention(q, kp, vp, L, kt, vt, mask.ancestor_mask(par), scale)
    leaves = [i for i in range(N) if i not in set(par)]
    for leaf in leaves:
        path = []
        j = leaf
        while j >= 0:
            path.append(j)
            j = int(par[j])
        path = path[::-1]
        for h in range(hq):
            g = h // (hq // hkv)
            Q = np.concatenate([np.zeros((L, dh)), q[path, h]])
            K = np.concatenate([kp[g, :L], kt[path, g]])
            Vv = np.concatenate([vp[g, :L], vt[path, g]])
            ref = attention.causal_attention(Q, K, Vv, scale)[L:]
            assert np.allclose(out[path, h], ref, rtol=1e-12, atol=1e-12)


def test_single_node_is_decode_attention():
    rng = np.random.default_rng(3)
    L, dh = 20, 16
    q = rng.standard_normal((1, 1, dh))
    kp = rng.standard_normal((1, L, dh))
    vp = rng.standard_normal((1, L, dh))
    kt = rng.standard_normal((1, 1, dh))
    vt = rng.standard_normal((1, 1, dh))
    out = attention.tree_attention(q, kp, vp, L, kt, vt, np.ones((1, 1), bool), 0.25)
    K = np.concatenate([kp[0], kt[0]])
    Vv = np.concatenate([vp[0], vt[0]])
    s = K @ q[0, 0] * 0.25
    w = np.exp(s - s.max())
    w /= w.sum()
    assert np.allclose(out[0, 0], w @ Vv, rtol=1e-13)
