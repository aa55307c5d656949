"""Pins of the synthetic EAGLE draft-head oracle (oracle/draft.py).

Each pin uses weights chosen so that the head reduces to something with a
closed form, so that a dropped term, a swapped operand or a wrong index in the
oracle fails:
* FC order and feature feed-back (EAGLE-1 notes section 3.1, EAGLE-3 notes
  inference pipeline): with the attention and MLP outputs switched off the head
  is linear, a_n = A a_{n-1} + B E[x_n], and its outputs along a path have
  the closed form sum_j A^{n-j} B E[x_j] + A^{n+1} f.
* Attention visibility and head grouping: with zero query weights the
  attention is a plain average over the visible keys; constant prefix values
  per kv head and zero tree values give L / (L + j + 1) times the head's
  constant for a node at depth j.
* MLP: with identity-like weights the MLP adds silu(g) * u elementwise, with
  silu computed from scipy's logistic function.
* The per-depth expansion with a chain (top-k 1, greedy) is greedy decoding
  with the head: each next token is the argmax of the head's row.
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import draft


def _head(rng, H=8, hq=2, hkv=1, dh=4, I=8, V=11, L=5, **over):
    w = {
        "E": rng.standard_normal((V, H)),
        "fc": rng.standard_normal((H, 2 * H)) / np.sqrt(2 * H),
        "q": rng.standard_normal((hq * dh, H)) / np.sqrt(H),
        "k": rng.standard_normal((hkv * dh, H)) / np.sqrt(H),
        "v": rng.standard_normal((hkv * dh, H)) / np.sqrt(H),
        "o": rng.standard_normal((H, hq * dh)) / np.sqrt(hq * dh),
        "g": rng.standard_normal((I, H)) / np.sqrt(H),
        "u": rng.standard_normal((I, H)) / np.sqrt(H),
        "d": rng.standard_normal((H, I)) / np.sqrt(I),
    }
    w.update(over)
    lm = rng.standard_normal((V, H))
    kp = rng.standard_normal((hkv, L + 3, dh))
    vp = rng.standard_normal((hkv, L + 3, dh))
    return w, lm, kp, vp


@pytest.mark.parametrize("seed", range(4))
def test_linear_head_closed_form(seed):
    rng = np.random.default_rng(seed)
    H = 8
    A = rng.standard_normal((H, H)) * 0.4
    Bm = rng.standard_normal((H, H)) * 0.4
    w, lm, kp, vp = _head(rng, H=H, fc=np.concatenate([A, Bm], axis=1), o=np.zeros((H, 8)), d=np.zeros((H, 8)))
    head = draft.DraftHead(w, 2, 1, 4, lm, kp, vp, 5)
    f = rng.standard_normal(H)
    path = [int(t) for t in rng.integers(0, 11, size=5)]
    outs = head.path_outputs(f, path)[0]
    for n in range(len(path)):
        want = np.linalg.matrix_power(A, n + 1) @ f
        for j in range(n + 1):
            want = want + np.linalg.matrix_power(A, n - j) @ Bm @ w["E"][path[j]]
        np.testing.assert_allclose(outs[n], want, rtol=1e-12, atol=1e-12)
    # the row is the LM head on the last output
    np.testing.assert_allclose(head.row(f, path), (lm @ outs[-1]).astype(np.float32), rtol=1e-6)


@pytest.mark.parametrize("seed", range(4))
def test_attention_visibility_and_grouping(seed):
    rng = np.random.default_rng(seed)
    H, hq, hkv, dh, L = 8, 4, 2, 2, 6           # hq * dh == H; two query heads per kv head
    vp = np.empty((hkv, L + 2, dh))
    for g in range(hkv):
        vp[g] = g + 1.0
    vp[:, L:] = 1e6                             # past the prefix length: never visible
    w, lm, kp, _ = _head(rng, H=H, hq=hq, hkv=hkv, dh=dh, L=L, q=np.zeros((hq * dh, H)),
                         v=np.zeros((hkv * dh, H)), o=np.eye(H), d=np.zeros((H, 8)))
    head = draft.DraftHead(w, hq, hkv, dh, lm, kp, vp, L)
    f = rng.standard_normal(H)
    path = [int(t) for t in rng.integers(0, 11, size=4)]
    outs = head.path_outputs(f, path)[0]
    fin = f
    for j, x in enumerate(path):
        u = w["fc"] @ np.concatenate([fin, w["E"][x]])
        head_const = np.repeat(np.arange(hq) // (hq // hkv) + 1.0, dh)   # query head h reads kv head h // 2
        np.testing.assert_allclose(outs[j] - u, head_const * L / (L + j + 1), rtol=1e-12)
        fin = outs[j]


def test_mlp_identity_weights():
    rng = np.random.default_rng(7)
    H = 8
    w, lm, kp, vp = _head(rng, H=H, I=H, o=np.zeros((H, 8)), g=np.eye(H), u=2 * np.eye(H), d=np.eye(H))
    head = draft.DraftHead(w, 2, 1, 4, lm, kp, vp, 5)
    f = rng.standard_normal(H)
    a = head.path_outputs(f, [3])[0][0]
    u = w["fc"] @ np.concatenate([f, w["E"][3]])
    n2 = u / np.sqrt(np.mean(u * u) + 1e-6)
    np.testing.assert_allclose(a, u + n2 * expit(n2) * (2 * n2), rtol=1e-12)


def test_rms_values():
    x = np.array([3.0, 4.0])
    np.testing.assert_allclose(draft.rms(x), x / np.sqrt(12.5 + 1e-6), rtol=1e-15)
    np.testing.assert_allclose(draft.rms(5 * x), draft.rms(x), rtol=1e-6)


def test_bf16_rounding_grid():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 1.5 * 2 ** -8), 3.0e-3])
    got = draft._bf16(x)
    np.testing.assert_array_equal(got[:4], [1.0, 1.0 + 4 * 2 ** -8, 1.0, -(1.0 + 2 * 2 ** -8)])
    assert abs(got[4] - 3.0e-3) <= 2 ** -17        # half an ulp of the binade [2^-9, 2^-8)


@pytest.mark.parametrize("seed", range(3))
def test_chain_is_greedy_decoding(seed):
    rng = np.random.default_rng(seed)
    w, lm, kp, vp = _head(rng, V=23)
    head = draft.DraftHead(w, 2, 1, 4, lm, kp, vp, 5)
    f = rng.standard_normal(8)
    D = 5
    out = draft.expand_with_head(head, f, 4, 0.0, 1, D, D)
    toks = [4]
    for _ in range(D):
        toks.append(int(np.argmax(lm @ head.path_outputs(f, toks)[0][-1])))
    np.testing.assert_array_equal(out["node_tok"], toks)
    np.testing.assert_array_equal(out["node_parent"], [-1] + list(range(D)))


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_tree_rows_follow_paths(T):
    """Every expanded slot's row is the head's row on that node's root path, and the
    tree is a valid EAGLE-2 tree (connected, values non-increasing down a path)."""
    rng = np.random.default_rng(11)
    w, lm, kp, vp = _head(rng, V=29)
    head = draft.DraftHead(w, 2, 1, 4, lm, kp, vp, 5)
    f = rng.standard_normal(8)
    k, D, m = 3, 4, 12
    out = draft.expand_with_head(head, f, 2, T, k, D, m, seed=5)
    S = 1 + (D - 1) * k
    for s in range(S):
        e = int(out["slot_src"][s]) if s > 0 else -1
        toks = []
        while e >= 0:
            toks.append(int(out["pool_tok"][e // k, e % k]))
            e = int(out["slot_src"][e // k]) if e // k > 0 else -1
        path = [2] + toks[::-1]
        np.testing.assert_array_equal(out["rows"][s], head.row(f, path))
    par, val = out["node_parent"], out["node_value"]
    for i in range(1, m + 1):
        assert 0 <= par[i] < i and val[i] <= val[par[i]]


def test_bf16_activations_stay_close():
    rng = np.random.default_rng(3)
    w, lm, kp, vp = _head(rng, H=64, hq=4, hkv=2, dh=16, I=128, V=50)
    f = rng.standard_normal(64)
    path = [1, 7, 9, 30]
    z = draft.DraftHead(w, 4, 2, 16, lm, kp, vp, 5).row(f, path)
    zb = draft.DraftHead(w, 4, 2, 16, lm, kp, vp, 5, act="bf16").row(f, path)
    assert np.max(np.abs(z - zb)) <= 2e-2 * np.max(np.abs(z))
    assert np.max(np.abs(z - zb)) > 0
