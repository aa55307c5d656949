"""Tree-masked attention of the verify pass (the oracle's step O8).

EAGLE-1 notes, sections 3.1 and 3.3: one target forward with tree attention
scores every token of the draft tree; hubwiz section 5: each root-to-leaf path
is scored as if it were an independent sequence.  Each tree query attends to
every prefix key of its request and to the tree keys its mask row allows.

Readings: the kv head of query head h is h // (hq / hkv) (grouped-query
attention); scores are q.k * scale; the softmax and the weighted sum are
evaluated in fp64.
"""
import numpy as np


def tree_attention(q, k_prefix, v_prefix, prefix_len, k_tree, v_tree, mask, scale):
    """One request.

    q        [N, hq, dh]      queries of the tree nodes
    k_prefix [hkv, >=L, dh]   prefix keys (first L used)
    v_prefix [hkv, >=L, dh]
    k_tree   [N, hkv, dh]     keys/values of the tree nodes
    v_tree   [N, hkv, dh]
    mask     [N, N] bool      mask[i, j]: tree key j visible to query i
    Returns fp64 [N, hq, dh].
    """
    q = np.asarray(q, np.float64)
    N, hq, dh = q.shape
    hkv = k_prefix.shape[0]
    G = hq // hkv
    L = int(prefix_len)
    out = np.zeros((N, hq, dh), np.float64)
    for h in range(hq):
        g = h // G
        kp = np.asarray(k_prefix[g, :L], np.float64)
        vp = np.asarray(v_prefix[g, :L], np.float64)
        kt = np.asarray(k_tree[:, g], np.float64)
        vt = np.asarray(v_tree[:, g], np.float64)
        s = np.concatenate([q[:, h] @ kp.T, q[:, h] @ kt.T], axis=1) * float(scale)
        vis = np.concatenate([np.ones((N, L), bool), np.asarray(mask, bool)], axis=1)
        s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h] = w @ np.concatenate([vp, vt], axis=0)
    return out


def causal_attention(q, k, v, scale):
    """Textbook causal attention of a linear sequence: q, k, v [T, dh] fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T = q.shape[0]
    s = (q @ k.T) * float(scale)
    s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v
