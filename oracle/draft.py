"""Synthetic EAGLE draft head and per-depth tree expansion with it.

TEST INFRASTRUCTURE ONLY (see the package docstring): fp64 numpy, no code
shared with the HIP path.

EAGLE-1 notes, section 3.1: the draft model is the target's embedding layer and
LM head around an autoregression head.  The head concatenates the feature
sequence with the embeddings of the tokens one step ahead (2 x hidden), an FC
layer maps that back to hidden, and one decoder layer predicts the next
feature; the LM head turns the predicted feature into the distribution the
next token is drawn from, and the predicted feature and the drawn token are
fed back in.  EAGLE-3 notes, inference pipeline: where the target's feature of
a drafted token does not exist yet, the draft head's own output takes its
place.  EAGLE-2 notes, "Expanding the Draft Tree": the tree grows one depth
per draft forward, the k best nodes of the newest layer being expanded.

Readings (the pages name the parts, not their internals):
* Decoder layer (Llama style, unit RMSNorm gains, SwiGLU MLP):
    u  = W_fc [f ; E[x]]
    h  = u + W_o attn(rms(u))
    a  = h + W_d (silu(W_g rms(h)) * (W_u rms(h)))
  rms(x) = x / sqrt(mean(x^2) + 1e-6).  Attention: q/k/v = W_q/W_k/W_v rms(u)
  per head, grouped-query heads, score scale 1/sqrt(dh), no positional
  rotation (as in the verify layer); a node attends to the draft's prefix
  K/V of its request and to the K/V of every node on its own root path,
  itself included.
* The node expanded as slot 0 is the root: f is the given feature of the
  position before it, x the root token.  Every other expanded node takes f =
  the head's output a at its parent and x = its own token.  Its draft row is
  the shared LM head on a: z = W a.
* act="bf16": every matmul input (the concatenated [f ; E[x]], rms outputs,
  q/k/v, the attention output, the MLP product, and a before the LM head and
  before it is fed back) is rounded to bf16, as a bf16 activation pipeline
  stores them; the arithmetic stays fp64.  act=None: fp64 throughout.
"""
from __future__ import annotations

import numpy as np

from . import attention, expand

EPS = 1e-6


def _bf16(x):
    """Round to the nearest bf16 value (ties to even), through fp32."""
    u = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def rms(x):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + EPS)


def silu(x):
    return x / (1.0 + np.exp(-x))


class DraftHead:
    """The draft head of one request.

    w: dict of weights (any float dtype): E [V, H], fc [H, 2H], q [hq*dh, H],
    k [hkv*dh, H], v [hkv*dh, H], o [H, hq*dh], g [I, H], u [I, H], d [H, I];
    lm: the shared LM-head weight [V, H]; kp, vp: the draft's prefix K/V of the
    request, [hkv, >= L, dh]; L its length."""

    def __init__(self, w, hq, hkv, dh, lm, kp, vp, L, act=None):
        self.w = {k: np.asarray(v, np.float64) for k, v in w.items() if k != "E"}
        self.E = w["E"]
        self.hq, self.hkv, self.dh = hq, hkv, dh
        self.lm = lm
        self.kp, self.vp, self.L = kp, vp, int(L)
        self.act = act
        self._cache = {}

    def _r(self, x):
        return _bf16(x) if self.act == "bf16" else np.asarray(x, np.float64)

    def step(self, f, x, path_k, path_v):
        """One node: feature f [H], token x; path_k/v: K/V [hkv, dh] of the nodes
        above it on its root path, root first.  Returns (a, k, v)."""
        w = self.w
        u = w["fc"] @ self._r(np.concatenate([np.asarray(f, np.float64), np.asarray(self.E[int(x)], np.float64)]))
        n1 = self._r(rms(u))
        q = self._r(w["q"] @ n1).reshape(1, self.hq, self.dh)
        k = self._r(w["k"] @ n1).reshape(self.hkv, self.dh)
        v = self._r(w["v"] @ n1).reshape(self.hkv, self.dh)
        kt = np.stack(list(path_k) + [k])[None] if path_k else k[None, None]
        vt = np.stack(list(path_v) + [v])[None] if path_v else v[None, None]
        kt, vt = kt[0], vt[0]                               # [j + 1, hkv, dh]
        n = kt.shape[0]
        o = attention.tree_attention(np.repeat(q, n, axis=0), self.kp, self.vp, self.L, kt, vt,
                                     np.ones((n, n), bool), 1.0 / np.sqrt(self.dh))[-1]
        h = u + w["o"] @ self._r(o.reshape(-1))
        n2 = self._r(rms(h))
        a = h + w["d"] @ self._r(silu(w["g"] @ n2) * (w["u"] @ n2))
        return a, k, v

    def path_outputs(self, f_root, path):
        """The head's output a at every node of a root path of tokens (root
        first), run causally: node j attends to the prefix and nodes 0..j."""
        key = tuple(int(t) for t in path)
        if key in self._cache:
            return self._cache[key]
        if len(path) > 1:
            outs, ks, vs = self.path_outputs(f_root, path[:-1])
            f = self._r(outs[-1])
        else:
            outs, ks, vs = [], [], []
            f = self._r(f_root)
        a, k, v = self.step(f, path[-1], ks, vs)
        res = (outs + [a], ks + [k], vs + [v])
        self._cache[key] = res
        return res

    def feature(self, f_root, path):
        """Feature a at the last node of `path` (rounded as it is fed on)."""
        return self._r(self.path_outputs(f_root, path)[0][-1])

    def row(self, f_root, path, cols=None):
        """Draft logits (fp32) at the last node of `path`; cols: a subset of the vocabulary."""
        a = self.feature(f_root, path)
        W = self.lm if cols is None else self.lm[np.asarray(cols)]
        return (np.asarray(W, np.float64) @ a).astype(np.float32)


def expand_with_head(head, f_root, root, T, k, D, m, seed=0, req=0, round_id=0, warp=None):
    """EAGLE-2 expansion where the row of each expanded node is the draft head's
    row on that node's root path, computed when the node joins the frontier
    (the tree construction, child selection and rerank of oracle.expand).
    warp = (top_k, top_p) (T > 0): children are drawn from each row's warped
    distribution, as oracle.expand.children_of_row draws them."""
    S = 1 + (D - 1) * k
    rows = np.zeros((S, np.asarray(head.lm).shape[0]), np.float32)
    stats = np.zeros((S, 2), np.float64)
    ties = [0]

    def children_fn(s, path):
        rows[s] = head.row(f_root, path)
        toks, q, M, Ssum, t = expand.children_of_row(rows[s], T, k, seed, s, req, round_id, warp)
        stats[s] = (M, Ssum)
        ties[0] += t
        return toks, q

    out = expand.build_tree(k, D, m, root, children_fn)
    out["slot_stats"] = stats
    out["rows"] = rows
    out["ties"]["children"] = ties[0]
    return out
