"""Acceptance walk down the verified tree (the oracle's steps O10-O11).

Sources:
* EAGLE-1 notes, background section A3: a draft token x is accepted with
  probability min(1, p(x)/q(x)); on rejection a token is resampled from
  norm(max(0, p - q)); this equals sampling from the target.
* EAGLE-1 notes, section 3.3 and appendix A.2: with a tree, speculative
  sampling is applied recursively at every node; after a rejection the next of
  the node's k candidates is tried against the adjusted distribution, and only
  when all k are rejected is a token drawn from the adjusted distribution.
* hubwiz section 1: if every draft token is accepted a bonus token is drawn
  from the target; each verify pass commits at least one token and at most the
  accepted draft tokens plus one.  Greedy decoding (EAGLE-1 notes, A.1)
  accepts a child exactly when it is the target argmax.

Readings:
* Candidates are a node's k sampled children in sampling order, including
  children the rerank pruned.  Accepting a pruned child commits it and ends the
  round (it has no verify row).
* After rejecting x_j: P <- norm(max(0, P - Q)) with the Q that x_j was drawn
  from, then Q(x_j) <- 0 and Q <- Q / sum(Q) (draws are without replacement).
  If Q(x) is 0 the ratio is +inf when P(x) > 0 and 0 otherwise; if the
  residual mass is 0, P is left unchanged.
* Draws: trial j at node u uses U[u, j]; the final draw (resample or bonus)
  uses U[u, k] by inverse CDF in token-id order: the first token whose
  cumulative mass exceeds U * total.
"""
from __future__ import annotations

import numpy as np

from .expand import softmax

TIE_ABS = 1e-6  # |u - min(1, ratio)| and inverse-CDF boundary window (relative to total)


class UniformChooser:
    """Takes the walk's random decisions from a table of uniforms U[N, k+1]."""

    def __init__(self, U, k):
        self.U = np.asarray(U, np.float64)
        self.k = k
        self.ties = 0

    def accept(self, u, j, prob):
        x = self.U[u, j]
        if abs(x - prob) < TIE_ABS:
            self.ties += 1
        return x < prob

    def draw(self, u, P):
        c = np.cumsum(P)
        tot = c[-1]
        x = self.U[u, self.k] * tot
        y = int(np.searchsorted(c, x, side="right"))
        y = min(y, P.shape[0] - 1)
        lo = c[y - 1] if y > 0 else 0.0
        if (x - lo) < TIE_ABS * tot or (c[y] - x) < TIE_ABS * tot:
            self.ties += 1
        return y


def _children(node_parent, u):
    return [int(c) for c in np.nonzero(np.asarray(node_parent) == u)[0]]


def candidates(pool_tok, pool_flat, slot, k):
    """The sampled children of `slot` in sampling order: (j, token, flat index or -1).

    A dynamic tree's slot has k of them; a static tree's slot has its own
    count k_s <= k, and its pool row is -1 past them (the list ends there)."""
    out = []
    for j in range(k):
        x = int(pool_tok[slot, j])
        if x < 0:
            break
        out.append((j, x, int(pool_flat[slot, j])))
    return out


def ratio(P, Q, x):
    """P(x) / Q(x); +inf if Q(x) = 0 < P(x), and 0 if both are 0."""
    if Q[x] > 0:
        return P[x] / Q[x]
    return np.inf if P[x] > 0 else 0.0


def residual(P, Q):
    """norm(max(0, P - Q)); P is kept if the residual mass is 0."""
    r = np.maximum(0.0, P - Q)
    z = r.sum()
    return r / z if z > 0 else P


def remove_candidate(Q, x):
    """Draw without replacement: Q(x) <- 0, then renormalise."""
    Q = Q.copy()
    Q[x] = 0.0
    s = Q.sum()
    return Q / s if s > 0 else Q


def walk(tree, k, p_fn, q_fn, chooser):
    """Multi-round speculative sampling from the root down the tree.

    tree: dict with node_slot [N], pool_tok [S, k], pool_flat [S, k].
    p_fn(u) -> target distribution at flat node u (fp64 [V]).
    q_fn(slot) -> draft distribution of expanded slot (fp64 [V]).
    Returns (accepted flat nodes, committed tokens).
    """
    node_slot = tree["node_slot"]
    pool_tok = tree["pool_tok"]
    pool_flat = tree["pool_flat"]
    path, committed = [], []
    u = 0
    while True:
        slot = int(node_slot[u])
        p = p_fn(u)
        if slot < 0:                      # leaf: bonus token from the target
            committed.append(chooser.draw(u, p))
            return path, committed
        P = np.array(p, np.float64)
        Q = np.array(q_fn(slot), np.float64)
        acc = None
        for j, x, f in candidates(pool_tok, pool_flat, slot, k):
            if chooser.accept(u, j, min(1.0, ratio(P, Q, x))):
                acc = (x, f)
                break
            P = residual(P, Q)
            Q = remove_candidate(Q, x)
        if acc is None:                   # all k rejected: draw from the residual
            committed.append(chooser.draw(u, P))
            return path, committed
        x, f = acc
        committed.append(x)
        if f < 0:                         # accepted a pruned candidate: no verify row
            return path, committed
        path.append(f)
        u = f


def walk_greedy(tree, argmax_fn):
    """Greedy verification: follow the child whose token is the target argmax."""
    node_tok = tree["node_tok"]
    node_parent = tree["node_parent"]
    path, committed = [], []
    u = 0
    while True:
        y = int(argmax_fn(u))
        committed.append(y)
        nxt = [c for c in _children(node_parent, u) if int(node_tok[c]) == y]
        if not nxt:
            return path, committed
        u = nxt[0]
        path.append(u)


def _pack(path, committed, D):
    ap = np.full(D, -1, np.int64)
    ap[: len(path)] = path
    cm = np.full(D + 1, -1, np.int64)
    cm[: len(committed)] = committed
    return len(path), ap, cm, len(committed)


def accept_request(tree, target_logits, draft_rows, T, k, D, U=None, target_argmax=None, warp=None):
    """Acceptance for one request.

    target_logits [N, V] fp32 (row u = verify logits at flat node u);
    draft_rows [S, V] fp32; U [N, k+1] uniforms (T > 0).
    warp = (top_k, top_p) (T > 0 only): both distributions are warped the same
    way before the walk (oracle/warp.py, at least k tokens kept).
    Returns dict(accept_len, accept_path[D], committed[D+1], n_committed, ties).
    """
    if T > 0:
        ch = UniformChooser(U, k)
        if warp is None:
            p_fn = lambda u: softmax(target_logits[u], T)  # noqa: E731
            q_fn = lambda s: softmax(draft_rows[s], T)  # noqa: E731
        else:
            from .warp import warped_softmax
            p_fn = lambda u: warped_softmax(target_logits[u], T, warp[0], warp[1], k)  # noqa: E731
            q_fn = lambda s: warped_softmax(draft_rows[s], T, warp[0], warp[1], k)  # noqa: E731
        path, com = walk(tree, k, p_fn, q_fn, ch)
        ties = ch.ties
    else:
        if target_argmax is None:
            target_argmax = np.argmax(np.asarray(target_logits, np.float32), axis=1)
        path, com = walk_greedy(tree, lambda u: target_argmax[u])
        ties = 0
    al, ap, cm, nc = _pack(path, com, D)
    return dict(accept_len=al, accept_path=ap, committed=cm, n_committed=nc, ties=ties)
