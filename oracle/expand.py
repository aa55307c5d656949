"""Draft-tree expansion, rerank and flattening (the oracle's steps O2-O6).

Sources:
* EAGLE-2 notes, "Expanding the Draft Tree": the value of a draft token is the
  product of the draft confidences on its root path (the value equation), and
  only the k highest-value tokens of the current layer are expanded.
* EAGLE-2 notes, "Rerank draft tokens": all draft tokens are reranked and the
  m highest-value ones kept; a node's value never exceeds its parent's, equal
  values prefer the shallower node, so the kept set is a connected tree.
* EAGLE-2 notes, "Tree Attention Mask": the kept tokens are flattened into one
  sequence.
* EAGLE-1 notes, appendix A.1: greedy drafting takes the top-k tokens as
  children, non-greedy drafting samples k tokens.

Readings (where the pages are silent):
* Slot 0 is the root (last committed token, value 1).  Layer 1 is the root's k
  children; for d = 1..D-1 the frontier is the top-k of layer d by
  (value desc, cidx asc) and frontier rank i at depth d expands slot
  1 + (d-1)k + i.  cidx of a layer-(d+1) child is i*k + j (j = its rank among
  its parent's children); layer-1 cidx is j.  The pool is layers 1..D.
* Non-greedy children are k draws without replacement from q, realised with
  the Gumbel-top-k construction (Kool, van Hoof, Welling 2019): keys
  t_v + g_v with g = -ln(-ln u), u from Philox4x32-10; the key order is the
  sampling order.  The key is evaluated in fp64 from t_v = fp32(z_v / T).
* Confidence q = softmax(t) at T' = T (T > 0) or 1 (greedy), rounded to fp32;
  values are fp32 products V_child = fp32(V_parent * q_child).
* Rerank order (value desc, depth asc, cidx asc); flatten order
  (depth asc, parent flat index asc, sibling rank asc).
"""
from __future__ import annotations

import numpy as np

from .philox import gumbel_uniforms

# Near-tie windows: decisions whose deciding gap is below these are reported so
# that a comparison with another implementation can exclude them.
KEY_TIE_REL = 1e-12     # fp64 Gumbel keys (differences only from log rounding)
VALUE_TIE_REL = 2e-6    # fp32 values (q may differ by an ulp per level)


def scaled_logits(z, T):
    """t = fp32(z / T'), with T' = T for T > 0 and T' = 1 for greedy."""
    tp = np.float32(T if T > 0 else 1.0)
    return (np.asarray(z, dtype=np.float32) / tp).astype(np.float32)


def softmax_stats(z, T):
    """(M, S): M = max_v t_v, S = sum_v exp(t_v - M), in fp64."""
    t = scaled_logits(z, T).astype(np.float64)
    M = t.max()
    S = np.exp(t - M).sum()
    return M, S


def softmax(z, T):
    """Temperature-adjusted distribution exp(t - M) / S in fp64."""
    t = scaled_logits(z, T).astype(np.float64)
    M = t.max()
    e = np.exp(t - M)
    return e / e.sum()


def gumbel_keys(z, T, seed, slot, req, round_id):
    """fp64 keys t_v + g_v of one slot row (T > 0)."""
    t = scaled_logits(z, T).astype(np.float64)
    u = gumbel_uniforms(t.shape[0], slot, req, round_id, seed)
    w = 1.0 - u  # exact
    e = np.where(u > 0.5, -np.log1p(-w), -np.log(u))  # -ln u, full relative precision
    return t - np.log(e)


def _rel_gap(a, b):
    """Relative gap |a - b| / max(|a|, |b|) of two adjacent keys or values.

    Equal keys (infinite ones included) are a tie, gap 0; a finite key beside
    an infinite one (a token the warp drops sits at -inf) is a decided
    boundary, gap +inf.  Never NaN.
    """
    a, b = float(a), float(b)
    if a == b:
        return 0.0
    if not (np.isfinite(a) and np.isfinite(b)):
        return float("inf")
    return abs(a - b) / max(abs(a), abs(b), 1e-300)


def children_of_row(z, T, k, seed=0, slot=0, req=0, round_id=0, warp=None):
    """Children of one expanded slot: k tokens in sampling order and their q.

    Greedy (T == 0): the k largest logits ordered by (z desc, id asc).
    T > 0: the k largest Gumbel keys ordered by (key desc, id asc).
    warp = (top_k, top_p) (T > 0 only): the draws come from the warped
    distribution (oracle/warp.py, at least k tokens kept): keys outside its
    support are -inf, and q and S are those of the warped distribution.
    Returns (tokens int64[k], q float32[k], M, S, n_near_ties).
    """
    z = np.asarray(z, dtype=np.float32)
    V = z.shape[0]
    ids = np.arange(V)
    w = None
    if T > 0:
        key = gumbel_keys(z, T, seed, slot, req, round_id)
        if warp is not None:
            from .warp import warp_support
            w = warp_support(z, T, warp[0], warp[1], min_keep=k)
            key = np.where(w["mask"], key, -np.inf)
    else:
        key = z.astype(np.float64)
    order = np.lexsort((ids, -key))
    top = order[:k]
    ties = 0
    if T > 0:
        srt = key[order[: k + 1]]
        for i in range(min(k, V - 1)):
            if _rel_gap(srt[i], srt[i + 1]) < KEY_TIE_REL:
                ties += 1
    if w is not None:
        M, S = w["M"], w["S"]
        ties += int(w["tie"])
    else:
        M, S = softmax_stats(z, T)
    t = scaled_logits(z, T).astype(np.float64)
    q = (np.exp(t[top] - M) / S).astype(np.float32)
    return top.astype(np.int64), q, M, S, ties


def build_tree(k, D, m, root_token, children_fn, frontier_fn=None):
    """Expand, rerank and flatten one request's draft tree.

    children_fn(slot, path) -> (tokens[k], q_fp32[k]) gives the children of the
    node expanded as `slot`, whose root path is `path` (token list, root first).
    frontier_fn([(slot, path), ...]), if given, is told each depth's frontier
    before its children are asked for (a caller may batch work per depth).
    Returns a dict of numpy arrays (see keys below) plus near-tie counts.
    """
    S = 1 + (D - 1) * k
    P = k + (D - 1) * k * k
    if not (1 <= m <= P):
        raise ValueError("need 1 <= m <= P")
    pool_tok = np.full((S, k), -1, dtype=np.int64)
    pool_q = np.zeros((S, k), dtype=np.float32)
    pool_val = np.zeros((S, k), dtype=np.float32)
    pool_depth = np.zeros((S, k), dtype=np.int64)
    pool_cidx = np.zeros((S, k), dtype=np.int64)
    slot_src = np.full(S, -1, dtype=np.int64)   # pool index (s*k + j) expanded by slot s
    ties = {"frontier": 0, "rerank": 0}

    def parent_pool(e):
        return int(slot_src[e // k]) if e // k > 0 else -1

    def path_of(e):
        toks = []
        while e >= 0:
            toks.append(int(pool_tok[e // k, e % k]))
            e = parent_pool(e)
        return [int(root_token)] + toks[::-1]

    def add_children(s, v_parent, depth, cidx0, path):
        toks, qs = children_fn(s, path)
        for j in range(k):
            pool_tok[s, j] = toks[j]
            pool_q[s, j] = qs[j]
            pool_val[s, j] = np.float32(np.float32(v_parent) * np.float32(qs[j]))
            pool_depth[s, j] = depth
            pool_cidx[s, j] = cidx0 + j

    if frontier_fn is not None:
        frontier_fn([(0, [int(root_token)])])
    add_children(0, np.float32(1.0), 1, 0, [int(root_token)])
    layer = [j for j in range(k)]           # pool indices of layer 1
    for d in range(1, D):
        cand = sorted(layer, key=lambda e: (-float(pool_val.flat[e]), int(pool_cidx.flat[e])))
        for i in range(min(k, len(cand) - 1)):
            a, b = pool_val.flat[cand[i]], pool_val.flat[cand[i + 1]]
            same_q_sibs = (cand[i] // k == cand[i + 1] // k and pool_q.flat[cand[i]] == pool_q.flat[cand[i + 1]])
            if not same_q_sibs and _rel_gap(float(a), float(b)) < VALUE_TIE_REL:
                ties["frontier"] += 1
        nxt = []
        if frontier_fn is not None:
            frontier_fn([(1 + (d - 1) * k + i, path_of(e)) for i, e in enumerate(cand[:k])])
        for i, e in enumerate(cand[:k]):
            s = 1 + (d - 1) * k + i
            slot_src[s] = e
            add_children(s, pool_val.flat[e], d + 1, i * k, path_of(e))
            nxt.extend(s * k + j for j in range(k))
        layer = nxt

    # Rerank the whole pool: (value desc, depth asc, cidx asc), keep m.
    allp = list(range(S * k))
    ranked = sorted(allp, key=lambda e: (-float(pool_val.flat[e]), int(pool_depth.flat[e]), int(pool_cidx.flat[e])))
    if m < len(ranked):
        a, b = float(pool_val.flat[ranked[m - 1]]), float(pool_val.flat[ranked[m]])
        if _rel_gap(a, b) < VALUE_TIE_REL:
            ties["rerank"] += 1
    selected = set(ranked[:m])

    # Flatten in BFS order: (depth, parent flat index, sibling rank).
    N = m + 1
    flat_of = {-1: 0}
    order = []
    for d in range(1, D + 1):
        lvl = [e for e in selected if pool_depth.flat[e] == d]
        for e in lvl:
            if parent_pool(e) not in flat_of:
                raise AssertionError("rerank produced a disconnected tree")
        lvl.sort(key=lambda e: (flat_of[parent_pool(e)], e % k))
        for e in lvl:
            flat_of[e] = 1 + len(order)
            order.append(e)
    assert len(order) == m

    node_tok = np.zeros(N, np.int64)
    node_parent = np.full(N, -1, np.int64)
    node_depth = np.zeros(N, np.int64)
    node_sib = np.full(N, -1, np.int64)
    node_slot = np.full(N, -1, np.int64)
    node_value = np.ones(N, np.float32)
    node_q = np.ones(N, np.float32)
    node_pool = np.full(N, -1, np.int64)
    node_tok[0] = root_token
    node_slot[0] = 0
    slot_of_pool = {int(slot_src[s]): s for s in range(1, S)}
    for f, e in enumerate(order, start=1):
        node_tok[f] = pool_tok.flat[e]
        node_parent[f] = flat_of[parent_pool(e)]
        node_depth[f] = pool_depth.flat[e]
        node_sib[f] = e % k
        node_slot[f] = slot_of_pool.get(e, -1)
        node_value[f] = pool_val.flat[e]
        node_q[f] = pool_q.flat[e]
        node_pool[f] = e
    pool_flat = np.full((S, k), -1, np.int64)
    for e, f in flat_of.items():
        if e >= 0:
            pool_flat.flat[e] = f
    return dict(node_tok=node_tok, node_parent=node_parent, node_depth=node_depth,
                node_sib=node_sib, node_slot=node_slot, node_value=node_value,
                node_q=node_q, node_pool=node_pool, pool_tok=pool_tok, pool_q=pool_q,
                pool_val=pool_val, pool_depth=pool_depth, pool_cidx=pool_cidx,
                pool_flat=pool_flat, slot_src=slot_src, ties=ties)


def expand_request(rows, root_token, T, k, D, m, seed=0, req=0, round_id=0, warp=None):
    """Expansion of one request from its draft rows [S, V] given by slot."""
    rows = np.asarray(rows, dtype=np.float32)
    S = 1 + (D - 1) * k
    assert rows.shape[0] >= S
    stats = np.zeros((S, 2), np.float64)
    child_ties = [0]

    def children_fn(s, path):
        toks, q, M, Ssum, t = children_of_row(rows[s], T, k, seed, s, req, round_id, warp)
        stats[s] = (M, Ssum)
        child_ties[0] += t
        return toks, q

    out = build_tree(k, D, m, root_token, children_fn)
    out["slot_stats"] = stats
    out["ties"]["children"] = child_ties[0]
    return out


def expand_batch(draft_logits, roots, T, k, D, m, seed=0, round_id=0, warp=None):
    """Expansion of every request; arrays stacked on a leading batch axis."""
    outs = [expand_request(draft_logits[b], roots[b], T, k, D, m, seed, b, round_id, warp)
            for b in range(len(roots))]
    res = {key: np.stack([o[key] for o in outs]) for key in outs[0] if key != "ties"}
    res["ties"] = [o["ties"] for o in outs]
    return res
