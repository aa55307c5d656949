"""A static (EAGLE-1) draft tree: expansion on a fixed shape (test infrastructure).

Sources:
* EAGLE-1 notes, appendix A.1 ("tree structure"): the draft tree has a fixed
  shape; the number of children k of each node is read off the shape (k = 4
  at the root); greedy drafting takes the top-k tokens as children, sampling
  drafts k tokens; tree or chain, the draft model runs 5 forward passes.
  The shape is not tuned: branches that start from more probable tokens are
  made deeper and wider.
* EAGLE-3 notes ("EAGLE and EAGLE-2"): EAGLE-1's tree is predefined, static
  and independent of the context.

Readings (the pages give the figure's root only):
* A shape is a flattened rooted tree given by its parent array: node 0 is the
  root (the last committed token), parent[i] < i, and the children of a node
  appear in increasing sibling rank (rank = order among its parent's children
  in flat order).  Every node with children is a slot; slots are numbered in
  flat order, and slot s has k_s children.
* Slot s draws its k_s children from its draft row: the top-k_s logits
  (greedy) or k_s draws without replacement (Gumbel-top-k, the same keys as the
  dynamic tree's with slot index s), in sampling order; child j of slot s is
  the node of sibling rank j under the slot's node.  Values are the fp32
  products of the confidences on the root path, as in the dynamic tree (they
  decide nothing here).
* DEFAULT_SHAPE is this build's own shape following the stated rules (root 4
  children, depth 5 so that 5 draft passes fill it, the more probable
  branches deeper and wider); it is not the paper's figure, which the pages do
  not reproduce.
* Acceptance walks the same way as on the dynamic tree; a slot's candidates
  are exactly its k_s draws (pool entries past k_s are marked -1).
"""
from __future__ import annotations

import numpy as np

from .expand import children_of_row, softmax_stats

# Paths of sibling ranks from the root, in flat (BFS) order.
DEFAULT_PATHS = (
    (0,), (1,), (2,), (3,),
    (0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (2, 0), (3, 0),
    (0, 0, 0), (0, 0, 1), (0, 1, 0), (1, 0, 0), (2, 0, 0),
    (0, 0, 0, 0), (0, 0, 0, 1), (0, 1, 0, 0), (1, 0, 0, 0),
    (0, 0, 0, 0, 0), (0, 1, 0, 0, 0),
)


def parents_from_paths(paths):
    """Parent array of the flattened tree whose nodes 1.. are `paths` (root = node 0)."""
    index = {(): 0}
    par = [-1]
    for i, p in enumerate(paths, start=1):
        par.append(index[tuple(p[:-1])])
        index[tuple(p)] = i
    return np.array(par, np.int64)


DEFAULT_SHAPE = parents_from_paths(DEFAULT_PATHS)


def shape_info(parent):
    """Depth, sibling rank and slot of every node; children count of every slot."""
    parent = np.asarray(parent, np.int64)
    n = parent.shape[0]
    if n < 1 or parent[0] != -1 or any(not (0 <= parent[i] < i) for i in range(1, n)):
        raise ValueError("shape: parent[0] must be -1 and 0 <= parent[i] < i")
    depth = np.zeros(n, np.int64)
    sib = np.full(n, -1, np.int64)
    nchild = np.zeros(n, np.int64)
    for i in range(1, n):
        depth[i] = depth[parent[i]] + 1
        sib[i] = nchild[parent[i]]
        nchild[parent[i]] += 1
    slot = np.full(n, -1, np.int64)
    slot_node = []
    for i in range(n):
        if nchild[i] > 0:
            slot[i] = len(slot_node)
            slot_node.append(i)
    slot_k = nchild[slot_node]
    return dict(n=n, depth=depth, sib=sib, slot=slot, slot_node=np.array(slot_node, np.int64),
                slot_k=slot_k, S=len(slot_node), D=int(depth.max()), kmax=int(slot_k.max()) if len(slot_node) else 0)


def build_static_tree(parent, root_token, children_fn):
    """Fill a static shape.  children_fn(slot, path, kk) -> (tokens[kk], q_fp32[kk]).

    Slots are asked in flat order, so a slot's root path is known when it is
    asked.  Returns node arrays [n] and the pool [S, kmax] (-1 / 0 past a
    slot's kk children)."""
    info = shape_info(parent)
    n, S, kmax = info["n"], info["S"], info["kmax"]
    pool_tok = np.full((S, kmax), -1, np.int64)
    pool_q = np.zeros((S, kmax), np.float32)
    node_tok = np.zeros(n, np.int64)
    node_tok[0] = root_token
    node_value = np.ones(n, np.float32)
    node_q = np.ones(n, np.float32)
    paths = [[int(root_token)]]
    for i in range(1, n):
        paths.append(None)
    for s, u in enumerate(info["slot_node"]):
        kk = int(info["slot_k"][s])
        toks, q = children_fn(s, paths[u], kk)
        pool_tok[s, :kk] = toks[:kk]
        pool_q[s, :kk] = q[:kk]
        for c in range(u + 1, n):
            if parent[c] == u:
                j = int(info["sib"][c])
                node_tok[c] = int(toks[j])
                node_q[c] = q[j]
                node_value[c] = np.float32(np.float32(node_value[u]) * np.float32(q[j]))
                paths[c] = paths[u] + [int(toks[j])]
    pool_flat = np.full((S, kmax), -1, np.int64)
    slot_src = np.full(S, -1, np.int64)
    for c in range(1, n):
        s = int(info["slot"][parent[c]])
        pool_flat[s, info["sib"][c]] = c
    for s, u in enumerate(info["slot_node"]):
        if u > 0:
            ps = int(info["slot"][parent[u]])
            slot_src[s] = ps * kmax + int(info["sib"][u])
    node_sib = info["sib"].copy()
    return dict(node_tok=node_tok, node_parent=np.asarray(parent, np.int64).copy(), node_depth=info["depth"].copy(),
                node_sib=node_sib, node_slot=info["slot"].copy(), node_value=node_value, node_q=node_q,
                pool_tok=pool_tok, pool_q=pool_q, pool_flat=pool_flat, slot_src=slot_src)


def expand_static_request(rows, parent, root_token, T, seed=0, req=0, round_id=0):
    """Static tree of one request from its draft rows [S, V] by slot."""
    info = shape_info(parent)
    stats = np.zeros((info["S"], 2), np.float64)
    ties = [0]
    kmax = info["kmax"]

    def children_fn(s, path, kk):
        toks, q, M, Ssum, t = children_of_row(rows[s], T, kmax, seed, s, req, round_id)
        stats[s] = (M, Ssum)
        # only the boundaries inside the slot's own kk draws decide the tree
        if t:
            toks_k, _, _, _, t_k = children_of_row(rows[s], T, kk, seed, s, req, round_id)
            ties[0] += t_k
        return toks[:kk], q[:kk]

    out = build_static_tree(parent, root_token, children_fn)
    out["slot_stats"] = stats
    out["ties"] = ties[0]
    return out


def expand_static_batch(rows, parent, roots, T, seed=0, round_id=0):
    outs = [expand_static_request(rows[b], parent, roots[b], T, seed, b, round_id) for b in range(len(roots))]
    res = {key: np.stack([o[key] for o in outs]) for key in outs[0] if key != "ties"}
    res["ties"] = [o["ties"] for o in outs]
    return res


def target_static_rows(inp, T, parent, weights=None):
    """Draft rows [B, S, V] of a static shape, slot by slot (the dynamic tree's
    reading R15): the row of slot s is the target's logits at the slot's node,
    computed on the node's root path alone, plus sigma_b * eps[b, s]; slots are
    filled in flat order, so each slot's path is drawn before it is needed."""
    from .round import _Weights, attention_rows
    c = inp.cfg
    if c.draft == "iid":
        return inp.iid_draft_rows()
    wts = weights or _Weights(inp)
    info = shape_info(parent)
    rows = np.zeros((c.B, info["S"], c.V), np.float32)
    for b in range(c.B):
        sig = np.float64(inp.sigma[b])

        def children_fn(s, path, kk, b=b, sig=sig):
            x, _ = attention_rows(inp, b, path, np.arange(len(path)) - 1)
            z = wts.logits(x[-1:])[0]
            rows[b, s] = (z + sig * inp.eps[b, s].astype(np.float64)).astype(np.float32)
            toks, q, _, _, _ = children_of_row(rows[b, s], T, info["kmax"], inp.gumbel_seed, s, b, 0)
            return toks[:kk], q[:kk]

        build_static_tree(parent, int(inp.roots[b]), children_fn)
    return rows


def run_static_round(inp, T, parent, rows=None, round_id=0, weights=None):
    """Every stage of one round on a static shape (expand, mask, attention, LM head, accept)."""
    from . import accept, lmhead, mask
    from .round import _Weights, attention_rows
    c = inp.cfg
    wts = weights or _Weights(inp)
    if rows is None:
        rows = target_static_rows(inp, T, parent, wts)
    ex = expand_static_batch(rows, parent, inp.roots, T, inp.gumbel_seed, round_id)
    n = len(parent)
    X = np.zeros((c.B, n, c.H), np.float32)
    O64 = np.zeros((c.B, n, c.hq, c.dh), np.float64)
    for b in range(c.B):
        X[b], O64[b] = attention_rows(inp, b, ex["node_tok"][b], ex["node_parent"][b])
    z64 = wts.logits(X.reshape(c.B * n, c.H))
    z32 = z64.astype(np.float32)
    stats, am = lmhead.row_stats(z32, T)
    info = shape_info(parent)
    acc = []
    for b in range(c.B):
        tree = {key: ex[key][b] for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat")}
        acc.append(accept.accept_request(tree, z32[b * n:(b + 1) * n], rows[b], T, info["kmax"], info["D"],
                                         inp.uniforms[b], am[b * n:(b + 1) * n]))
    masks = np.stack([mask.pack_bits(mask.ancestor_mask(ex["node_parent"][b])) for b in range(c.B)])
    return dict(rows=rows, expand=ex, mask=masks, attn=O64, x=X, logits64=z64, logits=z32, stats=stats, argmax=am,
                accept=acc)
