"""One whole round on the CPU, and the synthetic draft rows it consumes.

Round order (EAGLE-2 notes: expand, rerank, flatten + mask; EAGLE-1 notes
section 3.3 and hubwiz section 5: one tree-attention verify pass, then the
acceptance walk): expand -> mask -> tree attention -> LM head -> accept.

Readings:
* Tree-node queries, keys and values are per-token rows (q_tab/k_tab/v_tab of
  the synthetic inputs), looked up by the node's token; the verify layer has no
  other projection.  The LM-head input of node i is its attention output,
  concatenated over heads and rounded to the workload's dtype.
* "Draft logits = target logits + noise" is realised slot by slot: the row of
  the slot that expands node f is the target logits at f, computed on f's root
  path alone (the ancestor-only mask makes them equal to f's verify row), plus
  sigma * eps[slot].  Workloads marked "iid" use sigma * eps directly.
"""
from __future__ import annotations

import numpy as np

from . import accept, attention, expand, lmhead, mask
from synth.gen import bf16_round


def _act_round(x, dtype):
    x32 = np.asarray(x, np.float64).astype(np.float32)
    return bf16_round(x32) if dtype == "bf16" else x32


class _Weights:
    """fp64 copy of the LM-head weight, made once per inputs object."""

    def __init__(self, inp):
        self.inp = inp
        self._w64 = None

    def logits(self, x):
        if self._w64 is None:
            self._w64 = np.asarray(self.inp.w, np.float64)
        return np.asarray(x, np.float64) @ self._w64.T


def attention_rows(inp, b, tokens, parent):
    """Attention outputs [n, H] (workload dtype) of nodes with `tokens`/`parent`."""
    c = inp.cfg
    tokens = np.asarray(tokens, np.int64)
    n = tokens.shape[0]
    q = inp.q_tab[tokens].reshape(n, c.hq, c.dh)
    kt = inp.k_tab[tokens].reshape(n, c.hkv, c.dh)
    vt = inp.v_tab[tokens].reshape(n, c.hkv, c.dh)
    mb = mask.ancestor_mask(parent)
    scale = np.float32(1.0 / np.sqrt(c.dh))
    o = attention.tree_attention(q, inp.k_prefix[b], inp.v_prefix[b], inp.prefix_len[b],
                                 kt, vt, mb, scale)
    return _act_round(o.reshape(n, c.hq * c.dh), c.dtype), o


def target_draft_rows(inp, T, weights=None):
    """Draft rows [B, S, V] fp32 built slot by slot from the target (see module doc)."""
    c = inp.cfg
    if c.draft == "iid":
        return inp.iid_draft_rows()
    wts = weights or _Weights(inp)
    rows = np.zeros((c.B, c.S, c.V), np.float32)
    for b in range(c.B):
        sig = np.float64(inp.sigma[b])

        def frontier_fn(items, b=b, sig=sig):
            # The k frontier nodes of one depth: attend on each node's root path,
            # then one LM-head product for the depth.
            xs = []
            for s, path in items:
                n = len(path)
                x, _ = attention_rows(inp, b, path, np.arange(n) - 1)
                xs.append(x[-1])
            z = wts.logits(np.stack(xs))
            for (s, _), zr in zip(items, z):
                rows[b, s] = (zr + sig * inp.eps[b, s].astype(np.float64)).astype(np.float32)

        def children_fn(s, path, b=b):
            toks, q, _, _, _ = expand.children_of_row(rows[b, s], T, c.k, inp.gumbel_seed, s, b, 0)
            return toks, q

        expand.build_tree(c.k, c.D, c.m, int(inp.roots[b]), children_fn, frontier_fn)
    return rows


def run_round(inp, T, rows=None, round_id=0, weights=None, warp=None):
    """Every stage of one round; returns a dict of per-stage results.

    warp = (top_k, top_p): both distributions warped before use (T > 0; see
    oracle/warp.py), at least k tokens kept."""
    c = inp.cfg
    wts = weights or _Weights(inp)
    if rows is None:
        rows = target_draft_rows(inp, T, wts)
    ex = expand.expand_batch(rows, inp.roots, T, c.k, c.D, c.m, inp.gumbel_seed, round_id, warp)
    masks = np.stack([mask.pack_bits(mask.ancestor_mask(ex["node_parent"][b])) for b in range(c.B)])
    pos = np.stack([mask.positions(ex["node_depth"][b], inp.prefix_len[b]) for b in range(c.B)])
    X = np.zeros((c.B, c.N, c.H), np.float32)
    O64 = np.zeros((c.B, c.N, c.hq, c.dh), np.float64)
    for b in range(c.B):
        X[b], O64[b] = attention_rows(inp, b, ex["node_tok"][b], ex["node_parent"][b])
    z64 = wts.logits(X.reshape(c.B * c.N, c.H))
    z32 = z64.astype(np.float32)
    stats, am = lmhead.row_stats(z32, T)
    acc = []
    for b in range(c.B):
        tree = {key: ex[key][b] for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat")}
        acc.append(accept.accept_request(tree, z32[b * c.N:(b + 1) * c.N], rows[b], T, c.k, c.D,
                                         inp.uniforms[b], am[b * c.N:(b + 1) * c.N], warp))
    return dict(rows=rows, expand=ex, mask=masks, pos=pos, attn=O64, x=X, logits64=z64,
                logits=z32, stats=stats, argmax=am, accept=acc)
