"""A synthetic EAGLE draft head on the device, and depth-by-depth drafting.

`DeviceDraftHead` holds the head's weights (bf16; the matrices packed once for
the streaming GEMM), the root features, the draft's own prefix K/V cache and
its workspace.  `draft_tree` runs one round's drafting through the C ABI:

    for d in 0 .. D-1:  eagle_draft_forward(d)  ->  eagle_expand_depth(d)
    eagle_expand_finish

every step in libeagle's kernels on the current HIP stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops


def _dev(a, dtype, device):
    return torch.from_numpy(a).to(device=device).to(dtype).contiguous()


class DeviceDraftHead:
    """dinp: synth.draft.DraftInputs (weights, root features, draft prefix K/V);
    wts: the round's DeviceWeights (its packed LM head is shared)."""

    def __init__(self, cfg, dinp, wts, device="cuda"):
        if cfg.dtype != "bf16" or not wts.packed:
            raise ValueError("the draft head runs on bf16 workloads with a packed LM head")
        c = self.cfg = cfg
        bf = torch.bfloat16
        w = dinp.weights
        self.embed = _dev(w["E"], bf, device)
        pk = lambda a: ops.pack_lmhead_weight(_dev(a, bf, device))  # noqa: E731
        self.fc = pk(w["fc"])
        self.qkv = pk(np.concatenate([w["q"], w["k"], w["v"]], axis=0))
        self.o = pk(w["o"])
        self.gate_up = pk(np.concatenate([w["g"], w["u"]], axis=0))
        self.down = pk(w["d"])
        self.lm = wts.w_packed
        self.root_feat = _dev(dinp.root_feat, bf, device)
        self.k_prefix = _dev(dinp.k_prefix, bf, device)
        self.v_prefix = _dev(dinp.v_prefix, bf, device)
        self.inter = dinp.inter
        self.cap = dinp.cap
        self.dims = ops.draft_dims(c.H, c.hq, c.hkv, c.dh, self.inter, self.cap)
        self.lm_z = getattr(wts, "w_z", None)  # the round's z-packed LM head, read by depths of few rows
        self.weights = ops.draft_weights(self.embed, self.fc, self.qkv, self.o, self.gate_up, self.down, self.lm,
                                         self.lm_z)
        n = ops.draft_workspace_size(ops.tree_params(c.B, c.V, c.D, c.k, c.m, 1.0), self.dims)
        if n == 0:
            raise ValueError("invalid draft-head shape")
        self.ws = torch.empty(n, dtype=torch.uint8, device=device)

    def forward(self, p, depth, roots, prefix_len, tree, rows, status=None):
        ops.draft_forward(p, depth, self.dims, self.weights, roots, self.root_feat, self.k_prefix, self.v_prefix,
                          prefix_len, tree["pool_tok"], tree["slot_src"], rows, self.ws, status)


def draft_tree(head, rnd, data, T, round_id=0, warp=None, draft_bound=None):
    """Draft one round's tree depth by depth into rnd.tree, with data.rows as the
    [B, S, V] draft-row buffer (rnd: a DeviceRound, data: its DeviceInputs).
    warp = (top_k, top_p) with T > 0: each depth's rows are warped before its
    children are drawn, their bounds kept in draft_bound [B, S, 2] uint32."""
    p = rnd.params(T, round_id, data.seed)
    for d in range(rnd.cfg.D):
        head.forward(p, d, data.roots, data.prefix_len, rnd.tree, data.rows, rnd.status)
        ops.expand_depth(p, d, data.rows, rnd.tree, rnd.ws, rnd.status, warp=warp, draft_bound=draft_bound)
    ops.expand_finish(p, data.roots, rnd.tree, rnd.status)
