"""Tree attention mask (the oracle's step O7).

EAGLE-2 notes, "Tree Attention Mask": tokens of different branches must not
see one another; each flattened token sees only its ancestors (plus itself and,
in the attention, the whole context).  hubwiz section 5 states the same: every
candidate sees its own ancestors and the original context, never its siblings.
"""
import numpy as np


def ancestor_mask(node_parent):
    """Boolean [N, N]: mask[i, j] is True iff j == i or j is an ancestor of i."""
    par = np.asarray(node_parent)
    N = par.shape[0]
    m = np.zeros((N, N), dtype=bool)
    for i in range(N):
        j = i
        while j >= 0:
            m[i, j] = True
            j = int(par[j])
    return m


def pack_bits(mbool):
    """Pack a boolean [N, N] mask into uint64 words [N, ceil(N/64)] (bit j%64 of word j//64)."""
    N = mbool.shape[0]
    W = (N + 63) // 64
    out = np.zeros((N, W), dtype=np.uint64)
    for i in range(N):
        for j in np.nonzero(mbool[i])[0]:
            out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def positions(node_depth, prefix_len):
    """Position of each flattened token: prefix length + depth (root at L)."""
    return np.asarray(node_depth, dtype=np.int64) + int(prefix_len)
