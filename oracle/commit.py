"""Post-accept commit: the accepted path extends the context (a step after the
round's hot path; test infrastructure like the rest of this package).

EAGLE-1 notes, section 3.3: the accepted tokens and their features are kept
for the next round's drafting; hubwiz section 5: the single longest
consistent path is committed, the other branches collapse, and the loop
repeats from the new, longer context.

Readings:
* The committed rows are the root (flat index 0, the last committed token of
  the previous round, whose key/value the verify pass computed) followed by the
  accepted draft nodes in path order.  Their tree keys/values are appended to
  the request's prefix cache at positions L, L+1, ..., L+a (a = accepted draft
  nodes), and the prefix length becomes L + a + 1.  The token drawn after the
  last accepted node (resample or bonus) has no key/value yet: it is the next
  round's root.
* The features kept for the next draft are the LM-head inputs of the same
  rows (root first), written to rows 0..a of a [depth + 1, hidden] block;
  rows past a are zero.
* A path that names a node outside [1, N) or a length outside [0, depth]
  commits nothing (features zero); a cache without room for a + 1 more rows
  keeps its prefix and length (the features are still written).
"""
import numpy as np


def commit(k_prefix, v_prefix, prefix_len, k_tree, v_tree, x, accept_len, accept_path, depth):
    """One request.

    k_prefix, v_prefix [hkv, Lmax, dh]   the prefix cache (not modified)
    prefix_len          int              rows in use
    k_tree, v_tree      [N, hkv, dh]     keys/values of the tree nodes
    x                   [N, H]           LM-head inputs (features) of the tree nodes
    accept_len          int              a, accepted draft nodes
    accept_path         [depth]          their flat indices (first a used)
    Returns (k_prefix', v_prefix', prefix_len', features [depth + 1, H], flags)
    with flags a set of {"bad_path", "cache_full"}.
    """
    kp = np.array(k_prefix, copy=True)
    vp = np.array(v_prefix, copy=True)
    N = np.asarray(k_tree).shape[0]
    H = np.asarray(x).shape[1]
    feat = np.zeros((depth + 1, H), np.asarray(x).dtype)
    flags = set()
    a = int(accept_len)
    L = int(prefix_len)
    if a < 0 or a > depth or any(not (1 <= int(accept_path[r]) < N) for r in range(max(a, 0) if a <= depth else 0)):
        flags.add("bad_path")
        return kp, vp, L, feat, flags
    rows = [0] + [int(accept_path[r]) for r in range(a)]
    for r, node in enumerate(rows):
        feat[r] = x[node]
    Lmax = kp.shape[1]
    if L < 0 or L + a + 1 > Lmax:
        flags.add("cache_full")
        return kp, vp, L, feat, flags
    for r, node in enumerate(rows):
        kp[:, L + r] = k_tree[node]
        vp[:, L + r] = v_tree[node]
    return kp, vp, L + a + 1, feat, flags
