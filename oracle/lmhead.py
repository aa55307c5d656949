"""LM-head logits and the softmax at every node (the oracle's step O9).

EAGLE-1 notes, background section A3: the LM head maps the feature f_j to the
next-token distribution p_{j+1} = LMHead(f_j).  Temperature adjusts the
distribution before the acceptance test (hubwiz section 2).

Readings: logits z = X W^T accumulated in fp64; p = softmax(fp32(z)/T') with
T' = T (T > 0) or 1 (greedy); the greedy choice is the argmax of z with ties
to the lowest token id.
"""
import numpy as np

from .expand import softmax_stats


def logits(x, w, block=16384):
    """z = X W^T in fp64.  x [R, H], w [V, H] (any float dtype)."""
    x = np.asarray(x, np.float64)
    V = w.shape[0]
    out = np.empty((x.shape[0], V), np.float64)
    for lo in range(0, V, block):
        hi = min(V, lo + block)
        out[:, lo:hi] = x @ np.asarray(w[lo:hi], np.float64).T
    return out


def row_stats(z32, T):
    """Per row (M, S) of softmax(fp32(z)/T') and the argmax of z (lowest id on ties)."""
    z32 = np.asarray(z32, np.float32)
    st = np.array([softmax_stats(r, T) for r in z32])
    am = np.argmax(z32, axis=1)  # first maximal index
    return st, am
