"""Sampling warps: top-k and nucleus applied to a row before it is used
(test infrastructure, like the rest of this package).

hubwiz section 2: speculative decoding stays exact for sampling with
temperature, top-k or nucleus when both distributions (target and draft) are
adjusted the same way before the acceptance test.

Readings:
* A row's tokens are ordered by (t desc, id asc) with t = fp32(z / T') (the
  temperature-scaled logit the softmax uses).  top-k keeps the first
  min(k, V) tokens of that order (k = 0: all).  The nucleus then keeps the
  shortest prefix of those whose softmax mass (renormalised over the top-k
  set) reaches top_p, the token that crosses it included (top_p = 1: all).
  The warped distribution is softmax(t) restricted to the kept prefix and
  renormalised.
* At least min_keep tokens are kept (a tree draws its k children without
  replacement from the draft's warped distribution, so both sides keep at
  least k); top-k must then be 0 or at least min_keep.
* The kept set is a prefix of the order, so it is described by its last token
  (t_b, id_b): token v is kept iff t_v > t_b, or t_v == t_b and v <= id_b.
* Masses are exp(t - max t) in fp64 summed in the order above; a nucleus whose
  crossing point lies within NUCLEUS_TIE_REL of the target (relative to the
  top-k mass, which is at least 1) is reported as a near tie.  The window
  covers an implementation that sums the masses as fixed-point integers of
  2^(62 - ceil(log2 V)) per unit: its cumulative masses differ from exact ones
  by at most V * 2^-(63 - ceil(log2 V)), about 2e-9 at V = 128256.
* Greedy decoding (T = 0) takes the argmax and uses no warp.
"""
from __future__ import annotations

import numpy as np

from .expand import scaled_logits

NUCLEUS_TIE_REL = 1e-8


def warp_support(z, T, top_k=0, top_p=1.0, min_keep=1):
    """Kept prefix of one row.

    Returns dict(order=ids in (t desc, id asc) order, n=kept count,
    t_b, id_b (last kept token), M=max t, S=sum of exp(t - M) over the kept
    tokens (fp64), mask=bool[V], tie=near-tie flag of the nucleus cut).
    """
    t32 = scaled_logits(z, T)
    t = t32.astype(np.float64)
    V = t.shape[0]
    ids = np.arange(V)
    order = np.lexsort((ids, -t))
    kk = V if top_k <= 0 else min(int(top_k), V)
    M = t.max()
    e = np.exp(t[order[:kk]] - M)
    n = kk
    tie = False
    if top_p < 1.0:
        SA = e.sum()
        c = np.cumsum(e)
        target = float(top_p) * SA
        nn = int(np.searchsorted(c, target, side="left")) + 1   # first prefix whose mass reaches the target
        nn = min(nn, kk)
        lo = c[nn - 2] if nn >= 2 else 0.0
        if nn >= min_keep and (abs(c[nn - 1] - target) < NUCLEUS_TIE_REL * SA or abs(lo - target) < NUCLEUS_TIE_REL * SA):
            tie = True
        n = max(nn, min(int(min_keep), kk))
    kept = order[:n]
    mask = np.zeros(V, bool)
    mask[kept] = True
    S = e[:n].sum()
    return dict(order=order, n=n, t_b=float(t32[kept[-1]]), id_b=int(kept[-1]), M=M, S=S, mask=mask, tie=tie)


def warped_softmax(z, T, top_k=0, top_p=1.0, min_keep=1):
    """The warped distribution (fp64 [V]): softmax(t) on the kept prefix, renormalised."""
    w = warp_support(z, T, top_k, top_p, min_keep)
    t = scaled_logits(z, T).astype(np.float64)
    p = np.where(w["mask"], np.exp(t - w["M"]), 0.0)
    return p / p.sum()
