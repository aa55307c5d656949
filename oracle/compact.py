"""Compact target rows: the LM head's logits stored without fp32 rows
(test infrastructure, like the rest of this package).

EAGLE-1 notes, background A3 and section 3.3: the verify pass gives the
target's distribution p at every tree node from the LM head; the walk needs p
at the candidates and, after a rejection, over the whole vocabulary (the
residual and the final draw).  Storing every node's row in fp32 costs 4 bytes
per logit; this form stores 2.

Reading (the pages fix no storage format): a row is cut into blocks of 128
columns.  Each block keeps its largest finite logit m (fp32) and every logit
as d = fp16(z - m), the fp32 difference rounded to nearest even (non-finite
logits and blocks with no finite logit store -inf).  The decoded logit is
z~ = fp32(m + fp32(d)); the block maximum decodes exactly.  Every use of the
row (the statistics M and S, the acceptance ratios, the residual sums, the
draws) reads z~, so the walk is exact for the distribution softmax(z~ / T).
For tokens with p >= 1e-6 of the row's largest p, |z - m| <= 13.82 T (m is at
least the token's own logit and at most the row's), and the fp16 rounding of d
moves z by at most 2^-11 |d| <= 0.0068 T: p changes by a factor within
exp(+-0.0068) (0.7%) before the normalisation, which adds at most as much
again: about 1.4% at worst, inside the 2e-2 bar for probabilities of bf16
workloads.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def encode(z32):
    """(d fp16 [R, V], m fp32 [R, ceil(V / 128)]) of fp32 logits [R, V]."""
    z = np.asarray(z32, np.float32)
    z = np.where(np.isfinite(z), z, np.float32(-np.inf)).astype(np.float32)
    R, V = z.shape
    nb = (V + BLOCK - 1) // BLOCK
    zp = np.full((R, nb * BLOCK), -np.inf, np.float32)
    zp[:, :V] = z
    m = zp.reshape(R, nb, BLOCK).max(axis=2).astype(np.float32)
    mv = np.repeat(m, BLOCK, axis=1)[:, :V]
    with np.errstate(invalid="ignore", over="ignore"):
        diff = (z - mv).astype(np.float32)   # one fp32 subtraction per logit
        d = diff.astype(np.float16)          # round to nearest even; beyond the range: -inf
    d = np.where((mv == -np.inf) | (z == -np.inf), np.float16(-np.inf), d)
    return d, m


def decode(d16, m):
    """Decoded fp32 logits z~ = fp32(m + fp32(d)) of a compact row block set."""
    d = np.asarray(d16, np.float16)
    R, V = d.shape
    mv = np.repeat(np.asarray(m, np.float32), BLOCK, axis=1)[:, :V]
    df = d.astype(np.float32)
    with np.errstate(invalid="ignore"):
        z = (mv + df).astype(np.float32)
    return np.where(df == -np.inf, np.float32(-np.inf), z).astype(np.float32)
