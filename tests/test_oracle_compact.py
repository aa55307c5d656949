"""Pins of the compact target-row form (oracle/compact.py).

* The block maximum decodes exactly, every decoded logit stays at or below its
  block maximum, and the order of logits inside a block is kept (ties may be
  created by the rounding, never reversed).
* The fp16 offset is the round-to-nearest-even of the fp32 difference: decoded
  values lie within half an fp16 ulp of |z - m| of the fp32 logit.
* Probabilities of tokens at >= 1e-6 of the row's largest differ from the fp32
  row's by less than the 2e-2 bar (the bound is about 1.4%: 0.7% for the token,
  as much again from the normalisation); M is the fp32 row's exactly and S
  differs by < 1e-2.
* Non-finite logits and all -inf blocks decode to -inf; a ragged last block.
"""
import numpy as np

from oracle import compact
from oracle.expand import softmax


def _rows(seed, R=6, V=1000, scale=2.0):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((R, V))).astype(np.float32)


def test_block_max_exact_and_order_kept():
    z = _rows(1, V=5003)
    d, m = compact.encode(z)
    zt = compact.decode(d, m)
    assert m.shape == (6, (5003 + 127) // 128)
    for r in range(z.shape[0]):
        for b in range(m.shape[1]):
            blk = z[r, b * 128:(b + 1) * 128]
            dblk = zt[r, b * 128:(b + 1) * 128]
            j = int(np.argmax(blk))
            assert dblk[j] == blk[j] == m[r, b]
            assert (dblk <= m[r, b]).all()
            o = np.argsort(blk, kind="stable")
            assert (np.diff(dblk[o]) >= 0).all()


def test_offsets_are_round_to_nearest_of_the_difference():
    z = _rows(2, V=777, scale=5.0)
    d, m = compact.encode(z)
    mv = np.repeat(m, 128, axis=1)[:, :777]
    diff = (z - mv).astype(np.float64)
    err = np.abs(d.astype(np.float64) - diff)
    half_ulp = np.abs(diff) * 2.0 ** -11 + 2.0 ** -25   # fp16: 11 significant bits; subnormal step 2^-24
    assert (err <= half_ulp).all()


def test_probabilities_within_the_bar():
    for seed, scale, T in [(3, 1.0, 1.0), (4, 4.0, 1.0), (5, 3.0, 0.7), (6, 8.0, 1.3)]:
        z = _rows(seed, V=4096, scale=scale)
        zt = compact.decode(*compact.encode(z))
        for r in range(z.shape[0]):
            p, pt = softmax(z[r], T), softmax(zt[r], T)
            keep = p >= 1e-6 * p.max()
            rel = np.abs(pt[keep] - p[keep]) / p[keep]
            assert rel.max() < 1.4e-2, (seed, rel.max())
            tp = (z[r] / np.float32(T)).astype(np.float64)
            tt = (zt[r] / np.float32(T)).astype(np.float64)
            assert tp.max() == tt.max()
            S, St = np.exp(tp - tp.max()).sum(), np.exp(tt - tt.max()).sum()
            assert abs(St - S) / S < 1e-2


def test_non_finite_and_empty_blocks():
    z = _rows(7, R=2, V=300)
    z[0, 5] = np.inf
    z[0, 6] = np.nan
    z[1, 128:256] = -np.inf      # a whole block without finite logits
    z[1, 299] = -np.inf
    d, m = compact.encode(z)
    zt = compact.decode(d, m)
    assert zt[0, 5] == -np.inf and zt[0, 6] == -np.inf
    assert m[1, 1] == -np.inf and (zt[1, 128:256] == -np.inf).all()
    assert zt[1, 299] == -np.inf
    assert np.isfinite(zt[0, 7])
    assert m.shape == (2, 3)   # ragged last block of 44 columns


def test_planted_truncation_breaks_the_rounding_pin(monkeypatch):
    """Offsets truncated toward zero instead of rounded would fail the half-ulp pin."""
    z = _rows(8, V=512, scale=5.0)
    d, m = compact.encode(z)
    mv = np.repeat(m, 128, axis=1)[:, :512]
    diff = (z - mv).astype(np.float32)
    bits = diff.view(np.uint32) & np.uint32(0xFFFFE000)   # drop 13 of 23 mantissa bits: truncation
    trunc = bits.view(np.float32).astype(np.float16)
    err = np.abs(trunc.astype(np.float64) - diff.astype(np.float64))
    half_ulp = np.abs(diff.astype(np.float64)) * 2.0 ** -11 + 2.0 ** -25
    assert (err > half_ulp).any()
