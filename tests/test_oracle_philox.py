"""Pins of the oracle's Philox4x32-10 and its uniform mapping."""
import os

import numpy as np

from oracle import philox

GOLD = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(x, 16) for x in line.split()]
        yield w[:4], w[4:6], w[6:10]


def test_known_answer_vectors():
    n = 0
    for ctr, key, exp in _kat():
        got = philox.philox4x32_10(*ctr, *key)
        assert [int(g) for g in got] == exp
        n += 1
    assert n == 3


def test_vectorised_matches_scalar():
    c0 = np.arange(37)
    got = philox.philox4x32_10(c0, 5, 9, 11, 0x1234, 0x9876)
    for i in range(37):
        one = philox.philox4x32_10(i, 5, 9, 11, 0x1234, 0x9876)
        assert [int(g[i]) for g in got] == [int(o) for o in one]


def test_uniform_mapping_open_interval_and_exact_in_fp32():
    u = philox.gumbel_uniforms(4099, 3, 1, 7, (0xABCDEF << 32) | 0x13579)
    assert u.shape == (4099,)
    assert (u > 0).all() and (u < 1).all()
    assert (u.astype(np.float32).astype(np.float64) == u).all()
    # odd multiples of 2^-24
    j = u * 2.0 ** 24
    assert (j == np.round(j)).all() and (np.round(j) % 2 == 1).all()
    # token v uses word v & 3 of counter v >> 2
    w = philox.philox4x32_10(5, 3, 1, 7, 0x13579, 0xABCDEF)
    for t in range(4):
        assert u[20 + t] == (2.0 * (int(w[t]) >> 9) + 1.0) * 2.0 ** -24


def test_uniform_mean_and_spread():
    u = philox.gumbel_uniforms(200000, 0, 0, 0, 42)
    assert abs(u.mean() - 0.5) < 0.005
    assert abs(u.var() - 1.0 / 12.0) < 0.002
