"""Pins of the oracle's LM head and row statistics (textbook closed forms)."""
import numpy as np

from oracle import lmhead


def test_logits_special_cases():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 8))
    w = np.zeros((5, 8))
    w[0, 2] = 1.0           # picks feature 2
    w[1] = 1.0              # sums features
    w[3, 7] = -2.0
    z = lmhead.logits(x, w, block=2)
    assert np.array_equal(z[:, 0], x[:, 2])
    assert np.allclose(z[:, 1], x.sum(axis=1), rtol=1e-14)
    assert np.array_equal(z[:, 2], np.zeros(3))
    assert np.array_equal(z[:, 3], -2.0 * x[:, 7])
    # blocking does not change the result: a single column at a time
    w2 = rng.standard_normal((37, 8))
    a = lmhead.logits(x, w2, block=5)
    b = np.stack([[float(np.dot(x[r], w2[v])) for v in range(37)] for r in range(3)])
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_row_stats_and_argmax():
    z = np.array([[1.0, 3.0, 3.0, -1.0], [0.0, 0.0, 0.0, 0.0]], np.float32)
    st, am = lmhead.row_stats(z, 1.0)
    assert list(am) == [1, 0]        # ties go to the lowest id
    assert st[0, 0] == 3.0
    assert np.isclose(st[0, 1], 2.0 + np.exp(-2.0) + np.exp(-4.0))
    assert st[1, 1] == 4.0
    st2, _ = lmhead.row_stats(z, 0.5)
    assert st2[0, 0] == 6.0
