"""Parity of eagle_sampling_warp (through the C ABI) with oracle/warp.py.

The kept set of every row must equal the oracle's exactly (compared as the
token mask the returned bound describes), M bit for bit and S to fp32
rounding, except rows where the oracle flags the nucleus cut as a near tie.
Rows cover random logits, heavy exact ties, flat and peaked rows, -inf
entries, vocabularies with a ragged tail and the 8B vocabulary.
"""
import numpy as np
import pytest

from oracle import expand as oexpand
from oracle import warp as owarp

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _codes(t):
    t = np.asarray(t, np.float32) + np.float32(0.0)
    b = t.view(np.uint32)
    return np.where(b >> 31, ~b, b | np.uint32(0x80000000)).astype(np.uint32)


def _rows(kind, R, V, rng):
    if kind == "normal":
        return (rng.standard_normal((R, V)) * 2.0).astype(np.float32)
    if kind == "ties":
        return np.round(rng.standard_normal((R, V)) * 3.0).astype(np.float32)
    if kind == "flat":
        return np.zeros((R, V), np.float32)
    if kind == "peaked":
        z = (rng.standard_normal((R, V)) * 0.5).astype(np.float32)
        z[np.arange(R), rng.integers(0, V, R)] += 30.0
        return z
    if kind == "neginf":
        z = rng.standard_normal((R, V)).astype(np.float32)
        z[rng.random((R, V)) < 0.3] = -np.inf
        return z
    raise ValueError(kind)


def _run(z, top_k, top_p, min_keep, T):
    from eagle_draft_tree_expand_amd import ops
    R, V = z.shape
    dz = torch.from_numpy(z).cuda()
    st = torch.zeros((R, 2), dtype=torch.float32, device="cuda")
    bd = torch.zeros((R, 2), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.sampling_warp(R, V, top_k, top_p, min_keep, T, dz, st, bd, status)
    torch.cuda.synchronize()
    return st.cpu().numpy(), bd.cpu().numpy().view(np.uint32), int(status.item())


WARPS = [(50, 1.0, 1), (0, 0.9, 1), (40, 0.5, 10), (10, 0.95, 10), (1, 1.0, 1), (0, 1.0, 1), (0, 1e-6, 10),
         (2000, 0.99, 1)]


@pytest.mark.parametrize("kind", ["normal", "ties", "flat", "peaked", "neginf"])
@pytest.mark.parametrize("V", [5003, 4096])
def test_warp_matches_oracle(kind, V):
    rng = np.random.default_rng(hash((kind, V)) % 2**32)
    z = _rows(kind, 6, V, rng)
    compared = total = 0
    for T in (1.0, 0.7):
        for top_k, top_p, min_keep in WARPS:
            st, bd, status = _run(z, top_k, top_p, min_keep, T)
            t = oexpand.scaled_logits(z, T)
            codes = _codes(t)
            flagged = 0
            for r in range(z.shape[0]):
                w = owarp.warp_support(z[r], T, top_k, top_p, min_keep)
                if w["tie"]:
                    flagged += 1
                    continue
                mask = (codes[r] > bd[r, 0]) | ((codes[r] == bd[r, 0]) & (np.arange(V) <= bd[r, 1]))
                assert np.array_equal(mask, w["mask"]), (kind, V, T, top_k, top_p, min_keep, r)
                assert st[r, 0] == np.float32(w["M"])
                np.testing.assert_allclose(st[r, 1], w["S"], rtol=2e-7)
                compared += 1
            total += z.shape[0]
            assert bool(status & 0x2) == bool(np.any(~np.isfinite(z)))
    # exact crossings (equal masses) are flagged; most rows are compared
    assert compared >= 0.75 * total, (compared, total)


def test_warp_full_vocab_rows():
    """61 rows of the 8B vocabulary (the verify rows of one request), two warps."""
    rng = np.random.default_rng(11)
    V = 128256
    z = (rng.standard_normal((61, V)) * 0.06).astype(np.float32)   # near-uniform rows, as with random weights
    z[::7] = (rng.standard_normal((9, V)) * 3.0).astype(np.float32)
    for top_k, top_p, min_keep in [(50, 0.9, 10), (0, 0.95, 10)]:
        st, bd, _ = _run(z, top_k, top_p, min_keep, 1.0)
        codes = _codes(z)
        for r in range(61):
            w = owarp.warp_support(z[r], 1.0, top_k, top_p, min_keep)
            if w["tie"]:
                continue
            mask = (codes[r] > bd[r, 0]) | ((codes[r] == bd[r, 0]) & (np.arange(V) <= bd[r, 1]))
            assert np.array_equal(mask, w["mask"]), (top_k, top_p, r)
            np.testing.assert_allclose(st[r, 1], w["S"], rtol=2e-7)
