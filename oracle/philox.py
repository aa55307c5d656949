"""Philox4x32-10 counter-based generator, written from its published definition
(Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC'11): 10 rounds of two 32x32->64 multiplies on a 4-word counter with a
2-word key bumped by the Weyl constants between rounds.

Used only to draw the Gumbel noise for non-greedy child sampling: the pages say
k tokens are sampled per node (EAGLE-1 notes, appendix A.1) but fix no
generator, so the draws are a counter-based function of
(seed, vocab quad, slot, request, round) that both sides compute.
"""
import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four output words for counters (c0..c3) and key (k0, k1).

    Counters broadcast as numpy arrays of uint32-range integers; the key is a
    pair of Python ints.  Result: 4 uint32 arrays.
    """
    c0 = np.asarray(c0, dtype=np.uint64) & _MASK
    c1 = np.asarray(c1, dtype=np.uint64) & _MASK
    c2 = np.asarray(c2, dtype=np.uint64) & _MASK
    c3 = np.asarray(c3, dtype=np.uint64) & _MASK
    k0 = int(k0) & _MASK
    k1 = int(k1) & _MASK
    for r in range(10):
        if r:
            k0 = (k0 + W0) & _MASK
            k1 = (k1 + W1) & _MASK
        p0 = c0 * np.uint64(M0)
        p1 = c2 * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def gumbel_uniforms(vocab: int, slot: int, req: int, round_id: int, seed: int) -> np.ndarray:
    """Uniform draws u_v in (0, 1) for every token v of one slot row.

    Counter (v >> 2, slot, req, round_id mod 2^32), key = (seed low word,
    seed high word); token v takes output word v & 3.  The 32-bit word x is
    mapped to u = (2 * (x >> 9) + 1) * 2^-24, an odd multiple of 2^-24, which
    is exact in fp32 and never 0 or 1.  Returned as float64.
    """
    v = np.arange(vocab, dtype=np.uint64)
    quad = np.arange((vocab + 3) // 4, dtype=np.uint64)
    words = philox4x32_10(quad, slot, req, round_id & _MASK, seed & _MASK, (seed >> 32) & _MASK)
    allw = np.stack(words, axis=1).reshape(-1)[:vocab]
    assert allw.shape[0] == v.shape[0]
    j = (allw >> np.uint32(9)).astype(np.float64)
    return (2.0 * j + 1.0) * 2.0 ** -24
