"""Seeded weights and inputs of a synthetic EAGLE draft head (no method
arithmetic here).

The head has the target's shape (hidden H, hq/hkv heads of dim dh) plus an MLP
width `inter`; weights are random (N(0, 1/fan_in) so activations stay O(1)),
bf16-representable for bf16 workloads.  Per request: the feature that enters
the root's draft step and the draft's own prefix K/V cache (same lengths as
the target's prefix).  The embedding table and LM head are the target's:
`E` is drawn here, the LM head is the round's `w`.
"""
from __future__ import annotations

from functools import cached_property

import numpy as np

from .configs import RoundConfig
from .gen import _threads, bf16_round

_BLOCK = 1 << 22
_DSTREAMS = ("embed", "fc", "wq", "wk", "wv", "wo", "wg", "wu", "wd", "rootfeat", "dkprefix", "dvprefix")

# MLP widths: the Llama-3-8B / Llama-2-13B / Llama-3-70B shapes, else 3H rounded to 128.
INTER = {"8b": 14336, "b64": 14336, "8b_chain": 14336, "13b": 13824, "70b": 28672}


def inter_of(cfg: RoundConfig) -> int:
    return INTER.get(cfg.name, (3 * cfg.H + 127) // 128 * 128)


def _normal(master, stream, set_idx, shape, std):
    from concurrent.futures import ThreadPoolExecutor
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    sid = 100 + _DSTREAMS.index(stream)
    nblk = (n + _BLOCK - 1) // _BLOCK

    def work(i):
        rng = np.random.default_rng(np.random.SeedSequence(entropy=master, spawn_key=(sid, set_idx, i)))
        lo, hi = i * _BLOCK, min(n, (i + 1) * _BLOCK)
        rng.standard_normal(out=out[lo:hi], dtype=np.float32)
        out[lo:hi] *= np.float32(std)

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out.reshape(shape)


class DraftInputs:
    """Lazily drawn arrays (float32, bf16-exact for bf16 workloads)."""

    def __init__(self, cfg: RoundConfig, set_idx: int = 0, inter: int | None = None, cap: int | None = None):
        self.cfg, self.set_idx = cfg, set_idx
        self.master = cfg.seed * 7919 + 17
        self.inter = inter or inter_of(cfg)
        self.cap = cap or cfg.Lmax

    def _w(self, stream, shape, std):
        a = _normal(self.master, stream, 0, shape, std)
        return bf16_round(a) if self.cfg.dtype == "bf16" else a

    @cached_property
    def weights(self):
        c, I = self.cfg, self.inter
        H, Q, KV = c.H, c.hq * c.dh, c.hkv * c.dh
        return {
            "E": self._w("embed", (c.V, H), 1.0),
            "fc": self._w("fc", (H, 2 * H), (2 * H) ** -0.5),
            "q": self._w("wq", (Q, H), H ** -0.5),
            "k": self._w("wk", (KV, H), H ** -0.5),
            "v": self._w("wv", (KV, H), H ** -0.5),
            "o": self._w("wo", (H, Q), Q ** -0.5),
            "g": self._w("wg", (I, H), H ** -0.5),
            "u": self._w("wu", (I, H), H ** -0.5),
            "d": self._w("wd", (H, I), I ** -0.5),
        }

    @cached_property
    def root_feat(self):
        a = _normal(self.master, "rootfeat", self.set_idx, (self.cfg.B, self.cfg.H), 1.0)
        return bf16_round(a) if self.cfg.dtype == "bf16" else a

    def _kv(self, stream):
        c = self.cfg
        a = _normal(self.master, stream, self.set_idx, (c.B, c.hkv, self.cap, c.dh), 1.0)
        return bf16_round(a) if c.dtype == "bf16" else a

    @cached_property
    def k_prefix(self):
        return self._kv("dkprefix")

    @cached_property
    def v_prefix(self):
        return self._kv("dvprefix")


def make_draft_inputs(cfg: RoundConfig, set_idx: int = 0, **kw) -> DraftInputs:
    return DraftInputs(cfg, set_idx, **kw)
