"""Seeded draws for one draft-tree round (no method arithmetic here).

Every array is a pure function of (config, master seed, input-set index).  A
master seed is split into independent named streams with numpy's SeedSequence;
large arrays are drawn in fixed-size blocks, each block from its own
SeedSequence child, so the values do not depend on how many threads draw them.

Values that the bf16 workloads store in bf16 are returned as float32 arrays
whose values are exactly representable in bf16 (round-to-nearest-even), so the
oracle can widen them to fp64 exactly and the device can take the high 16 bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from functools import cached_property

import numpy as np

from .configs import RoundConfig

_BLOCK = 1 << 22  # elements per independently seeded block

# Named streams of one master seed.
_STREAMS = ("kvprefix", "tokrows", "lmhead", "roots", "draftnoise",
            "uniforms", "gumbelseed", "prefixlens", "sigmas")


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); float32 out."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """High 16 bits of bf16-representable float32 values, as uint16."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _blocked(master: int, stream: str, set_idx: int, n: int, fill) -> np.ndarray:
    """Fill a flat float32 array of n elements block by block (deterministic)."""
    out = np.empty(n, dtype=np.float32)
    sid = _STREAMS.index(stream)
    nblk = (n + _BLOCK - 1) // _BLOCK

    def work(i):
        ss = np.random.SeedSequence(entropy=master, spawn_key=(sid, set_idx, i))
        rng = np.random.default_rng(ss)
        lo, hi = i * _BLOCK, min(n, (i + 1) * _BLOCK)
        fill(rng, out[lo:hi])

    if nblk == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out


def _normal(master, stream, set_idx, shape, std=1.0):
    n = int(np.prod(shape))

    def fill(rng, dst):
        rng.standard_normal(out=dst, dtype=np.float32)
        if std != 1.0:
            dst *= np.float32(std)

    return _blocked(master, stream, set_idx, n, fill).reshape(shape)


def _rng(master, stream, set_idx):
    return np.random.default_rng(
        np.random.SeedSequence(entropy=master, spawn_key=(_STREAMS.index(stream), set_idx, 1 << 30)))


class RoundInputs:
    """Lazily drawn inputs of one round (input set `set_idx`) of a config.

    Fields shared by every input set (weights, token rows) ignore set_idx.
    Shapes:
      w          [V, H]            LM-head weight, N(0, w_std)
      k_prefix   [B, hkv, Lmax, dh] prefix keys, N(0, 1); positions >= L_b unused
      v_prefix   [B, hkv, Lmax, dh] prefix values
      prefix_len [B]               int32
      q_tab      [V, hq*dh]        per-token query rows of the verify layer
      k_tab      [V, hkv*dh]       per-token key rows
      v_tab      [V, hkv*dh]       per-token value rows
      roots      [B]               int32 root token (last committed token)
      eps        [B, S, V]         N(0,1) draft noise per slot
      sigma      [B]               float32 noise std per request
      uniforms   [B, N, k+1]       float32 in [0, 1): acceptance draws per tree node
      gumbel_seed                  uint64 Philox key for child sampling
    """

    def __init__(self, cfg: RoundConfig, set_idx: int = 0):
        self.cfg = cfg
        self.set_idx = set_idx
        self.master = cfg.seed

    def _maybe_bf16(self, a):
        return bf16_round(a) if self.cfg.dtype == "bf16" else a

    @cached_property
    def w(self):
        c = self.cfg
        return self._maybe_bf16(_normal(self.master, "lmhead", 0, (c.V, c.H), c.w_std))

    @cached_property
    def prefix_len(self):
        c = self.cfg
        lo, hi = c.L
        if lo == hi:
            return np.full(c.B, lo, dtype=np.int32)
        return _rng(self.master, "prefixlens", self.set_idx).integers(lo, hi + 1, size=c.B).astype(np.int32)

    @cached_property
    def _kv(self):
        c = self.cfg
        a = _normal(self.master, "kvprefix", self.set_idx, (2, c.B, c.hkv, c.Lmax, c.dh))
        return self._maybe_bf16(a)

    @property
    def k_prefix(self):
        return self._kv[0]

    @property
    def v_prefix(self):
        return self._kv[1]

    @cached_property
    def _tok(self):
        c = self.cfg
        width = (c.hq + 2 * c.hkv) * c.dh
        return self._maybe_bf16(_normal(self.master, "tokrows", 0, (c.V, width)))

    @property
    def q_tab(self):
        c = self.cfg
        return self._tok[:, : c.hq * c.dh]

    @property
    def k_tab(self):
        c = self.cfg
        return self._tok[:, c.hq * c.dh: (c.hq + c.hkv) * c.dh]

    @property
    def v_tab(self):
        c = self.cfg
        return self._tok[:, (c.hq + c.hkv) * c.dh:]

    @cached_property
    def roots(self):
        c = self.cfg
        return _rng(self.master, "roots", self.set_idx).integers(0, c.V, size=c.B).astype(np.int32)

    @cached_property
    def eps(self):
        c = self.cfg
        return _normal(self.master, "draftnoise", self.set_idx, (c.B, c.S, c.V))

    @cached_property
    def sigma(self):
        c = self.cfg
        lo, hi = c.sigma
        if lo == hi:
            return np.full(c.B, lo, dtype=np.float32)
        return _rng(self.master, "sigmas", self.set_idx).uniform(lo, hi, size=c.B).astype(np.float32)

    @cached_property
    def uniforms(self):
        c = self.cfg
        u = _rng(self.master, "uniforms", self.set_idx).random((c.B, c.N, c.k + 1), dtype=np.float32)
        return u

    @cached_property
    def gumbel_seed(self) -> int:
        return int(_rng(self.master, "gumbelseed", self.set_idx).integers(0, 2**63 - 1, dtype=np.int64))

    def iid_draft_rows(self):
        """Draft rows that do not depend on the target: sigma_b * eps (float32)."""
        return (self.eps * self.sigma[:, None, None]).astype(np.float32)


def make_inputs(cfg: RoundConfig, set_idx: int = 0) -> RoundInputs:
    return RoundInputs(cfg, set_idx)
