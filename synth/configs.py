"""Workload shapes for one draft-tree round.

Shapes follow the draft-tree sizes the pages quote (depth 8, top-k 10, m = 60 /
50 / 48 draft nodes for 8B / 13B / 70B targets; hubwiz "LLM 推测性解码原理解读"
section 5) and the model dims of the named Llama-3-8B / 13B / 70B shapes.
Everything is synthetic: N(0,1) KV prefix, N(0, 0.02) LM head, seeded.

Symbols: B batch, H hidden, hq/hkv heads, dh head dim, L prefix length,
V vocab, D depth (draft levels), k top-k, m selected draft nodes.
Derived: N = m + 1 tree nodes (root included), S = 1 + (D-1)k expanded slots,
P = k + (D-1)k^2 pool nodes.
"""
from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class RoundConfig:
    name: str
    B: int
    H: int
    hq: int
    hkv: int
    dh: int
    L: Tuple[int, int]          # prefix length range (inclusive); fixed if lo == hi
    V: int
    D: int
    k: int
    m: int
    dtype: str                  # "f32" or "bf16": activations, KV and LM-head weight
    temps: Tuple[float, ...]    # temperatures to run (0.0 = greedy)
    draft: str                  # "iid": rows are sigma * N(0,1); "target": target logits + sigma * N(0,1)
    sigma: Tuple[float, float]  # noise std range (per request, uniform); fixed if lo == hi
    seed: int
    w_std: float = 0.02
    # A static (EAGLE-1) tree: the parent array of its flattened shape (node 0
    # the root) and its number of slots (nodes with children); empty for the
    # dynamic tree.
    static_parent: Tuple[int, ...] = ()
    static_slots: int = 0

    @property
    def N(self) -> int:
        return self.m + 1

    @property
    def S(self) -> int:
        if self.static_parent:
            return self.static_slots
        return 1 + (self.D - 1) * self.k

    @property
    def P(self) -> int:
        return self.k + (self.D - 1) * self.k * self.k

    @property
    def Lmax(self) -> int:
        return self.L[1]

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def with_(self, **kw) -> "RoundConfig":
        return replace(self, **kw)


CONFIGS = {
    # Tiny fp32 case the oracle finishes instantly.
    "tiny": RoundConfig("tiny", B=1, H=64, hq=4, hkv=4, dh=16, L=(32, 32), V=256,
                        D=3, k=2, m=10, dtype="f32", temps=(1.0,), draft="iid",
                        sigma=(2.0, 2.0), seed=101),
    # Llama-3-8B-shaped verify layer, batch 1.
    "8b": RoundConfig("8b", B=1, H=4096, hq=32, hkv=8, dh=128, L=(2048, 2048), V=128256,
                      D=8, k=10, m=60, dtype="bf16", temps=(1.0, 0.0), draft="target",
                      sigma=(1.0, 1.0), seed=202),
    # 13B-shaped (MHA), batch 1.
    "13b": RoundConfig("13b", B=1, H=5120, hq=40, hkv=40, dh=128, L=(4096, 4096), V=32000,
                       D=8, k=10, m=50, dtype="bf16", temps=(1.0,), draft="target",
                       sigma=(1.5, 1.5), seed=303),
    # 70B-shaped single-layer share, batch 1.
    "70b": RoundConfig("70b", B=1, H=8192, hq=64, hkv=8, dh=128, L=(4096, 4096), V=32000,
                       D=8, k=10, m=48, dtype="bf16", temps=(1.0, 0.0), draft="target",
                       sigma=(1.0, 1.0), seed=404),
    # Batched 8B shape, ragged prefixes, per-request noise level.
    "b64": RoundConfig("b64", B=64, H=4096, hq=32, hkv=8, dh=128, L=(512, 4096), V=128256,
                       D=8, k=10, m=60, dtype="bf16", temps=(1.0,), draft="target",
                       sigma=(0.5, 2.0), seed=505),
}

# The 8B shape drafting a chain instead of a tree (top-k 1: each depth expands
# its single child; m = D draft tokens), for the tree-vs-chain comparison.
CONFIGS["8b_chain"] = CONFIGS["8b"].with_(name="8b_chain", k=1, m=8, temps=(1.0,))

# A static EAGLE-1-style tree (EAGLE-1 notes, appendix A.1: the root has 4
# children, 5 draft passes fill it, branches of more probable tokens are deeper
# and wider): 22 draft nodes over depth 5, 14 of them slots.  Flat (BFS) order;
# node i's parent is STATIC_SHAPE[i].  This build's own shape following those
# rules; the pages do not reproduce the figure itself.
STATIC_SHAPE = (-1, 0, 0, 0, 0, 1, 1, 1, 2, 2, 3, 4, 5, 5, 6, 8, 10, 12, 12, 14, 15, 17, 19)
CONFIGS["8b_static"] = CONFIGS["8b"].with_(name="8b_static", D=5, k=4, m=len(STATIC_SHAPE) - 1,
                                          static_parent=STATIC_SHAPE, static_slots=14)
# The chain with as many draft passes (EAGLE-1 notes, tree-attention ablation: a
# chain and a tree drafted with the same number of forward passes).
CONFIGS["8b_chain5"] = CONFIGS["8b"].with_(name="8b_chain5", D=5, k=1, m=5, temps=(1.0,))
# The 8B workload with draft rows close to the target's: noise sigma 0.01 in
# place of 1, against target logits that spread ~0.03 (random weights), so the
# draft's and the target's top-50 tokens partly agree and rounds under top-k /
# top-p warps accept draft tokens too (measured: warped tau 1.75, unwarped 2.65;
# sigma 0 gives 2.0 and 2.55, sigma 0.02 1.5 and 2.6).
CONFIGS["8b_close"] = CONFIGS["8b"].with_(name="8b_close", sigma=(0.01, 0.01), temps=(1.0,))

# Reduced shapes for element-by-element parity: several tiles and ragged tails
# in every dimension (vocab not a multiple of the 256-column tile, prefix not a
# multiple of the key chunk), yet small enough for the oracle in seconds.
CONFIGS.update({
    "mid_bf16": RoundConfig("mid_bf16", B=3, H=512, hq=4, hkv=2, dh=128, L=(70, 333), V=5003,
                            D=4, k=3, m=14, dtype="bf16", temps=(1.0, 0.7, 0.0), draft="target",
                            sigma=(0.5, 2.0), seed=606),
    "mid_f32": RoundConfig("mid_f32", B=2, H=128, hq=4, hkv=2, dh=32, L=(40, 300), V=3001,
                           D=4, k=3, m=9, dtype="f32", temps=(1.0, 0.0), draft="target",
                           sigma=(1.0, 1.0), seed=707),
})


# The static shape at the reduced parity size.
CONFIGS["mid_static"] = CONFIGS["mid_bf16"].with_(name="mid_static", D=5, k=4, m=len(STATIC_SHAPE) - 1,
                                                  static_parent=STATIC_SHAPE, static_slots=14)
CONFIGS["tiny_static"] = CONFIGS["tiny"].with_(name="tiny_static", D=5, k=4, m=len(STATIC_SHAPE) - 1,
                                               static_parent=STATIC_SHAPE, static_slots=14)


def get_config(name: str) -> RoundConfig:
    return CONFIGS[name]
