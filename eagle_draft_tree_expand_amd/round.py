"""One draft-tree round on the device, wired through the C ABI.

`DeviceRound` owns the device buffers of a workload shape and runs

    expand -> mask -> (gather tree q/k/v rows) -> tree attention -> LM head -> accept

on the current HIP stream, every step in libeagle's kernels, and `commit`
appends the accepted path to the prefix cache for the next round.  `DeviceInputs`
holds one input set on the device.  `device_draft_rows` builds the synthetic
draft rows "target logits + noise" slot by slot with the same kernels (the
ancestor-only mask makes a node's target logits depend on its root path only,
so they can be computed before the tree exists).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import ops

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _t(a, dtype=None, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


class DeviceWeights:
    """Inputs shared by every input set: LM-head weight and per-token q/k/v rows."""

    def __init__(self, inp, device="cuda", packed=True, zpacked=True):
        c = inp.cfg
        dt = _TORCH_DT[c.dtype]
        self.w = _t(inp.w, dt, device)
        # bf16 weights are also packed once into the MFMA-native streaming layout,
        # and into its lossless 12-bit form, which the streaming kernel (verify
        # rounds of at most EAGLE_ZPACK_MAX_ROWS rows) reads instead
        self.packed = packed and c.dtype == "bf16"
        self.w_packed = ops.pack_lmhead_weight(self.w) if self.packed else None
        self.w_z, self.z_raw = None, 0
        if self.packed and zpacked and ops.zpack_supported(c.V, c.H):
            self.w_z, self.z_raw = ops.zpack_lmhead_weight(self.w)
        self.q_tab = _t(inp.q_tab, dt, device)
        self.k_tab = _t(inp.k_tab, dt, device)
        self.v_tab = _t(inp.v_tab, dt, device)

    def lm_weight(self, rows):
        """(tensor, layout flag for ops) of the LM-head weight a launch of `rows` rows reads."""
        if self.w_z is not None and rows <= ops.ZPACK_MAX_ROWS:
            return self.w_z, "z"
        return (self.w_packed, True) if self.packed else (self.w, False)


class DeviceInputs:
    """One input set: prefix KV, prefix lengths, roots, uniforms, draft rows, noise.

    `room` extra cache positions per request (zero-filled) leave space for
    committed paths; the cache stride is then `cap` = Lmax + room."""

    def __init__(self, inp, device="cuda", with_eps=False, room=0):
        c = inp.cfg
        dt = _TORCH_DT[c.dtype]
        self.cap = c.Lmax + int(room)
        self.k_prefix = self._cache(inp.k_prefix, dt, device)
        self.v_prefix = self._cache(inp.v_prefix, dt, device)
        self.prefix_len = _t(inp.prefix_len, torch.int32, device)
        self.roots = _t(inp.roots, torch.int32, device)
        self.uniforms = _t(inp.uniforms, torch.float32, device)
        self.seed = inp.gumbel_seed
        self.sigma = inp.sigma
        self.rows = torch.zeros((c.B, c.S, c.V), dtype=torch.float32, device=device)
        self.eps = _t(inp.eps, torch.float32, device) if with_eps else None

    def _cache(self, a, dt, device):
        t = _t(a, dt, device)
        if self.cap == t.shape[2]:
            return t
        out = torch.zeros((t.shape[0], t.shape[1], self.cap, t.shape[3]), dtype=dt, device=device)
        out[:, :, :t.shape[2]] = t
        return out

    def set_rows(self, rows_np):
        self.rows.copy_(torch.from_numpy(np.ascontiguousarray(rows_np, dtype=np.float32)))


class DeviceRound:
    """Device buffers + the five entry points of one round for a config."""

    def __init__(self, cfg, device="cuda", n=None, B=None, cap=None, compact=False):
        self.cfg = c = cfg
        # compact target rows (fp16 offsets + 128-column block maxima) instead of fp32 logits
        self.compact = bool(compact)
        self.cap = cap or c.Lmax  # largest prefix-cache stride the workspace is sized for
        self.B = B = B or c.B
        self.N = N = n or c.N
        self.dev = device
        dt = _TORCH_DT[c.dtype]
        i32, f32 = torch.int32, torch.float32
        z = lambda *s, dtype=i32: torch.zeros(s, dtype=dtype, device=device)  # noqa: E731
        self.tree = {k: z(B, N) for k in ("node_tok", "node_parent", "node_depth", "node_sib", "node_slot")}
        self.tree["node_value"] = z(B, N, dtype=f32)
        self.tree["node_q"] = z(B, N, dtype=f32)
        self.tree["pool_tok"] = z(B, c.S, c.k)
        self.tree["pool_q"] = z(B, c.S, c.k, dtype=f32)
        self.tree["pool_flat"] = z(B, c.S, c.k)
        self.tree["slot_src"] = z(B, c.S)
        self.tree["slot_stats"] = z(B, c.S, 2, dtype=f32)
        W = (N + 63) // 64
        self.mask = torch.zeros((B, N, W), dtype=torch.int64, device=device)
        self.pos = z(B, N)
        self.q = torch.zeros((B, N, c.hq, c.dh), dtype=dt, device=device)
        self.kt = torch.zeros((B, N, c.hkv, c.dh), dtype=dt, device=device)
        self.vt = torch.zeros((B, N, c.hkv, c.dh), dtype=dt, device=device)
        self.x = torch.zeros((B, N, c.hq, c.dh), dtype=dt, device=device)
        self.feat = torch.zeros((B, c.D + 1, c.H), dtype=dt, device=device)
        if self.compact:
            self.logits = None
            self.z16 = torch.zeros((B * N, c.V), dtype=torch.float16, device=device)
            self.bmax = torch.zeros((B * N, (c.V + 127) // 128), dtype=f32, device=device)
        else:
            self.logits = torch.zeros((B * N, c.V), dtype=f32, device=device)
        self.stats = z(B * N, 2, dtype=f32)
        self.argmax = z(B * N)
        # sampling-warp outputs: bounds of the draft slot rows and of the target rows, warped target stats
        self.d_bound = z(B * c.S, 2)
        self.d_wstats = z(B * c.S, 2, dtype=f32)
        self.t_bound = z(B * N, 2)
        self.t_wstats = z(B * N, 2, dtype=f32)
        self.acc = {"accept_len": z(B), "accept_path": z(B, c.D), "committed": z(B, c.D + 1),
                    "n_committed": z(B), "near_tie": z(B)}
        self.status = z(1)
        self.scale = float(np.float32(1.0 / math.sqrt(c.dh)))
        self.static = tuple(c.static_parent) if c.static_parent else None
        if self.static:
            p = self.params(1.0)
            nbytes = ops.static_workspace_size(p, self.static, c.hq, c.hkv, c.dh, self.cap, c.H)
        else:
            p = self.params(1.0, m=min(max(self.N - 1, 1), c.P))  # sizing only: at least one draft node
            nbytes = ops.workspace_size(p, c.hq, c.hkv, c.dh, self.cap, c.H)
        if nbytes == 0:
            raise ValueError("invalid round shape")
        self.ws = ops.new_workspace(nbytes, device)

    def params(self, T, round_id=0, seed=0, depth=None, m=None):
        c = self.cfg
        return ops.tree_params(self.B, c.V, depth or c.D, c.k, m or (self.N - 1), T, seed, round_id)

    # -- the stages -----------------------------------------------------------
    def expand(self, data, T, round_id=0, warp=None):
        """warp = (top_k, top_p) with T > 0: the draft rows are warped first (at least k tokens kept)."""
        c = self.cfg
        if self.static:
            if warp is not None:
                raise ValueError("static trees take no sampling warp")
            ops.expand_static(self.params(T, round_id, data.seed), self.static, data.rows, data.roots, self.tree,
                              self.ws, self.status)
            return
        bound = None
        if warp is not None and T > 0:
            ops.sampling_warp(self.B * c.S, c.V, warp[0], warp[1], c.k, T, data.rows, self.d_wstats, self.d_bound,
                              self.status)
            bound = self.d_bound
        ops.expand_tree(self.params(T, round_id, data.seed), data.rows, data.roots, self.tree, self.ws, self.status,
                        draft_bound=bound)

    def mask_pos(self, data):
        ops.build_tree_mask(self.B, self.N, self.tree["node_parent"], self.tree["node_depth"], data.prefix_len,
                            self.mask, self.pos, self.status)

    def gather_qkv(self, wts, node_tok=None):
        c = self.cfg
        tok = (node_tok if node_tok is not None else self.tree["node_tok"]).reshape(-1)
        n = tok.numel()
        ops.gather_rows_multi(n, tok, [(wts.q_tab, self.q), (wts.k_tab, self.kt), (wts.v_tab, self.vt)], self.status)

    def attention(self, data):
        c = self.cfg
        ops.tree_attention(self.B, self.N, c.hq, c.hkv, c.dh, data.cap, self.q, data.k_prefix, data.v_prefix,
                           data.prefix_len, self.kt, self.vt, self.mask, self.scale, self.x, self.ws, self.status)

    def lmhead(self, wts, T):
        c = self.cfg
        w, layout = wts.lm_weight(self.B * self.N)
        if self.compact:
            ops.lmhead_softmax_compact(self.B * self.N, c.H, c.V, self.x.view(self.B * self.N, c.H), w, T, self.z16,
                                       self.bmax, self.stats, self.argmax, self.ws, status=self.status,
                                       packed=layout)
            return
        ops.lmhead_softmax(self.B * self.N, c.H, c.V, self.x.view(self.B * self.N, c.H), w, T, self.logits,
                           self.stats, self.argmax, self.ws, status=self.status, packed=layout)

    def accept(self, data, T, round_id=0, warp=None):
        """warp = (top_k, top_p) with T > 0: the target rows are warped first, the draft rows were
        warped by expand (their bounds are reused)."""
        c = self.cfg
        if self.compact:
            if warp is not None:
                raise ValueError("compact target rows take no sampling warp")
            ops.verify_accept_compact(self.params(T, round_id, data.seed), c.S if self.static else 0, self.tree,
                                      self.z16, self.bmax, self.stats, self.argmax, data.rows,
                                      self.tree["slot_stats"], data.uniforms, self.acc, self.ws, self.status)
            return
        if self.static:
            ops.verify_accept_static(self.params(T, round_id, data.seed), c.S, self.tree, self.logits, self.stats,
                                     self.argmax, data.rows, self.tree["slot_stats"], data.uniforms, self.acc,
                                     self.ws, self.status)
            return
        if warp is not None and T > 0:
            ops.sampling_warp(self.B * self.N, c.V, warp[0], warp[1], c.k, T, self.logits, self.t_wstats,
                              self.t_bound, self.status)
            ops.verify_accept(self.params(T, round_id, data.seed), self.tree, self.logits, self.t_wstats, self.argmax,
                              data.rows, self.tree["slot_stats"], data.uniforms, self.acc, self.ws, self.status,
                              target_bound=self.t_bound, draft_bound=self.d_bound)
            return
        ops.verify_accept(self.params(T, round_id, data.seed), self.tree, self.logits, self.stats, self.argmax,
                          data.rows, self.tree["slot_stats"], data.uniforms, self.acc, self.ws, self.status)

    def commit(self, data):
        """Append the accepted path's keys/values to data's prefix cache, grow its
        lengths, and write the path's features to self.feat [B, D + 1, H]."""
        c = self.cfg
        ops.commit_accepted(self.B, self.N, c.hkv, c.dh, data.cap, c.H, c.D, self.acc["accept_len"],
                            self.acc["accept_path"], self.kt, self.vt, self.x, data.k_prefix, data.v_prefix,
                            data.prefix_len, self.feat, self.status)

    def expand_masked(self, data, T, round_id=0):
        """expand + mask_pos in one call (dynamic trees without a warp)."""
        ops.expand_tree_masked(self.params(T, round_id, data.seed), data.rows, data.roots, data.prefix_len,
                               self.tree, self.mask, self.pos, self.ws, self.status)

    def step(self, wts, data, T, round_id=0, warp=None):
        """One whole round (the expansion with the mask written by its assembly step,
        the q/k/v row gathers, attention, LM head, acceptance; with a sampling warp or
        a static tree, the expansion and the mask are separate calls, and a warp
        adds the two row warps)."""
        if warp is None and not self.static:
            self.expand_masked(data, T, round_id)
        else:
            self.expand(data, T, round_id, warp)
            self.mask_pos(data)
        self.gather_qkv(wts)
        self.attention(data)
        self.lmhead(wts, T)
        self.accept(data, T, round_id, warp)

    def host(self):
        """Copy every output to host numpy arrays (synchronises)."""
        out = {k: v.cpu().numpy() for k, v in self.tree.items()}
        out.update({k: v.cpu().numpy() for k, v in self.acc.items()})
        out["mask"] = self.mask.cpu().numpy().view(np.uint64)
        out["pos"] = self.pos.cpu().numpy()
        out["x"] = self.x.float().cpu().numpy()
        if self.compact:
            out["z16"] = self.z16.cpu().numpy()
            out["bmax"] = self.bmax.cpu().numpy()
        else:
            out["logits"] = self.logits.cpu().numpy()
        out["stats"] = self.stats.cpu().numpy()
        out["argmax"] = self.argmax.cpu().numpy()
        out["status"] = int(self.status.item())
        return out


def device_draft_rows(cfg, wts, data, T, round_id=0, device="cuda"):
    """Fill data.rows with synthetic draft rows, slot by slot, on the device.

    Slot s of request b gets the target logits at the node it expands
    (attention on the node's root path alone, then the LM head) plus
    sigma_b * eps[b, s].  Workloads marked "iid" get sigma_b * eps directly.
    Frontier nodes are found with eagle_expand_tree itself, depth by depth.
    """
    c = cfg
    if data.eps is None:
        raise ValueError("input set was created without noise")
    sig = torch.from_numpy(np.asarray(data.sigma, np.float32)).to(device).view(c.B, 1)
    if c.draft == "iid":
        data.rows.copy_(data.eps * sig.view(c.B, 1, 1))
        return
    data.rows.zero_()
    for d in range(c.D):
        # frontier of depth d: slot 0 (root) or the k slots 1+(d-1)k+i
        if d == 0:
            paths = [[[int(r)]] for r in data.roots.cpu().numpy()]
            slots = [0]
        else:
            Sd = 1 + d * c.k
            Pd = Sd * c.k
            part = DeviceRound(c.with_(D=d + 1, m=min(c.m, Pd)), device, n=min(c.m, Pd) + 1)
            tmp = DeviceInputs.__new__(DeviceInputs)
            tmp.rows = data.rows[:, :Sd].contiguous()
            tmp.roots, tmp.seed = data.roots, data.seed
            part.expand(tmp, T, round_id)
            pool_tok = part.tree["pool_tok"].cpu().numpy()
            slot_src = part.tree["slot_src"].cpu().numpy()
            slots = [1 + (d - 1) * c.k + i for i in range(c.k)]
            paths = []
            for b in range(c.B):
                pb = []
                for s in slots:
                    toks, e = [], int(slot_src[b, s])
                    while e >= 0:
                        toks.append(int(pool_tok[b, e // c.k, e % c.k]))
                        e = int(slot_src[b, e // c.k]) if e // c.k > 0 else -1
                    pb.append([int(data.roots[b].item())] + toks[::-1])
                paths.append(pb)
        _rows_on_paths(c, wts, data, slots, paths, T, d, sig, device)
    torch.cuda.synchronize()


def _rows_on_paths(c, wts, data, slots, paths, T, d, sig, device):
    """data.rows[:, s] = target logits at the end of paths[b][i] (length d + 1) + sigma_b * eps[:, s]
    for slots[i]: one mini tree per request, the root plus one chain per path (no sharing)."""
    nf = len(slots)
    n = 1 + nf * d
    tok = np.zeros((c.B, n), np.int32)
    par = np.full((c.B, n), -1, np.int32)
    dep = np.zeros((c.B, n), np.int32)
    ends = []
    for i in range(nf):
        for t in range(d):
            j = 1 + i * d + t
            par[:, j] = 0 if t == 0 else j - 1
            dep[:, j] = t + 1
        ends.append(1 + i * d + d - 1 if d > 0 else 0)
    for b in range(c.B):
        tok[b, 0] = paths[b][0][0]
        for i in range(nf):
            for t in range(d):
                tok[b, 1 + i * d + t] = paths[b][i][t + 1]
    # the mini trees are plain flattened trees (no static shape)
    mini = DeviceRound(c.with_(static_parent=(), static_slots=0), device, n=n)
    mini.tree["node_parent"].copy_(torch.from_numpy(par))
    mini.tree["node_depth"].copy_(torch.from_numpy(dep))
    mini.tree["node_tok"].copy_(torch.from_numpy(tok))
    mini.mask_pos(data)
    mini.gather_qkv(wts)
    mini.attention(data)
    mini.lmhead(wts, T)
    z = mini.logits.view(c.B, n, c.V)
    for i, s in enumerate(slots):
        data.rows[:, s] = z[:, ends[i]] + sig * data.eps[:, s]


def device_static_rows(cfg, wts, data, T, round_id=0, device="cuda"):
    """device_draft_rows for a static shape: the rows of the slots at depth d
    are the target logits on their nodes' root paths (plus noise), once the
    slots above have drawn the tokens of those paths."""
    c = cfg
    if data.eps is None:
        raise ValueError("input set was created without noise")
    par = list(c.static_parent)
    n = len(par)
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[par[i]] + 1
    slot_node = [i for i in range(n) if any(par[j] == i for j in range(i + 1, n))]
    sig = torch.from_numpy(np.asarray(data.sigma, np.float32)).to(device).view(c.B, 1)
    data.rows.zero_()
    rnd = DeviceRound(c, device)
    for d in range(c.D):
        slots = [s for s, u in enumerate(slot_node) if depth[u] == d]
        if not slots:
            continue
        rnd.expand(data, T, round_id)
        tok = rnd.tree["node_tok"].cpu().numpy()
        paths = []
        for b in range(c.B):
            pb = []
            for s in slots:
                u, seq = slot_node[s], []
                while u >= 0:
                    seq.append(int(tok[b, u]))
                    u = par[u]
                pb.append(seq[::-1])
            paths.append(pb)
        _rows_on_paths(c, wts, data, slots, paths, T, d, sig, device)
    torch.cuda.synchronize()
