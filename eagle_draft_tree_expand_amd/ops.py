"""The five round entry points (and helpers) on torch device tensors.

Thin wrappers over the C ABI: they check tensor dtypes/shapes, pass raw device
pointers and the current HIP stream, and raise EagleError on a non-zero return
code.  No computation happens here.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import EAGLE_BF16, EAGLE_F32, EAGLE_W_PACKED, EAGLE_W_ROWMAJOR, EAGLE_W_ZPACKED, DraftDims, DraftWeights, TreeParams, check

_DT = {torch.float32: EAGLE_F32, torch.bfloat16: EAGLE_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def tree_params(batch, vocab, depth, topk, m, temperature, seed=0, round_id=0) -> TreeParams:
    return TreeParams(int(batch), int(vocab), int(depth), int(topk), int(m), float(temperature),
                      int(seed) & (2**64 - 1), int(round_id) & (2**64 - 1))


def workspace_size(p: TreeParams, hq=0, hkv=0, head_dim=0, max_prefix=0, hidden=0) -> int:
    return int(_lib.load().eagle_workspace_size(p, hq, hkv, head_dim, max_prefix, hidden))


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    check("eagle_workspace_init", _lib.load().eagle_workspace_init(_ptr(ws), nbytes, _stream()))
    return ws


def expand_tree(p: TreeParams, draft_logits, root_token, out, ws, status=None, draft_bound=None):
    """out: dict with node_tok/node_parent/node_depth/node_sib/node_slot/node_value/node_q,
    pool_tok/pool_q/pool_flat, slot_src, slot_stats (device tensors).  draft_bound: the draft
    rows' sampling-warp bounds (eagle_sampling_warp), or None."""
    assert draft_logits.dtype == torch.float32 and draft_logits.is_contiguous()
    lib = _lib.load()
    pre = (p, _ptr(draft_logits), _ptr(draft_bound)) if draft_bound is not None else (p, _ptr(draft_logits))
    fn = lib.eagle_expand_tree_warped if draft_bound is not None else lib.eagle_expand_tree
    rc = fn(
        *pre, _ptr(root_token),
        _ptr(out["node_tok"]), _ptr(out["node_parent"]), _ptr(out["node_depth"]), _ptr(out["node_sib"]),
        _ptr(out["node_slot"]), _ptr(out["node_value"]), _ptr(out["node_q"]),
        _ptr(out["pool_tok"]), _ptr(out["pool_q"]), _ptr(out["pool_flat"]), _ptr(out["slot_src"]),
        _ptr(out["slot_stats"]), _ptr(ws), ws.numel(), _ptr(status), _stream())
    check("eagle_expand_tree_warped" if draft_bound is not None else "eagle_expand_tree", rc)


def expand_tree_masked(p: TreeParams, draft_logits, root_token, prefix_len, out, mask, pos, ws, status=None):
    """expand_tree and build_tree_mask in one call (the assembly writes the mask and positions)."""
    assert draft_logits.dtype == torch.float32 and draft_logits.is_contiguous()
    rc = _lib.load().eagle_expand_tree_masked(
        p, _ptr(draft_logits), _ptr(root_token), _ptr(prefix_len),
        _ptr(out["node_tok"]), _ptr(out["node_parent"]), _ptr(out["node_depth"]), _ptr(out["node_sib"]),
        _ptr(out["node_slot"]), _ptr(out["node_value"]), _ptr(out["node_q"]),
        _ptr(out["pool_tok"]), _ptr(out["pool_q"]), _ptr(out["pool_flat"]), _ptr(out["slot_src"]),
        _ptr(out["slot_stats"]), _ptr(mask), _ptr(pos), _ptr(ws), ws.numel(), _ptr(status), _stream())
    check("eagle_expand_tree_masked", rc)


def expand_tree_noalloc(p: TreeParams, draft_logits, root_token, out, status=None):
    """eagle_expand_tree without a workspace: the library's static scratch holds the records."""
    assert draft_logits.dtype == torch.float32 and draft_logits.is_contiguous()
    rc = _lib.load().eagle_expand_tree_noalloc(
        p, _ptr(draft_logits), _ptr(root_token),
        _ptr(out["node_tok"]), _ptr(out["node_parent"]), _ptr(out["node_depth"]), _ptr(out["node_sib"]),
        _ptr(out["node_slot"]), _ptr(out["node_value"]), _ptr(out["node_q"]),
        _ptr(out["pool_tok"]), _ptr(out["pool_q"]), _ptr(out["pool_flat"]), _ptr(out["slot_src"]),
        _ptr(out["slot_stats"]), _ptr(status), _stream())
    check("eagle_expand_tree_noalloc", rc)


def build_tree_mask(batch, n, node_parent, node_depth, prefix_len, mask, pos, status=None):
    rc = _lib.load().eagle_build_tree_mask(batch, n, _ptr(node_parent), _ptr(node_depth), _ptr(prefix_len),
                                          _ptr(mask), _ptr(pos), _ptr(status), _stream())
    check("eagle_build_tree_mask", rc)


def tree_attention(batch, n, hq, hkv, head_dim, max_prefix, q, k_prefix, v_prefix, prefix_len, k_tree, v_tree,
                   mask, scale, out, ws, status=None):
    dt = _DT[q.dtype]
    rc = _lib.load().eagle_tree_attention(batch, n, hq, hkv, head_dim, max_prefix, dt, _ptr(q), _ptr(k_prefix),
                                         _ptr(v_prefix), _ptr(prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(mask),
                                         float(scale), _ptr(out), _ptr(ws), ws.numel(), _ptr(status), _stream())
    check("eagle_tree_attention", rc)


def lmhead_softmax(rows, hidden, vocab, x, w, temperature, logits, row_stats, row_argmax, ws, probs=None,
                   status=None, packed=False):
    dt = _DT[x.dtype]
    layout = _layout(packed)
    rc = _lib.load().eagle_lmhead_softmax(rows, hidden, vocab, dt, _ptr(x), _ptr(w), layout, float(temperature),
                                         _ptr(logits), _ptr(row_stats), _ptr(row_argmax), _ptr(probs), _ptr(ws),
                                         ws.numel(), _ptr(status), _stream())
    check("eagle_lmhead_softmax", rc)


def _layout(packed):
    """packed: False (row-major), True (packed) or "z" (z-packed)."""
    if packed == "z":
        return EAGLE_W_ZPACKED
    return EAGLE_W_PACKED if packed else EAGLE_W_ROWMAJOR


ZPACK_MAX_ROWS = 192  # EAGLE_ZPACK_MAX_ROWS: the streaming kernel's row range


def zpack_supported(vocab, hidden):
    return int(_lib.load().eagle_lmhead_zpack_bytes(vocab, hidden)) > 0


def zpack_lmhead_weight(w):
    """z-packed copy of a row-major bf16 LM-head weight [vocab, hidden] (new
    device tensor) and the number of its fragments kept raw (synchronises)."""
    vocab, hidden = w.shape
    n = int(_lib.load().eagle_lmhead_zpack_bytes(vocab, hidden))
    if n == 0:
        raise ValueError("no z-packed layout for this shape")
    wz = torch.empty(n, dtype=torch.uint8, device=w.device)
    raw = torch.zeros(1, dtype=torch.int32, device=w.device)
    check("eagle_lmhead_zpack_weight",
          _lib.load().eagle_lmhead_zpack_weight(vocab, hidden, _ptr(w), _ptr(wz), _ptr(raw), _stream()))
    return wz, int(raw.item())


def pack_lmhead_weight(w):
    """Packed copy of a row-major bf16 LM-head weight [vocab, hidden] (new device tensor)."""
    vocab, hidden = w.shape
    n = int(_lib.load().eagle_lmhead_packed_bytes(vocab, hidden, EAGLE_BF16))
    if n == 0:
        raise ValueError("no packed layout for this shape/dtype")
    wp = torch.empty(n // 2, dtype=torch.bfloat16, device=w.device)
    check("eagle_lmhead_pack_weight",
          _lib.load().eagle_lmhead_pack_weight(vocab, hidden, EAGLE_BF16, _ptr(w), _ptr(wp), _stream()))
    return wp


def verify_accept(p: TreeParams, tree, target_logits, target_stats, target_argmax, draft_logits, slot_stats,
                  uniforms, out, ws, status=None, target_bound=None, draft_bound=None):
    lib = _lib.load()
    warped = target_bound is not None or draft_bound is not None
    pre = (p, _ptr(target_bound), _ptr(draft_bound)) if warped else (p,)
    rc = (lib.eagle_verify_accept_warped if warped else lib.eagle_verify_accept)(
        *pre, _ptr(tree["node_tok"]), _ptr(tree["node_parent"]), _ptr(tree["node_slot"]), _ptr(tree["pool_tok"]),
        _ptr(tree["pool_flat"]), _ptr(target_logits), _ptr(target_stats), _ptr(target_argmax),
        _ptr(draft_logits), _ptr(slot_stats), _ptr(uniforms), _ptr(out["accept_len"]), _ptr(out["accept_path"]),
        _ptr(out["committed"]), _ptr(out["n_committed"]), _ptr(out["near_tie"]), _ptr(ws), ws.numel(),
        _ptr(status), _stream())
    check("eagle_verify_accept", rc)


def _shape_arg(shape_parent):
    arr = (ctypes.c_int32 * len(shape_parent))(*[int(x) for x in shape_parent])
    return arr


def static_tree_info(shape_parent):
    """(n_slots, depth, kmax, slot_k list) of a static shape (parent array, host)."""
    n = len(shape_parent)
    arr = _shape_arg(shape_parent)
    ns, d, km = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    sk = (ctypes.c_int32 * n)()
    rc = _lib.load().eagle_static_tree_info(n, arr, ctypes.byref(ns), ctypes.byref(d), ctypes.byref(km), sk)
    check("eagle_static_tree_info", rc)
    return ns.value, d.value, km.value, [sk[i] for i in range(ns.value)]


def static_workspace_size(p: TreeParams, shape_parent, hq=0, hkv=0, head_dim=0, max_prefix=0, hidden=0) -> int:
    return int(_lib.load().eagle_static_workspace_size(p, len(shape_parent), _shape_arg(shape_parent), hq, hkv,
                                                       head_dim, max_prefix, hidden))


def expand_static(p: TreeParams, shape_parent, draft_logits, root_token, out, ws, status=None):
    """A static shape filled for every request (out: the same dict as expand_tree's)."""
    assert draft_logits.dtype == torch.float32 and draft_logits.is_contiguous()
    rc = _lib.load().eagle_expand_static(
        p, len(shape_parent), _shape_arg(shape_parent), _ptr(draft_logits), _ptr(root_token),
        _ptr(out["node_tok"]), _ptr(out["node_parent"]), _ptr(out["node_depth"]), _ptr(out["node_sib"]),
        _ptr(out["node_slot"]), _ptr(out["node_value"]), _ptr(out["node_q"]),
        _ptr(out["pool_tok"]), _ptr(out["pool_q"]), _ptr(out["pool_flat"]), _ptr(out["slot_src"]),
        _ptr(out["slot_stats"]), _ptr(ws), ws.numel(), _ptr(status), _stream())
    check("eagle_expand_static", rc)


def verify_accept_static(p: TreeParams, n_slots, tree, target_logits, target_stats, target_argmax, draft_logits,
                         slot_stats, uniforms, out, ws, status=None):
    rc = _lib.load().eagle_verify_accept_static(
        p, int(n_slots), _ptr(tree["node_tok"]), _ptr(tree["node_parent"]), _ptr(tree["node_slot"]),
        _ptr(tree["pool_tok"]), _ptr(tree["pool_flat"]), _ptr(target_logits), _ptr(target_stats),
        _ptr(target_argmax), _ptr(draft_logits), _ptr(slot_stats), _ptr(uniforms), _ptr(out["accept_len"]),
        _ptr(out["accept_path"]), _ptr(out["committed"]), _ptr(out["n_committed"]), _ptr(out["near_tie"]), _ptr(ws),
        ws.numel(), _ptr(status), _stream())
    check("eagle_verify_accept_static", rc)


def lmhead_softmax_compact(rows, hidden, vocab, x, w, temperature, z16, block_max, row_stats, row_argmax, ws,
                           status=None, packed=False):
    """The LM head without fp32 rows: z16 [rows, V] fp16 offsets, block_max [rows, ceil(V/128)]."""
    assert z16.dtype == torch.float16 and block_max.dtype == torch.float32
    layout = _layout(packed)
    rc = _lib.load().eagle_lmhead_softmax_compact(rows, hidden, vocab, _ptr(x), _ptr(w), layout, float(temperature),
                                                 _ptr(z16), _ptr(block_max), _ptr(row_stats), _ptr(row_argmax),
                                                 _ptr(ws), ws.numel(), _ptr(status), _stream())
    check("eagle_lmhead_softmax_compact", rc)


def verify_accept_compact(p: TreeParams, n_slots, tree, z16, block_max, target_stats, target_argmax, draft_logits,
                          slot_stats, uniforms, out, ws, status=None):
    """The walk on compact target rows (n_slots 0: dynamic tree; > 0: static tree)."""
    rc = _lib.load().eagle_verify_accept_compact(
        p, int(n_slots), _ptr(tree["node_tok"]), _ptr(tree["node_parent"]), _ptr(tree["node_slot"]),
        _ptr(tree["pool_tok"]), _ptr(tree["pool_flat"]), _ptr(z16), _ptr(block_max), _ptr(target_stats),
        _ptr(target_argmax), _ptr(draft_logits), _ptr(slot_stats), _ptr(uniforms), _ptr(out["accept_len"]),
        _ptr(out["accept_path"]), _ptr(out["committed"]), _ptr(out["n_committed"]), _ptr(out["near_tie"]), _ptr(ws),
        ws.numel(), _ptr(status), _stream())
    check("eagle_verify_accept_compact", rc)


def gather_rows(n_rows, row_elems, table, idx, out, status=None):
    dt = _DT[table.dtype]
    rc = _lib.load().eagle_gather_rows(n_rows, row_elems, dt, _ptr(table), table.shape[0], _ptr(idx), _ptr(out),
                                      _ptr(status), _stream())
    check("eagle_gather_rows", rc)


def gather_rows_multi(n_rows, idx, pairs, status=None):
    """One launch: out[r, :] = table[idx[r], :] for every (table, out) in `pairs` (at most 4)."""
    import ctypes
    n = len(pairs)
    dt = _DT[pairs[0][0].dtype]
    elems = (ctypes.c_int32 * n)(*[int(t.numel() // t.shape[0]) for t, _ in pairs])
    tabs = (ctypes.c_void_p * n)(*[_ptr(t) for t, _ in pairs])
    outs = (ctypes.c_void_p * n)(*[_ptr(o) for _, o in pairs])
    rc = _lib.load().eagle_gather_rows_multi(n, n_rows, dt, pairs[0][0].shape[0], _ptr(idx), ctypes.addressof(elems),
                                            ctypes.addressof(tabs), ctypes.addressof(outs), _ptr(status), _stream())
    check("eagle_gather_rows_multi", rc)


def commit_accepted(batch, n, hkv, head_dim, max_prefix, hidden, depth, accept_len, accept_path, k_tree, v_tree, x,
                    k_prefix, v_prefix, prefix_len, feat, status=None):
    """Append the accepted path's keys/values to the prefix cache (in place), grow prefix_len,
    and write the path's features to feat [B, depth + 1, hidden]."""
    dt = _DT[k_tree.dtype]
    rc = _lib.load().eagle_commit_accepted(batch, n, hkv, head_dim, max_prefix, hidden, depth, dt, _ptr(accept_len),
                                          _ptr(accept_path), _ptr(k_tree), _ptr(v_tree), _ptr(x), _ptr(k_prefix),
                                          _ptr(v_prefix), _ptr(prefix_len), _ptr(feat), _ptr(status), _stream())
    check("eagle_commit_accepted", rc)


def sampling_warp(rows, vocab, top_k, top_p, min_keep, temperature, logits, row_stats, bound, status=None):
    """Warp logits rows [rows, vocab]: row_stats (M, S) of the warped softmax and the kept prefix's bound."""
    rc = _lib.load().eagle_sampling_warp(rows, vocab, int(top_k), float(top_p), int(min_keep), float(temperature),
                                        _ptr(logits), _ptr(row_stats), _ptr(bound), _ptr(status), _stream())
    check("eagle_sampling_warp", rc)


def draft_dims(hidden, hq, hkv, head_dim, inter, max_prefix) -> DraftDims:
    return DraftDims(int(hidden), int(hq), int(hkv), int(head_dim), int(inter), int(max_prefix))


def draft_weights(embed, fc, qkv, o, gate_up, down, lm_head, lm_head_z=None) -> DraftWeights:
    """Device tensors: embed row-major [V, H]; the others packed (pack_lmhead_weight)."""
    return DraftWeights(*[_ptr(t) for t in (embed, fc, qkv, o, gate_up, down, lm_head, lm_head_z)])


def draft_workspace_size(p: TreeParams, dims: DraftDims) -> int:
    return int(_lib.load().eagle_draft_workspace_size(p, dims))


DRAFT_BUFFERS = ("slot_k", "slot_v", "slot_feat", "slot_mask", "idx", "x0", "u", "n1", "qkv", "q", "attn", "h", "n2",
                 "gu", "m", "y", "a")


def draft_workspace_layout(p: TreeParams, dims: DraftDims) -> dict:
    """Byte offsets of the drafting's intermediates in its workspace, by name."""
    n = len(DRAFT_BUFFERS)
    arr = (ctypes.c_size_t * n)()
    rc = _lib.load().eagle_draft_workspace_layout(p, dims, arr, n)
    if rc < 0:
        check("eagle_draft_workspace_layout", rc)
    return {DRAFT_BUFFERS[i]: int(arr[i]) for i in range(rc)}


def draft_forward(p: TreeParams, depth, dims: DraftDims, w: DraftWeights, root_token, root_feat, k_prefix, v_prefix,
                  prefix_len, pool_tok, slot_src, draft_logits, ws, status=None):
    """The draft head's forward for one depth: rows of that depth's slots in draft_logits [B, S, V]."""
    rc = _lib.load().eagle_draft_forward(p, int(depth), dims, w, _ptr(root_token), _ptr(root_feat), _ptr(k_prefix),
                                        _ptr(v_prefix), _ptr(prefix_len), _ptr(pool_tok), _ptr(slot_src),
                                        _ptr(draft_logits), _ptr(ws), ws.numel(), _ptr(status), _stream())
    check("eagle_draft_forward", rc)


def expand_depth(p: TreeParams, depth, draft_logits, tree, ws, status=None, warp=None, draft_bound=None):
    """Children of one depth's frontier slots (and the next frontier) into tree's pool arrays.
    warp = (top_k, top_p): the depth's rows are warped first, their bounds written
    to draft_bound [B, S, 2] uint32 at their slots (eagle_expand_depth_warped)."""
    if warp is not None:
        if draft_bound is None:
            raise ValueError("a warped expansion needs a draft_bound buffer")
        rc = _lib.load().eagle_expand_depth_warped(p, int(depth), int(warp[0]), float(warp[1]), _ptr(draft_logits),
                                                  _ptr(draft_bound), _ptr(tree["pool_tok"]), _ptr(tree["pool_q"]),
                                                  _ptr(tree["slot_src"]), _ptr(tree["slot_stats"]), _ptr(ws),
                                                  ws.numel(), _ptr(status), _stream())
        check("eagle_expand_depth_warped", rc)
        return
    rc = _lib.load().eagle_expand_depth(p, int(depth), _ptr(draft_logits), _ptr(tree["pool_tok"]),
                                       _ptr(tree["pool_q"]), _ptr(tree["slot_src"]), _ptr(tree["slot_stats"]),
                                       _ptr(ws), ws.numel(), _ptr(status), _stream())
    check("eagle_expand_depth", rc)


def expand_finish(p: TreeParams, root_token, tree, status=None):
    rc = _lib.load().eagle_expand_finish(
        p, _ptr(root_token), _ptr(tree["pool_tok"]), _ptr(tree["pool_q"]), _ptr(tree["node_tok"]),
        _ptr(tree["node_parent"]), _ptr(tree["node_depth"]), _ptr(tree["node_sib"]), _ptr(tree["node_slot"]),
        _ptr(tree["node_value"]), _ptr(tree["node_q"]), _ptr(tree["pool_flat"]), _ptr(tree["slot_src"]),
        _ptr(status), _stream())
    check("eagle_expand_finish", rc)
