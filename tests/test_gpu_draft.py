"""Parity of depth-by-depth drafting with the synthetic EAGLE draft head
(eagle_draft_forward, eagle_expand_depth, eagle_expand_finish through the C
ABI) with oracle/draft.py.

* Per-depth expansion alone: draft rows written by the oracle's head are put
  in the row buffer and the three-call expansion runs without the head; tree,
  pool and statistics must equal the oracle's bit for bit (same rows, so the
  same decisions), as for eagle_expand_tree.
* Whole drafting: the device head computes the rows depth by depth.  Two bf16
  activation pipelines that differ only in accumulation order drift apart by
  bf16 rounding noise (about 6e-3 of a row's largest logit here), so the
  check is on the device's own tree: each drafted row must match the oracle's
  row for the same root path to the bf16 tolerance (2e-2 of the row's largest
  logit), and every decision the device took (children, frontiers, rerank cut,
  values) must be one the oracle's rows allow within the observed row error.
  Where the oracle's own decisions are clear of that error the trees must be
  identical.
* The 8B shape at batch 1: the root's row at sampled vocabulary columns, and
  the row of a depth-1 slot on the path the device drafted, against the oracle.
"""
import numpy as np
import pytest

import synth
from oracle import draft as odraft
from oracle import expand as oexpand
from synth.draft import make_draft_inputs

from gpu_helpers import compare_expand, tree_keys

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Decision gaps below these are not compared exactly: about twice the largest
# row error measured (1.3e-2 in logit units); a value at depth d carries d such
# errors (one per confidence on its path), so its margin is D times the key's.
KEY_MARGIN = 3e-2      # logit units


def value_margin(D):
    return KEY_MARGIN * D  # relative


class _Wts:
    """Only the packed LM head of the round's weights."""

    def __init__(self, inp, device="cuda"):
        from eagle_draft_tree_expand_amd import ops
        self.packed = True
        self.w_packed = ops.pack_lmhead_weight(torch.from_numpy(inp.w).to(device).to(torch.bfloat16).contiguous())


def _setup(cfg, set_idx=0):
    from eagle_draft_tree_expand_amd import draft_head, round as rt
    inp = synth.make_inputs(cfg, set_idx)
    dinp = make_draft_inputs(cfg, set_idx)
    rnd = rt.DeviceRound(cfg)
    data = rt.DeviceInputs(inp)
    head = draft_head.DeviceDraftHead(cfg, dinp, _Wts(inp))
    return inp, dinp, rnd, data, head


def _oracle_heads(cfg, inp, dinp):
    return [odraft.DraftHead(dinp.weights, cfg.hq, cfg.hkv, cfg.dh, inp.w, dinp.k_prefix[b], dinp.v_prefix[b],
                             inp.prefix_len[b], act="bf16") for b in range(cfg.B)]


def _margin(out, T, k, D, m, seed, req):
    """Smallest gap of the request's decisions: consecutive keys among each
    slot's k+1 best (logit units), consecutive values among each layer's k+1
    best and at the rerank cut (relative)."""
    S = 1 + (D - 1) * k
    gaps = []
    for s in range(S):
        z = out["rows"][s]
        key = oexpand.gumbel_keys(z, T, seed, s, req, 0) * T if T > 0 else z.astype(np.float64)
        top = np.sort(key)[::-1][: k + 1]
        gaps.append(float(np.min(top[:-1] - top[1:])) / KEY_MARGIN)
    val = out["pool_val"].reshape(-1).astype(np.float64)
    dep = out["pool_depth"].reshape(-1)
    for d in range(1, D):
        v = np.sort(val[dep == d])[::-1][: k + 1]
        if v.size > 1:
            gaps.append(float(np.min((v[:-1] - v[1:]) / v[:-1])) / value_margin(D))
    v = np.sort(val)[::-1]
    if m < v.size:
        gaps.append(float((v[m - 1] - v[m]) / v[m - 1]) / value_margin(D))
    return min(gaps)


def _host(rnd):
    out = {key: rnd.tree[key].cpu().numpy() for key in rnd.tree}
    out["status"] = int(rnd.status.item())
    return out


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_expand_depth_matches_oracle_on_given_rows(T):
    """The three-call expansion on rows computed by the oracle's head."""
    from eagle_draft_tree_expand_amd import ops
    cfg = synth.get_config("mid_bf16")
    inp, dinp, rnd, data, head = _setup(cfg)
    heads = _oracle_heads(cfg, inp, dinp)
    ora = [odraft.expand_with_head(heads[b], dinp.root_feat[b], int(inp.roots[b]), T, cfg.k, cfg.D, cfg.m,
                                   inp.gumbel_seed, b) for b in range(cfg.B)]
    data.set_rows(np.stack([o["rows"] for o in ora]))
    p = rnd.params(T, 0, data.seed)
    rnd.status.zero_()
    for d in range(cfg.D):
        ops.expand_depth(p, d, data.rows, rnd.tree, rnd.ws, rnd.status)
    ops.expand_finish(p, data.roots, rnd.tree, rnd.status)
    dev = _host(rnd)
    assert dev["status"] & ~0x8 == 0
    stacked = {key: np.stack([o[key] for o in ora]) for key in ora[0] if key != "ties"}
    stacked["ties"] = [o["ties"] for o in ora]
    flagged = compare_expand(dev, stacked, cfg.k, f"T={T}")
    assert flagged <= 1


@pytest.mark.parametrize("T,warp", [(1.0, (50, 0.9)), (0.7, (0, 0.8)), (1.0, (12, 1.0))])
def test_expand_depth_warped_matches_oracle_on_given_rows(T, warp):
    """The three-call expansion with a sampling warp per depth, on rows computed
    by the oracle's head: the tree equals the oracle's warped expansion, and
    the bounds it keeps for the expanded slots are eagle_sampling_warp's on
    the same rows (min_keep = k)."""
    from eagle_draft_tree_expand_amd import ops
    cfg = synth.get_config("mid_bf16")
    inp, dinp, rnd, data, head = _setup(cfg)
    heads = _oracle_heads(cfg, inp, dinp)
    ora = [odraft.expand_with_head(heads[b], dinp.root_feat[b], int(inp.roots[b]), T, cfg.k, cfg.D, cfg.m,
                                   inp.gumbel_seed, b, warp=warp) for b in range(cfg.B)]
    data.set_rows(np.stack([o["rows"] for o in ora]))
    bound = torch.zeros((cfg.B, cfg.S, 2), dtype=torch.int32, device="cuda")
    p = rnd.params(T, 0, data.seed)
    rnd.status.zero_()
    for d in range(cfg.D):
        ops.expand_depth(p, d, data.rows, rnd.tree, rnd.ws, rnd.status, warp=warp, draft_bound=bound)
    ops.expand_finish(p, data.roots, rnd.tree, rnd.status)
    dev = _host(rnd)
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    stacked = {key: np.stack([o[key] for o in ora]) for key in ora[0] if key != "ties"}
    stacked["ties"] = [o["ties"] for o in ora]
    flagged = compare_expand(dev, stacked, cfg.k, f"warp {warp} T={T}")
    assert flagged <= 1
    ref_bound = torch.zeros_like(bound)
    ref_stats = torch.zeros((cfg.B, cfg.S, 2), dtype=torch.float32, device="cuda")
    ops.sampling_warp(cfg.B * cfg.S, cfg.V, warp[0], warp[1], cfg.k, T, data.rows, ref_stats, ref_bound, rnd.status)
    assert torch.equal(bound, ref_bound)
    # the expansion's slot statistics are the warped softmax's
    np.testing.assert_array_equal(dev["slot_stats"].reshape(cfg.B, cfg.S, 2)[..., 0],
                                  ref_stats.cpu().numpy()[..., 0])


@pytest.mark.parametrize("T,warp", [(1.0, (50, 0.9)), (0.7, (20, 0.95))])
def test_drafting_warped_equals_one_shot_warped_expansion(T, warp):
    """Drafting with a warp per depth, then the one-shot warped expansion of the
    rows the head drafted (bounds from eagle_sampling_warp on all slot rows):
    the same tree bit for bit, and the same bounds at every slot."""
    from eagle_draft_tree_expand_amd import draft_head, ops
    cfg = synth.get_config("mid_bf16")
    inp, dinp, rnd, data, head = _setup(cfg)
    bound = torch.zeros((cfg.B, cfg.S, 2), dtype=torch.int32, device="cuda")
    rnd.status.zero_()
    draft_head.draft_tree(head, rnd, data, T, warp=warp, draft_bound=bound)
    drafted = _host(rnd)
    assert drafted["status"] & ~0x8 == 0, hex(drafted["status"])
    ref_bound = torch.zeros_like(bound)
    ref_stats = torch.zeros((cfg.B, cfg.S, 2), dtype=torch.float32, device="cuda")
    ops.sampling_warp(cfg.B * cfg.S, cfg.V, warp[0], warp[1], cfg.k, T, data.rows, ref_stats, ref_bound, rnd.status)
    assert torch.equal(bound, ref_bound)
    ops.expand_tree(rnd.params(T, 0, data.seed), data.rows, data.roots, rnd.tree, rnd.ws, rnd.status,
                    draft_bound=ref_bound)
    one = _host(rnd)
    for key in tree_keys() + ("pool_q", "node_value", "node_q", "slot_stats"):
        assert np.array_equal(drafted[key], one[key]), key


def _validate(dev, rows, head, f_root, root, T, k, D, m, seed, b):
    """Check a device tree against the oracle's rows on the device's own root
    paths: every drafted row matches the oracle's row for its path, and every
    decision the device took (children of each slot, each depth's frontier,
    the rerank cut, node values) is one the oracle's rows allow once they are
    moved by at most the observed row error.  Returns (max relative row error,
    max absolute row error)."""
    S = 1 + (D - 1) * k
    Tp = T if T > 0 else 1.0
    zo, dz, rel = [], [], []
    for s in range(S):
        z = head.row(f_root, _slot_path(dev, s, root, k)).astype(np.float64)
        zo.append(z)
        dz.append(float(np.max(np.abs(rows[s] - z))))
        rel.append(dz[-1] / float(np.max(np.abs(z))))
        assert rel[-1] <= 2e-2, f"b={b} slot {s}: row error {rel[-1]:.2e}"
    err = max(dz) / Tp
    q = np.zeros((S, k))
    for s in range(S):
        z = zo[s]
        key = oexpand.gumbel_keys(z.astype(np.float32), T, seed, s, b, 0) if T > 0 else z
        ch = dev["pool_tok"][s]
        kth = np.sort(key)[::-1][k - 1]
        tol = 2 * err + 1e-9
        assert np.all(key[ch] >= kth - tol), f"b={b} slot {s}: a child outside the top {k}"
        assert np.all(np.diff(key[ch]) <= tol), f"b={b} slot {s}: children out of order"
        t = z / Tp
        q[s] = np.exp(t[ch] - t.max()) / np.exp(t - t.max()).sum()
    # values of every pool entry with the oracle's confidences along the device's tree
    val = np.zeros((S, k))
    for s in range(S):
        e = int(dev["slot_src"][s]) if s > 0 else -1
        val[s] = (val.flat[e] if e >= 0 else 1.0) * q[s]
    vtol = 4 * D * err + 1e-6
    for d in range(1, D):
        slots = [0] if d == 1 else list(range(1 + (d - 2) * k, 1 + (d - 1) * k))
        layer = [s * k + j for s in slots for j in range(k)]
        pick = [int(dev["slot_src"][1 + (d - 1) * k + i]) for i in range(k)]
        assert set(pick) <= set(layer)
        rest = [e for e in layer if e not in pick]
        if rest:
            assert min(val.flat[e] for e in pick) >= max(val.flat[e] for e in rest) * (1 - vtol), f"b={b} depth {d}"
        pv = np.array([val.flat[e] for e in pick])
        assert np.all(pv[1:] <= pv[:-1] * (1 + vtol)), f"b={b} depth {d}: frontier out of order"
    sel = dev["pool_flat"].reshape(-1) >= 0
    assert sel.sum() == m
    if (~sel).any():
        assert val.reshape(-1)[sel].min() >= val.reshape(-1)[~sel].max() * (1 - vtol), f"b={b}: rerank cut"
    for f in range(1, m + 1):
        e = int(np.flatnonzero(dev["pool_flat"].reshape(-1) == f)[0])
        np.testing.assert_allclose(dev["node_value"][f], val.flat[e], rtol=vtol)
    return max(rel), max(dz)


# The small tree (depth 2, k 2, m = P = 6: no rerank cut) has few decisions,
# so most of its trees are clear of the row error and are compared bit for bit;
# the test asserts that some are.  On the larger tree nearly every request has
# a decision inside the margin (values differ by the rows' small spread), so
# there the count is reported only.
@pytest.mark.parametrize("kw,T,min_compared", [({}, 1.0, 0), ({}, 0.0, 0),
                                               (dict(D=2, k=2, m=6), 1.0, 1), (dict(D=2, k=2, m=6), 0.0, 1)])
def test_drafting_matches_oracle(kw, T, min_compared):
    """Device drafting: rows and decisions validated on the device's paths; the
    trees compared bit for bit where the oracle's own decisions are clear of
    the row error."""
    from eagle_draft_tree_expand_amd import draft_head
    cfg = synth.get_config("mid_bf16").with_(**kw)
    compared = total = 0
    worst = worst_abs = 0.0
    for set_idx in range(3):
        inp, dinp, rnd, data, head = _setup(cfg, set_idx)
        rnd.status.zero_()
        draft_head.draft_tree(head, rnd, data, T)
        dev = _host(rnd)
        rows = data.rows.cpu().numpy()
        assert dev["status"] & ~0x8 == 0, hex(dev["status"])
        heads = _oracle_heads(cfg, inp, dinp)
        for b in range(cfg.B):
            total += 1
            root = int(inp.roots[b])
            db = {key: dev[key][b] for key in dev if key != "status"}
            r, a = _validate(db, rows[b], heads[b], dinp.root_feat[b], root, T, cfg.k, cfg.D, cfg.m,
                             inp.gumbel_seed, b)
            worst, worst_abs = max(worst, r), max(worst_abs, a)
            o = odraft.expand_with_head(heads[b], dinp.root_feat[b], root, T, cfg.k, cfg.D, cfg.m,
                                        inp.gumbel_seed, b)
            if _margin(o, T, cfg.k, cfg.D, cfg.m, inp.gumbel_seed, b) < 1.0:
                continue
            compared += 1
            for key in tree_keys():
                assert np.array_equal(dev[key][b], o[key]), f"set {set_idx} b={b} {key}: {dev[key][b]} vs {o[key]}"
    print(f"{kw} T={T}: {compared}/{total} trees compared exactly, worst row error {worst:.2e} "
          f"(abs {worst_abs:.2e})")
    assert compared >= min_compared


def _slot_path(out, s, root, k):
    if s == 0:
        return [root]
    toks, e = [], int(out["slot_src"][s])
    while e >= 0:
        toks.append(int(out["pool_tok"][e // k][e % k]))
        e = int(out["slot_src"][e // k]) if e // k > 0 else -1
    return [root] + toks[::-1]


def test_drafting_is_deterministic_and_resets():
    """Two rounds on one workspace give identical trees and rows (depth 0 resets the slot state)."""
    from eagle_draft_tree_expand_amd import draft_head
    cfg = synth.get_config("mid_bf16")
    inp, dinp, rnd, data, head = _setup(cfg, 1)
    outs = []
    for _ in range(2):
        rnd.status.zero_()
        draft_head.draft_tree(head, rnd, data, 1.0)
        outs.append((_host(rnd), data.rows.cpu().numpy().copy()))
    for key in tree_keys():
        assert np.array_equal(outs[0][0][key], outs[1][0][key])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_drafting_8b_shape_sampled():
    from eagle_draft_tree_expand_amd import draft_head
    cfg = synth.get_config("8b")
    inp, dinp, rnd, data, head = _setup(cfg)
    T = 1.0
    rnd.status.zero_()
    draft_head.draft_tree(head, rnd, data, T)
    dev = _host(rnd)
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    par, val = dev["node_parent"][0], dev["node_value"][0]
    for i in range(1, cfg.N):
        assert 0 <= par[i] < i and val[i] <= val[par[i]]
    rng = np.random.default_rng(0)
    cols = np.sort(rng.choice(cfg.V, 1024, replace=False))
    h = odraft.DraftHead(dinp.weights, cfg.hq, cfg.hkv, cfg.dh, inp.w, dinp.k_prefix[0], dinp.v_prefix[0],
                         inp.prefix_len[0], act="bf16")
    root = int(inp.roots[0])
    for s in (0, 1, cfg.k):
        path = _slot_path({key: dev[key][0] for key in ("slot_src", "pool_tok")}, s, root, cfg.k)
        zo = h.row(dinp.root_feat[0], path, cols).astype(np.float64)
        zd = data.rows[0, s].cpu().numpy()[cols]
        err = float(np.max(np.abs(zd - zo)) / np.max(np.abs(zo)))
        print(f"8b slot {s} path {path}: row error {err:.2e}")
        assert err <= 2e-2


def test_drafting_tiled_gemm_path():
    """Enough requests that every product of the head (B * k >= 193 rows) takes the
    tiled GEMM kernel with its output row map; a sample of requests is validated."""
    from eagle_draft_tree_expand_amd import draft_head
    cfg = synth.get_config("mid_bf16").with_(B=66, L=(40, 200))
    T = 1.0
    inp, dinp, rnd, data, head = _setup(cfg)
    rnd.status.zero_()
    draft_head.draft_tree(head, rnd, data, T)
    dev = _host(rnd)
    rows = data.rows.cpu().numpy()
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    heads = _oracle_heads(cfg, inp, dinp)
    worst = 0.0
    for b in (0, 1, 31, 64, 65):
        db = {key: dev[key][b] for key in dev if key != "status"}
        r, _ = _validate(db, rows[b], heads[b], dinp.root_feat[b], int(inp.roots[b]), T, cfg.k, cfg.D, cfg.m,
                         inp.gumbel_seed, b)
        worst = max(worst, r)
    print(f"B=66: worst row error {worst:.2e}")


@pytest.mark.parametrize("kw,T,zero_prefix", [
    (dict(D=1, k=3, m=3), 1.0, False),           # the root's children only
    (dict(D=5, k=1, m=5), 0.0, False),           # a chain, greedy
    (dict(D=6, k=16, m=100), 1.0, False),        # S = 81 slots: two mask words per slot
    (dict(D=3, k=2, m=5), 0.7, True),            # one request with an empty draft prefix
])
def test_drafting_edge_shapes(kw, T, zero_prefix):
    from eagle_draft_tree_expand_amd import draft_head
    from eagle_draft_tree_expand_amd import round as rt
    cfg = synth.get_config("mid_bf16").with_(**kw)
    inp = synth.make_inputs(cfg, 2)
    if zero_prefix:
        pl = np.array(inp.prefix_len, copy=True)
        pl[1] = 0
        inp.prefix_len = pl
    dinp = make_draft_inputs(cfg, 2)
    rnd = rt.DeviceRound(cfg)
    data = rt.DeviceInputs(inp)
    head = draft_head.DeviceDraftHead(cfg, dinp, _Wts(inp))
    rnd.status.zero_()
    draft_head.draft_tree(head, rnd, data, T)
    dev = _host(rnd)
    rows = data.rows.cpu().numpy()
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    heads = _oracle_heads(cfg, inp, dinp)
    for b in range(cfg.B):
        db = {key: dev[key][b] for key in dev if key != "status"}
        _validate(db, rows[b], heads[b], dinp.root_feat[b], int(inp.roots[b]), T, cfg.k, cfg.D, cfg.m,
                  inp.gumbel_seed, b)
