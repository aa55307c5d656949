"""Parity of eagle_commit_accepted (through the C ABI) with oracle/commit.py.

The commit is pure data movement, so caches, lengths and features must match
the oracle bit for bit (bf16 compared as raw 16-bit patterns), together with
the status bits of the degenerate requests (no room in the cache, an invalid
path).  Inputs are seeded random trees with random accepted root paths.
"""
import numpy as np
import pytest

import synth
from oracle import commit as ocommit
from oracle import round as oround

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CACHE_FULL, BAD_TREE = 0x80, 0x10


def _random_tree(rng, n, D):
    parent, depth = [-1], [0]
    for i in range(1, n):
        cands = [j for j in range(i) if depth[j] < D]
        p = int(rng.choice(cands))
        parent.append(p)
        depth.append(depth[p] + 1)
    return np.array(parent), np.array(depth)


def _root_path(parent, leaf):
    path = []
    while leaf != 0:
        path.append(leaf)
        leaf = parent[leaf]
    return path[::-1]


def _bits(t):
    """Host copy of a device tensor as exact bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


def _case(rng, B, n, D, hkv, dh, H, cap, special):
    """Per-request accept_len/path/prefix_len; `special` maps b -> kind of edge case."""
    acc_len = np.zeros(B, np.int32)
    acc_path = np.full((B, D), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        parent, _ = _random_tree(rng, n, D)
        path = _root_path(parent, int(rng.integers(0, n)))
        kind = special.get(b)
        if kind == "longest":
            leaf = int(np.argmax([len(_root_path(parent, u)) for u in range(n)]))
            path = _root_path(parent, leaf)
        elif kind == "none":
            path = []
        a = len(path)
        acc_len[b] = a
        acc_path[b, :a] = path
        plen[b] = int(rng.integers(0, cap - a))                  # room for a + 1 rows
        if kind == "exact_fit":
            plen[b] = cap - a - 1
        elif kind == "full":
            plen[b] = cap - a                                    # one row short
        elif kind == "bad_node":
            acc_len[b] = max(a, 1)
            acc_path[b, acc_len[b] - 1] = n                      # outside [1, n)
        elif kind == "root_in_path":
            acc_len[b] = max(a, 1)
            acc_path[b, 0] = 0
        elif kind == "too_long":
            acc_len[b] = D + 1
    return acc_len, acc_path, plen


def _run_oracle(kp, vp, plen, kt, vt, x, acc_len, acc_path, D):
    B = kp.shape[0]
    kp2, vp2 = kp.copy(), vp.copy()
    plen2 = plen.copy()
    feat = np.zeros((B, D + 1, x.shape[2]), x.dtype)
    flags = set()
    for b in range(B):
        kp2[b], vp2[b], plen2[b], feat[b], f = ocommit.commit(kp[b], vp[b], plen[b], kt[b], vt[b], x[b],
                                                              acc_len[b], acc_path[b], D)
        flags |= f
    return kp2, vp2, plen2, feat, flags


COMMIT_CASES = [
    # dtype, B, n, D, hkv, dh, H, cap, edge cases by request
    ("bf16", 6, 15, 4, 2, 128, 512, 64, {0: "longest", 1: "none", 2: "exact_fit", 3: "full", 4: "bad_node"}),
    ("f32", 5, 10, 3, 3, 32, 136, 20, {0: "root_in_path", 1: "too_long", 2: "longest", 3: "exact_fit"}),
    ("bf16", 4, 61, 8, 8, 64, 1024, 40, {0: "longest", 1: "none"}),
    ("bf16", 1, 2, 1, 1, 8, 8, 2, {0: "longest"}),                     # smallest: one child, cache of 2
    ("bf16", 3, 256, 16, 4, 128, 512, 300, {0: "longest", 1: "exact_fit"}),  # maximum nodes and depth
]


@pytest.mark.parametrize("dtype,B,n,D,hkv,dh,H,cap,special", COMMIT_CASES)
def test_commit_matches_oracle(dtype, B, n, D, hkv, dh, H, cap, special):
    from eagle_draft_tree_expand_amd import ops
    rng = np.random.default_rng(1000 + B * n + D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(B * 7 + n)
    kp = torch.randn(B, hkv, cap, dh, generator=g).to(tdt)
    vp = torch.randn(B, hkv, cap, dh, generator=g).to(tdt)
    kt = torch.randn(B, n, hkv, dh, generator=g).to(tdt)
    vt = torch.randn(B, n, hkv, dh, generator=g).to(tdt)
    x = torch.randn(B, n, H, generator=g).to(tdt)
    acc_len, acc_path, plen = _case(rng, B, n, D, hkv, dh, H, cap, special)
    h = {k: _bits(v) for k, v in dict(kp=kp, vp=vp, kt=kt, vt=vt, x=x).items()}
    want = _run_oracle(h["kp"], h["vp"], plen, h["kt"], h["vt"], h["x"], acc_len, acc_path, D)

    d = {k: v.cuda() for k, v in dict(kp=kp, vp=vp, kt=kt, vt=vt, x=x).items()}
    d_len = torch.from_numpy(acc_len).cuda()
    d_path = torch.from_numpy(acc_path).cuda()
    d_plen = torch.from_numpy(plen).cuda()
    feat = torch.full((B, D + 1, H), 7.0, dtype=tdt).cuda()      # stale contents must be overwritten
    status = torch.zeros(1, dtype=torch.int32).cuda()
    ops.commit_accepted(B, n, hkv, dh, cap, H, D, d_len, d_path, d["kt"], d["vt"], d["x"], d["kp"], d["vp"],
                        d_plen, feat, status)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_plen.cpu().numpy(), want[2])
    np.testing.assert_array_equal(_bits(d["kp"]), want[0])
    np.testing.assert_array_equal(_bits(d["vp"]), want[1])
    np.testing.assert_array_equal(_bits(feat), want[3])
    st = int(status.item())
    assert bool(st & CACHE_FULL) == ("cache_full" in want[4])
    assert bool(st & BAD_TREE) == ("bad_path" in want[4])
    assert st & ~(CACHE_FULL | BAD_TREE) == 0


def test_commit_twice_appends():
    """Two commits in a row: the second appends after the first (a two-round loop
    of the cache), then a smaller batch reuses the same buffers."""
    from eagle_draft_tree_expand_amd import ops
    rng = np.random.default_rng(55)
    B, n, D, hkv, dh, H, cap = 4, 20, 5, 2, 128, 256, 30
    g = torch.Generator().manual_seed(3)
    kp = torch.randn(B, hkv, cap, dh, generator=g).to(torch.bfloat16)
    vp = torch.randn(B, hkv, cap, dh, generator=g).to(torch.bfloat16)
    d_kp, d_vp = kp.cuda(), vp.cuda()
    h_kp, h_vp = _bits(kp), _bits(vp)
    plen = rng.integers(0, 10, size=B).astype(np.int32)
    d_plen = torch.from_numpy(plen).cuda()
    h_plen = plen.copy()
    status = torch.zeros(1, dtype=torch.int32).cuda()
    for step in range(3):
        Bs = B if step < 2 else 2          # the third call covers fewer requests
        kt = torch.randn(Bs, n, hkv, dh, generator=g).to(torch.bfloat16)
        vt = torch.randn(Bs, n, hkv, dh, generator=g).to(torch.bfloat16)
        x = torch.randn(Bs, n, H, generator=g).to(torch.bfloat16)
        acc_len, acc_path, _ = _case(rng, Bs, n, D, hkv, dh, H, cap, {})
        feat = torch.zeros(Bs, D + 1, H, dtype=torch.bfloat16).cuda()
        ops.commit_accepted(Bs, n, hkv, dh, cap, H, D, torch.from_numpy(acc_len).cuda(),
                            torch.from_numpy(acc_path).cuda(), kt.cuda(), vt.cuda(), x.cuda(), d_kp, d_vp,
                            d_plen, feat, status)
        w = _run_oracle(h_kp[:Bs], h_vp[:Bs], h_plen[:Bs], _bits(kt), _bits(vt), _bits(x), acc_len, acc_path, D)
        h_kp[:Bs], h_vp[:Bs], h_plen[:Bs] = w[0], w[1], w[2]
        torch.cuda.synchronize()
        np.testing.assert_array_equal(d_plen.cpu().numpy(), h_plen)
        np.testing.assert_array_equal(_bits(d_kp), h_kp)
        np.testing.assert_array_equal(_bits(d_vp), h_vp)
        np.testing.assert_array_equal(_bits(feat), w[3])
    assert int(status.item()) == 0


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_round_then_commit_end_to_end(T):
    """A device round followed by its commit, against the oracle's round and
    commit from the same inputs (fp32, so accepted paths agree unless a near tie
    is flagged); the grown cache then serves a second device round whose tree
    attention sees the committed rows."""
    from eagle_draft_tree_expand_amd import round as dround
    cfg = synth.get_config("mid_f32")
    inp = synth.make_inputs(cfg)
    room = cfg.D + 1
    ora = oround.run_round(inp, T)
    dr = dround.DeviceRound(cfg, cap=cfg.Lmax + room)
    wts = dround.DeviceWeights(inp)
    data = dround.DeviceInputs(inp, room=room)
    data.set_rows(ora["rows"])
    dr.step(wts, data, T)
    dr.commit(data)
    torch.cuda.synchronize()
    B, N = cfg.B, cfg.N
    kp0 = np.zeros((B, cfg.hkv, cfg.Lmax + room, cfg.dh), np.float32)
    vp0 = np.zeros_like(kp0)
    kp0[:, :, :cfg.Lmax] = inp.k_prefix
    vp0[:, :, :cfg.Lmax] = inp.v_prefix
    tok = ora["expand"]["node_tok"]
    kt = inp.k_tab[tok].reshape(B, N, cfg.hkv, cfg.dh)
    vt = inp.v_tab[tok].reshape(B, N, cfg.hkv, cfg.dh)
    acc_len = np.array([a["accept_len"] for a in ora["accept"]], np.int32)
    acc_path = np.stack([a["accept_path"] for a in ora["accept"]]).astype(np.int32)
    want = _run_oracle(kp0, vp0, inp.prefix_len, kt, vt, ora["x"].reshape(B, N, cfg.H), acc_len, acc_path, cfg.D)
    got_len = data.prefix_len.cpu().numpy()
    got_k, got_v, got_f = data.k_prefix.cpu().numpy(), data.v_prefix.cpu().numpy(), dr.feat.cpu().numpy()
    checked = 0
    for b, a in enumerate(ora["accept"]):
        if a["ties"]:
            continue
        checked += 1
        assert got_len[b] == want[2][b]
        np.testing.assert_array_equal(got_k[b], want[0][b])
        np.testing.assert_array_equal(got_v[b], want[1][b])
        ref = want[3][b]
        assert np.abs(got_f[b] - ref).max() <= 1e-5 * (1 + np.abs(ref).max())
    assert checked > 0
    assert int(dr.status.item()) & ~0x8 == 0
    # a second round on the grown cache: the device tree equals the oracle's
    # expansion for round 1, and the device attention over the committed
    # prefix equals the oracle's over the oracle's own committed cache
    from gpu_helpers import compare_expand
    from oracle import attention as oattn
    from oracle import expand as oexpand
    from oracle import mask as omask
    dr.step(wts, data, T, round_id=1)
    torch.cuda.synchronize()
    ex2 = oexpand.expand_batch(ora["rows"], inp.roots, T, cfg.k, cfg.D, cfg.m, inp.gumbel_seed, 1)
    dev2 = dr.host()
    compare_expand(dev2, ex2, cfg.k, "second round")
    x2 = dev2["x"].reshape(B, N, cfg.H)
    for b, a in enumerate(ora["accept"]):
        t2 = ex2["ties"][b]
        if a["ties"] or t2["children"] or t2["frontier"] or t2["rerank"]:
            continue
        tok2, par2 = ex2["node_tok"][b], ex2["node_parent"][b]
        o = oattn.tree_attention(inp.q_tab[tok2].reshape(N, cfg.hq, cfg.dh), want[0][b], want[1][b], want[2][b],
                                 inp.k_tab[tok2].reshape(N, cfg.hkv, cfg.dh),
                                 inp.v_tab[tok2].reshape(N, cfg.hkv, cfg.dh), omask.ancestor_mask(par2),
                                 np.float32(1.0 / np.sqrt(cfg.dh)))
        ref = o.reshape(N, cfg.H)
        assert np.abs(x2[b] - ref).max() <= 1e-5 * (1 + np.abs(ref).max())
