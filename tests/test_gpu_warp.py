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
    if kind == "band":  # one narrow band: the first key digit cannot separate the top tokens
        return (5.0 + 0.01 * rng.standard_normal((R, V))).astype(np.float32)
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


@pytest.mark.parametrize("kind", ["normal", "ties", "flat", "peaked", "band", "neginf"])
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


def _big_rows(kind, R, V, rng):
    """Rows for the one-pass top-k: the bound estimated from the first 16384
    tokens either holds (normal), lists too many tokens (ties, flat), too few
    (desc: the first tokens are the largest), or has the k-th token at the
    bound itself (ties)."""
    if kind == "desc":
        z = np.sort(rng.standard_normal((R, V)).astype(np.float32), axis=1)[:, ::-1]
        z[1] = z[1, ::-1]  # ascending: the largest tokens sit in the ragged last batch
        return np.ascontiguousarray(z)
    if kind == "sparse":  # 3% finite, the rest -inf
        z = rng.standard_normal((R, V)).astype(np.float32)
        z[rng.random((R, V)) < 0.97] = -np.inf
        return z
    if kind == "flat":
        return (1.0 + 1e-7 * rng.integers(0, 3, (R, V))).astype(np.float32)
    return _rows(kind, R, V, rng)


@pytest.mark.parametrize("kind", ["normal", "ties", "desc", "sparse", "flat", "peaked"])
@pytest.mark.parametrize("V", [40000, 40001])
def test_warp_multi_batch_rows(kind, V):
    """Rows of three 16384-token batches (vector loads at V = 40000, scalar at
    40001): the top-k cut agrees with the oracle whichever path decides it."""
    rng = np.random.default_rng(hash((kind, V, "big")) % 2**32)
    z = _big_rows(kind, 4, V, rng)
    compared = total = 0
    for T in (1.0, 0.7):
        for top_k, top_p, min_keep in [(50, 0.9, 10), (200, 1.0, 1), (1000, 0.95, 1), (1, 1.0, 1)]:
            st, bd, status = _run(z, top_k, top_p, min_keep, T)
            codes = _codes(oexpand.scaled_logits(z, T))
            for r in range(z.shape[0]):
                w = owarp.warp_support(z[r], T, top_k, top_p, min_keep)
                total += 1
                if w["tie"]:
                    continue
                mask = (codes[r] > bd[r, 0]) | ((codes[r] == bd[r, 0]) & (np.arange(V) <= bd[r, 1]))
                assert np.array_equal(mask, w["mask"]), (kind, V, T, top_k, top_p, min_keep, r)
                assert st[r, 0] == np.float32(w["M"])
                np.testing.assert_allclose(st[r, 1], w["S"], rtol=2e-7)
                compared += 1
            assert bool(status & 0x2) == bool(np.any(~np.isfinite(z)))
    assert compared >= 0.5 * total, (compared, total)


# ------------------------------------------------- warped expansion and walk
import synth  # noqa: E402
from gpu_helpers import compare_accept, compare_expand, small_cfg  # noqa: E402
from oracle import accept as oaccept  # noqa: E402


def _oracle_bounds(rows2d, T, top_k, top_p, min_keep):
    """[R, 2] uint32 bounds and [R, 2] (M, S) of the oracle's warp of each row, plus tie flags."""
    R = rows2d.shape[0]
    bd = np.zeros((R, 2), np.uint32)
    st = np.zeros((R, 2), np.float64)
    tie = np.zeros(R, bool)
    for r in range(R):
        w = owarp.warp_support(rows2d[r], T, top_k, top_p, min_keep)
        bd[r, 0] = _codes(np.array([w["t_b"]], np.float32))[0]
        bd[r, 1] = w["id_b"]
        st[r] = (w["M"], w["S"])
        tie[r] = w["tie"]
    return bd, st, tie


def _dev_int(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()


WARP_CASES = [("mid_bf16", {}, 1.0, (40, 1.0)), ("mid_bf16", {}, 0.7, (0, 0.9)), ("mid_bf16", dict(B=6), 1.0, (200, 0.5)),
              ("tiny", {}, 1.0, (8, 0.8)), ("mid_bf16", dict(k=16, D=3, m=40), 1.0, (16, 0.3))]


@pytest.mark.parametrize("name,kw,T,wp", WARP_CASES)
def test_warped_expand_matches_oracle(name, kw, T, wp):
    from eagle_draft_tree_expand_amd import round as dround
    cfg = small_cfg(name, **kw)
    inp = synth.make_inputs(cfg)
    rows = inp.iid_draft_rows()
    ora = oexpand.expand_batch(rows, inp.roots, T, cfg.k, cfg.D, cfg.m, inp.gumbel_seed, 0, wp)
    bd, _, _ = _oracle_bounds(rows.reshape(cfg.B * cfg.S, cfg.V), T, wp[0], wp[1], cfg.k)
    dr = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    from eagle_draft_tree_expand_amd import ops
    ops.expand_tree(dr.params(T, 0, data.seed), data.rows, data.roots, dr.tree, dr.ws, dr.status, draft_bound=_dev_int(bd))
    dev = dr.host()
    flagged = compare_expand(dev, ora, cfg.k, f"warped {name}{kw}")
    assert flagged <= max(1, cfg.B // 4)
    # children lie in the kept prefix; slot stats are the warped softmax's
    codes = _codes(oexpand.scaled_logits(rows.reshape(cfg.B * cfg.S, cfg.V), T))
    for b in range(cfg.B):
        for s in range(cfg.S):
            r = b * cfg.S + s
            if s == 0 or dev["slot_src"][b, s] >= 0:
                for x in dev["pool_tok"][b, s]:
                    assert codes[r, x] > bd[r, 0] or (codes[r, x] == bd[r, 0] and x <= bd[r, 1])
                np.testing.assert_allclose(dev["slot_stats"][b, s, 1], ora["slot_stats"][b, s, 1], rtol=1e-5)


@pytest.mark.parametrize("mode", ["independent", "close"])
@pytest.mark.parametrize("name,kw,T,wp", WARP_CASES[:4])
def test_warped_accept_matches_oracle(name, kw, T, wp, mode):
    from eagle_draft_tree_expand_amd import round as dround
    cfg = small_cfg(name, **kw)
    inp = synth.make_inputs(cfg)
    rows = inp.iid_draft_rows()
    rng = np.random.default_rng(7)
    ex = oexpand.expand_batch(rows, inp.roots, T, cfg.k, cfg.D, cfg.m, inp.gumbel_seed, 0, wp)
    logits = rng.standard_normal((cfg.B * cfg.N, cfg.V)).astype(np.float32)
    if mode == "close":
        for b in range(cfg.B):
            for u in range(cfg.N):
                s = ex["node_slot"][b, u]
                if s >= 0:
                    logits[b * cfg.N + u] = (rows[b, s] + 0.3 * rng.standard_normal(cfg.V)).astype(np.float32)
    tbd, tst, ttie = _oracle_bounds(logits, T, wp[0], wp[1], cfg.k)
    dbd, _, dtie = _oracle_bounds(rows.reshape(cfg.B * cfg.S, cfg.V), T, wp[0], wp[1], cfg.k)
    ora = []
    for b in range(cfg.B):
        tree = {key: ex[key][b] for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat")}
        o = oaccept.accept_request(tree, logits[b * cfg.N:(b + 1) * cfg.N], rows[b], T, cfg.k, cfg.D, inp.uniforms[b],
                                   warp=wp)
        o["ties"] += int(ttie[b * cfg.N:(b + 1) * cfg.N].any() or dtie[b * cfg.S:(b + 1) * cfg.S].any())
        ora.append(o)
    dr = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat"):
        dr.tree[key].copy_(torch.from_numpy(ex[key].astype(np.int32)))
    dr.tree["slot_stats"].copy_(torch.from_numpy(ex["slot_stats"].astype(np.float32)))
    dr.logits.copy_(torch.from_numpy(logits))
    dr.t_wstats.copy_(torch.from_numpy(tst.astype(np.float32)))
    from eagle_draft_tree_expand_amd import ops
    ops.verify_accept(dr.params(T, 0, data.seed), dr.tree, dr.logits, dr.t_wstats, dr.argmax, data.rows,
                      dr.tree["slot_stats"], data.uniforms, dr.acc, dr.ws, dr.status, target_bound=_dev_int(tbd),
                      draft_bound=_dev_int(dbd))
    dev = dr.host()
    flagged = compare_accept(dev, ora, f"warped {name}{kw} {mode}")
    assert flagged <= max(1, cfg.B // 4)
    assert dev["status"] & 0x1 == 0


@pytest.mark.parametrize("wp", [(30, 0.9), (0, 0.6)])
def test_warped_round_end_to_end(wp):
    """All device kernels chained (row warps, expansion, mask, attention, LM head, walk)
    against the oracle's warped round (fp32, so paths agree unless a near tie is flagged)."""
    from eagle_draft_tree_expand_amd import round as dround
    from oracle import round as oround
    cfg = synth.get_config("mid_f32")
    inp = synth.make_inputs(cfg)
    ora = oround.run_round(inp, 1.0, warp=wp)
    dr = dround.DeviceRound(cfg)
    wts = dround.DeviceWeights(inp)
    data = dround.DeviceInputs(inp)
    data.set_rows(ora["rows"])
    dr.step(wts, data, 1.0, warp=wp)
    dev = dr.host()
    assert compare_expand(dev, ora["expand"], cfg.k, f"warped e2e {wp}") == 0
    compare_accept(dev, ora["accept"], f"warped e2e {wp}")
    assert dev["status"] & ~0x8 == 0
