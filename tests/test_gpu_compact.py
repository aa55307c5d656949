"""Parity of compact target rows (eagle_lmhead_softmax_compact,
eagle_verify_accept_compact) with oracle/compact.py and the oracle's walk.

* The compact LM head computes the same fp32 logits as the fp32 mode (same
  kernels, same accumulation order), so its fp16 offsets and block maxima
  must equal the oracle's encoding of the fp32 mode's logits bit for bit; its
  argmax equals the fp32 mode's; its statistics are those of the decoded row.
* The decoded probabilities are within the 2e-2 bf16 bar of the fp64 oracle's
  (tokens at >= 1e-6 of the row's largest probability).
* The walk on compact rows takes the same paths as the oracle's walk fed the
  decoded rows (stage by stage), for dynamic and static trees.
* A whole round in compact mode at the 8B shape, stage by stage.
"""
import numpy as np
import pytest

import synth
from oracle import compact as ocmp
from oracle import expand as oexpand
from oracle import lmhead as olm
from oracle import static_tree as ost

from gpu_helpers import compare_accept, compare_expand, oracle_accept, rel_err_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _both_heads(cfg, inp, X, T, B=None):
    from eagle_draft_tree_expand_amd import round as dround
    wts = dround.DeviceWeights(inp)
    full = dround.DeviceRound(cfg, B=B)
    cmp = dround.DeviceRound(cfg, B=B, compact=True)
    for dr in (full, cmp):
        dr.x.copy_(torch.from_numpy(X).to(dr.x.dtype).view(dr.x.shape))
        dr.lmhead(wts, T)
    torch.cuda.synchronize()
    return full, cmp


@pytest.mark.parametrize("name,kw,T", [
    ("mid_bf16", {}, 1.0),                     # V 5003: ragged last block
    ("mid_bf16", dict(B=40), 0.7),             # 600 rows: tiled GEMM
    ("13b", {}, 1.0),                          # V 32000: hidden split and the compact combine
    ("8b", {}, 1.0),                           # the 8B head, 61 rows
    ("8b", {}, 0.0),
])
def test_compact_lmhead_matches_encoding(name, kw, T):
    cfg = synth.get_config(name).with_(**kw)
    inp = synth.make_inputs(cfg)
    rng = np.random.default_rng(21)
    X = synth.bf16_round((0.05 * rng.standard_normal((cfg.B * cfg.N, cfg.H))).astype(np.float32))
    full, cmp = _both_heads(cfg, inp, X, T)
    lg = full.logits.cpu().numpy()
    d, m = ocmp.encode(lg)
    z16 = cmp.z16.cpu().numpy()
    bm = cmp.bmax.cpu().numpy()
    assert np.array_equal(bm, m)
    assert np.array_equal(z16.view(np.uint16), d.view(np.uint16))
    assert np.array_equal(cmp.argmax.cpu().numpy(), full.argmax.cpu().numpy())
    zt = ocmp.decode(z16, bm)
    st, _ = olm.row_stats(zt, T)
    dst = cmp.stats.cpu().numpy()
    np.testing.assert_array_equal(dst[:, 0], st[:, 0].astype(np.float32))
    np.testing.assert_allclose(dst[:, 1], st[:, 1], rtol=1e-5)
    # probabilities against the fp64 oracle logits
    z64 = olm.logits(X, inp.w)
    worst = 0.0
    for r in range(0, z64.shape[0], max(1, z64.shape[0] // 24)):
        p = oexpand.softmax(z64[r].astype(np.float32), T)
        pt = oexpand.softmax(zt[r], T)
        keep = p >= 1e-6 * p.max()
        worst = max(worst, float((np.abs(pt[keep] - p[keep]) / p[keep]).max()))
    print(f"{name}{kw} T={T}: compact rows bit-exact; worst probability error {worst:.2e}")
    assert worst <= 2e-2
    assert int(cmp.status.item()) == 0


@pytest.mark.parametrize("B", [64, 10])  # 3904 rows: 256-row tiles; 610 rows: 128-row tiles
def test_compact_lmhead_b64_sampled_rows(B):
    cfg = synth.get_config("8b")
    inp = synth.make_inputs(cfg)
    rng = np.random.default_rng(22)
    X = synth.bf16_round((0.05 * rng.standard_normal((B * cfg.N, cfg.H))).astype(np.float32))
    full, cmp = _both_heads(cfg, inp, X, 1.0, B=B)
    rows = np.unique(np.concatenate([[0, B * cfg.N - 1], rng.choice(B * cfg.N, 62, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    lg = full.logits[idx].cpu().numpy()
    d, m = ocmp.encode(lg)
    assert np.array_equal(cmp.bmax[idx].cpu().numpy(), m)
    assert np.array_equal(cmp.z16[idx].cpu().numpy().view(np.uint16), d.view(np.uint16))
    assert np.array_equal(cmp.argmax[idx].cpu().numpy(), full.argmax[idx].cpu().numpy())
    st, _ = olm.row_stats(ocmp.decode(d, m), 1.0)
    np.testing.assert_allclose(cmp.stats[idx].cpu().numpy()[:, 1], st[:, 1], rtol=1e-5)


def _walk_case(cfg, T, mode, static):
    from eagle_draft_tree_expand_amd import round as dround
    inp = synth.make_inputs(cfg)
    rows = inp.iid_draft_rows()
    rng = np.random.default_rng(41)
    if static:
        ex = ost.expand_static_batch(rows, cfg.static_parent, inp.roots, T, inp.gumbel_seed, 0)
    else:
        ex = oexpand.expand_batch(rows, inp.roots, T, cfg.k, cfg.D, cfg.m, inp.gumbel_seed, 0)
    N = cfg.N
    logits = rng.standard_normal((cfg.B * N, cfg.V)).astype(np.float32)
    if mode != "independent":
        for b in range(cfg.B):
            for u in range(N):
                s = ex["node_slot"][b, u]
                if s >= 0:
                    noise = 0.0 if mode == "equal" else 0.3 * rng.standard_normal(cfg.V)
                    logits[b * N + u] = (rows[b, s] + noise).astype(np.float32)
    d, m = ocmp.encode(logits)
    zt = ocmp.decode(d, m)
    st, am = olm.row_stats(zt, T)
    ora = oracle_accept(cfg, ex, zt, rows, T, inp.uniforms, am)
    dr = dround.DeviceRound(cfg, compact=True)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat"):
        dr.tree[key].copy_(torch.from_numpy(ex[key].astype(np.int32)))
    dr.tree["slot_stats"].copy_(torch.from_numpy(ex["slot_stats"].astype(np.float32)))
    dr.z16.copy_(torch.from_numpy(d))
    dr.bmax.copy_(torch.from_numpy(m))
    dr.stats.copy_(torch.from_numpy(st.astype(np.float32)))
    dr.argmax.copy_(torch.from_numpy(am.astype(np.int32)))
    dr.accept(data, T)
    return dr.host(), ora


@pytest.mark.parametrize("mode", ["independent", "equal", "close"])
@pytest.mark.parametrize("name,kw,T", [("mid_bf16", {}, 1.0), ("mid_bf16", dict(B=8), 0.7), ("mid_bf16", {}, 0.0),
                                       ("mid_bf16", dict(V=4096 * 2 + 4, B=6, m=6), 1.0),
                                       ("mid_static", dict(B=5), 1.0)])
def test_compact_walk_matches_oracle(name, kw, T, mode):
    cfg = synth.get_config(name).with_(**kw)
    dev, ora = _walk_case(cfg, T, mode, static=bool(cfg.static_parent))
    flagged = compare_accept(dev, ora, f"compact {name}{kw} T={T} {mode}")
    assert flagged <= max(1, cfg.B // 4)
    for b in range(cfg.B):
        assert 1 <= dev["n_committed"][b] == dev["accept_len"][b] + 1 <= cfg.D + 1
    assert dev["status"] & 0x1 == 0


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_compact_round_8b_stagewise(T):
    """The 8B round in compact mode on iid draft rows: tree, attention, compact LM head and walk."""
    from eagle_draft_tree_expand_amd import round as dround
    from oracle import round as oround
    cfg = synth.get_config("8b")
    inp = synth.make_inputs(cfg)
    rows = inp.iid_draft_rows()
    dr = dround.DeviceRound(cfg, compact=True)
    wts = dround.DeviceWeights(inp)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    dr.step(wts, data, T)
    dev = dr.host()
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    ex = oexpand.expand_batch(rows, inp.roots, T, cfg.k, cfg.D, cfg.m, inp.gumbel_seed, 0)
    assert compare_expand(dev, ex, cfg.k, f"compact 8b T={T}") == 0
    _, o64 = oround.attention_rows(inp, 0, dev["node_tok"][0], dev["node_parent"][0])
    assert rel_err_rows(dev["x"][0].reshape(-1, cfg.dh), o64.reshape(-1, cfg.dh)) <= 2e-2
    X = dev["x"].reshape(cfg.B * cfg.N, cfg.H)
    z64 = olm.logits(X, inp.w)
    d, m = ocmp.encode(z64.astype(np.float32))
    zt = ocmp.decode(dev["z16"], dev["bmax"])
    # the device's rows decode to within the rounding of its own fp32 logits
    assert rel_err_rows(zt, z64) <= 2e-3
    tree = {key: dev[key] for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat")}
    staged = oracle_accept(cfg, tree, zt, rows, T, inp.uniforms, dev["argmax"])
    assert compare_accept(dev, staged, f"compact 8b T={T} walk") == 0
