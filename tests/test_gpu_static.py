"""Parity of the static (EAGLE-1) draft tree on the device with
oracle/static_tree.py: eagle_expand_static and eagle_verify_accept_static
through the C ABI.

* Expansion on identical rows: nodes, pool (including the -1 entries past each
  slot's child count), pool_flat, slot_src bit for bit; values, confidences
  and slot statistics as for the dynamic tree.
* Acceptance stage by stage: the oracle's walk on the device's tree and
  logits gives the same paths (per-slot candidate lists of k_s draws).
* A whole round at the reduced size and at the 8B shape, and host-side
  rejection of invalid shapes.
"""
import numpy as np
import pytest

import synth
from oracle import static_tree as ost
from oracle import lmhead as olm

from gpu_helpers import compare_accept, oracle_accept, rel_err_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KEYS = ("node_tok", "node_parent", "node_depth", "node_sib", "node_slot", "pool_tok", "pool_flat", "slot_src")


def _compare(dev, ora, label):
    flagged = 0
    for b in range(ora["node_tok"].shape[0]):
        if ora["ties"][b]:
            flagged += 1
            continue
        for key in KEYS:
            assert np.array_equal(dev[key][b], ora[key][b]), f"{label} b={b} {key}: {dev[key][b]} vs {ora[key][b]}"
        np.testing.assert_allclose(dev["node_value"][b], ora["node_value"][b], rtol=2e-6, atol=0)
        np.testing.assert_allclose(dev["pool_q"][b], ora["pool_q"][b], rtol=2e-6, atol=0)
        np.testing.assert_array_equal(dev["slot_stats"][b][:, 0], ora["slot_stats"][b][:, 0].astype(np.float32))
        np.testing.assert_allclose(dev["slot_stats"][b][:, 1], ora["slot_stats"][b][:, 1], rtol=1e-6)
    return flagged


@pytest.mark.parametrize("name,T", [("mid_static", 1.0), ("mid_static", 0.7), ("mid_static", 0.0),
                                    ("tiny_static", 1.0), ("8b_static", 1.0), ("8b_static", 0.0)])
def test_expand_static_matches_oracle(name, T):
    from eagle_draft_tree_expand_amd import round as dround
    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg)
    rows = inp.iid_draft_rows()
    dr = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    dr.expand(data, T, round_id=2)
    dev = dr.host()
    ora = ost.expand_static_batch(rows, cfg.static_parent, inp.roots, T, inp.gumbel_seed, 2)
    flagged = _compare(dev, ora, f"{name} T={T}")
    print(f"{name} T={T}: flagged {flagged}/{cfg.B}")
    assert flagged <= max(0, cfg.B // 4)
    assert dev["status"] & ~0x8 == 0


@pytest.mark.parametrize("mode", ["independent", "close"])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_accept_static_matches_oracle(T, mode):
    from eagle_draft_tree_expand_amd import round as dround
    cfg = synth.get_config("mid_static").with_(B=6)
    inp = synth.make_inputs(cfg)
    rows = inp.iid_draft_rows()
    rng = np.random.default_rng(31)
    ex = ost.expand_static_batch(rows, cfg.static_parent, inp.roots, T, inp.gumbel_seed, 0)
    N = cfg.N
    logits = rng.standard_normal((cfg.B * N, cfg.V)).astype(np.float32)
    if mode == "close":
        for b in range(cfg.B):
            for u in range(N):
                s = ex["node_slot"][b, u]
                if s >= 0:
                    logits[b * N + u] = (rows[b, s] + 0.3 * rng.standard_normal(cfg.V)).astype(np.float32)
    st, am = olm.row_stats(logits, T)
    ora = oracle_accept(cfg, ex, logits, rows, T, inp.uniforms, am)
    dr = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat"):
        dr.tree[key].copy_(torch.from_numpy(ex[key].astype(np.int32)))
    dr.tree["slot_stats"].copy_(torch.from_numpy(ex["slot_stats"].astype(np.float32)))
    dr.logits.copy_(torch.from_numpy(logits))
    dr.stats.copy_(torch.from_numpy(st.astype(np.float32)))
    dr.argmax.copy_(torch.from_numpy(am.astype(np.int32)))
    dr.accept(data, T)
    dev = dr.host()
    flagged = compare_accept(dev, ora, f"static T={T} {mode}")
    assert flagged <= 1
    for b in range(cfg.B):
        assert 1 <= dev["n_committed"][b] == dev["accept_len"][b] + 1 <= cfg.D + 1
    assert dev["status"] & 0x1 == 0


@pytest.mark.parametrize("name,T", [("mid_static", 1.0), ("mid_static", 0.0), ("8b_static", 1.0),
                                    ("8b_static", 0.0)])
def test_static_round_stagewise(name, T):
    """Whole static round on the oracle's pre-pass rows; each stage against the oracle fed the device's inputs."""
    from eagle_draft_tree_expand_amd import round as dround
    from oracle import round as oround
    cfg = synth.get_config(name)
    inp = synth.make_inputs(cfg)
    owts = oround._Weights(inp)
    print(f"[static] {name} T={T}: oracle pre-pass", flush=True)
    rows = ost.target_static_rows(inp, T, cfg.static_parent, owts)
    dr = dround.DeviceRound(cfg)
    wts = dround.DeviceWeights(inp)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    dr.step(wts, data, T)
    dev = dr.host()
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    ora = ost.expand_static_batch(rows, cfg.static_parent, inp.roots, T, inp.gumbel_seed, 0)
    assert _compare(dev, ora, f"{name} T={T}") == 0
    N = cfg.N
    worst = 0.0
    for b in range(cfg.B):
        _, o64 = oround.attention_rows(inp, b, dev["node_tok"][b], dev["node_parent"][b])
        err = rel_err_rows(dev["x"][b].reshape(N * cfg.hq, cfg.dh), o64.reshape(N * cfg.hq, cfg.dh))
        worst = max(worst, err)
        assert err <= (2e-2 if cfg.dtype == "bf16" else 1e-5)
    X = dev["x"].reshape(cfg.B * N, cfg.H)
    assert rel_err_rows(dev["logits"], owts.logits(X)) <= 1e-5
    tree = {key: dev[key] for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat")}
    staged = oracle_accept(cfg, tree, dev["logits"], rows, T, inp.uniforms, dev["argmax"])
    flagged = compare_accept(dev, staged, f"{name} T={T} walk")
    print(f"{name} T={T}: attention worst {worst:.2e}, walk flagged {flagged}/{cfg.B}, "
          f"committed {list(dev['n_committed'])}")
    assert flagged <= max(1, cfg.B // 4)


def test_static_shape_validation():
    from eagle_draft_tree_expand_amd import _lib, ops
    assert ops.static_tree_info(synth.get_config("8b_static").static_parent) == (14, 5, 4, [4, 3, 2, 1, 1, 2, 1, 1,
                                                                                          1, 2, 1, 1, 1, 1])
    for bad in ([0, 0], [-1, 1], [-1, 0, 2], [-1, -1], [-1] + [0] * 17):   # the last: 17 children > 16
        with pytest.raises(_lib.EagleError):
            ops.static_tree_info(bad)
    cfg = synth.get_config("mid_static")
    from eagle_draft_tree_expand_amd import round as dround
    dr = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(synth.make_inputs(cfg))
    p = ops.tree_params(cfg.B, cfg.V, cfg.D, cfg.k + 1, cfg.m, 1.0)   # topk not the shape's largest count
    with pytest.raises(_lib.EagleError):
        ops.expand_static(p, cfg.static_parent, data.rows, data.roots, dr.tree, dr.ws, dr.status)
