"""Stage-by-stage parity at the full workload shapes, in the launch
configuration the benchmark times (one DeviceRound.step through the C ABI).

For the 8B, 13B and 70B shapes (batch 1) the draft rows come from the oracle's
own pre-pass (target logits on each frontier node's root path plus noise), and
the device runs the whole round on them.  Every stage is then checked against
the oracle fed the device's inputs to that stage:

* expansion: the oracle's tree on the same rows, bit-exact (near ties flagged);
* mask and positions: the oracle's ancestor relation of the device's tree;
* tree attention: every (node, head) row of the device's tree against the
  fp64 oracle, max|a - b| / max|b| per row <= 2e-2 (bf16 output);
* LM head: every logit of every row (all V columns) against fp64 X W^T of the
  device's own X, relative 1e-5 per row; statistics and argmax;
* acceptance: the oracle's walk on the device's logits, bit-exact paths.

Batch 64 (8B shape, ragged prefixes 512..4096) runs the whole batch on the
device with the synthetic noise rows sigma_b * eps as draft rows (the target
pre-pass is not repeated for 64 requests) and checks six requests, including
the shortest and the longest prefix, through every stage the same way.
"""
import numpy as np
import pytest

import synth
from oracle import expand as oexpand
from oracle import lmhead as olm
from oracle import mask as omask
from oracle import round as oround

from gpu_helpers import compare_accept, compare_expand, oracle_accept, rel_err_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_CACHE = {}


def _shared(name):
    """Inputs, the oracle's fp64 weights and the device weights of a workload, made once."""
    if name not in _CACHE:
        from eagle_draft_tree_expand_amd import round as dround
        cfg = synth.get_config(name)
        inp = synth.make_inputs(cfg)
        _CACHE.clear()  # one workload's weights at a time
        _CACHE[name] = (cfg, inp, oround._Weights(inp), dround.DeviceWeights(inp))
    return _CACHE[name]


def _check_stages(dev, cfg, inp, owts, rows, T, reqs, label):
    """Every stage of the requests `reqs` of a device round against the oracle."""
    k, D, m, N = cfg.k, cfg.D, cfg.m, cfg.N
    # A: expansion on the same rows
    for b in reqs:
        ex = oexpand.expand_request(rows[b], inp.roots[b], T, k, D, m, inp.gumbel_seed, b, 0)
        one = {key: ex[key][None] for key in ex if key != "ties"}
        one["ties"] = [ex["ties"]]
        devb = {key: dev[key][b:b + 1] for key in dev if isinstance(dev[key], np.ndarray) and dev[key].ndim >= 1
                and dev[key].shape[0] == cfg.B}
        assert compare_expand(devb, one, k, f"{label} b={b}") == 0, f"{label} b={b}: near tie {ex['ties']}"
    # B: mask and positions of the device's tree
    for b in reqs:
        ref = omask.pack_bits(omask.ancestor_mask(dev["node_parent"][b]))
        assert np.array_equal(dev["mask"][b], ref), f"{label} b={b} mask"
        assert np.array_equal(dev["pos"][b], omask.positions(dev["node_depth"][b], inp.prefix_len[b]))
    # C: attention over the prefix and the device's tree, every (node, head) row
    worst = 0.0
    for b in reqs:
        _, o64 = oround.attention_rows(inp, b, dev["node_tok"][b], dev["node_parent"][b])
        got = dev["x"][b].reshape(N * cfg.hq, cfg.dh)
        err = rel_err_rows(got, o64.reshape(N * cfg.hq, cfg.dh))
        worst = max(worst, err)
        assert err <= 2e-2, f"{label} b={b}: attention error {err:.2e}"
    # D: LM head of the device's X, all columns
    rows_idx = np.concatenate([np.arange(b * N, (b + 1) * N) for b in reqs])
    X = dev["x"].reshape(cfg.B * N, cfg.H)[rows_idx]
    z64 = owts.logits(X)
    lg = dev["logits"][rows_idx]
    lm_err = rel_err_rows(lg, z64)
    assert lm_err <= 1e-5, f"{label}: LM-head error {lm_err:.2e}"
    st, am = olm.row_stats(lg, T)
    np.testing.assert_allclose(dev["stats"][rows_idx, 0], st[:, 0], rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(dev["stats"][rows_idx, 1], st[:, 1], rtol=1e-5)
    assert np.array_equal(dev["argmax"][rows_idx], am)
    srt = np.sort(z64, axis=1)
    clear = (srt[:, -1] - srt[:, -2]) > 1e-5 * np.abs(srt[:, -1]).clip(1e-3)
    assert np.array_equal(am[clear], np.argmax(z64, axis=1)[clear])
    # E: the oracle's walk on the device's tree and logits
    flagged = 0
    for b in reqs:
        tree = {key: dev[key][b:b + 1] for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat")}
        sub = cfg.with_(B=1)
        lb = dev["logits"][b * N:(b + 1) * N]
        ora = oracle_accept(sub, tree, lb, rows[b:b + 1], T, inp.uniforms[b:b + 1], dev["argmax"][b * N:(b + 1) * N])
        devb = {key: dev[key][b:b + 1] for key in ("n_committed", "accept_len", "accept_path", "committed")}
        flagged += compare_accept(devb, ora, f"{label} b={b}")
    print(f"{label}: attention worst {worst:.2e}, LM head {lm_err:.2e}, walk flagged {flagged}/{len(reqs)}")
    return flagged


@pytest.mark.parametrize("name,T", [("8b", 1.0), ("8b", 0.0), ("13b", 1.0), ("70b", 1.0), ("70b", 0.0)])
def test_full_round_stagewise(name, T):
    from eagle_draft_tree_expand_amd import round as dround
    cfg, inp, owts, wts = _shared(name)
    print(f"[fullshape] {name} T={T}: oracle pre-pass", flush=True)
    rows = oround.target_draft_rows(inp, T, owts)
    dr = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    dr.step(wts, data, T)
    dev = dr.host()
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    assert _check_stages(dev, cfg, inp, owts, rows, T, range(cfg.B), f"{name} T={T}") == 0
    for b in range(cfg.B):
        assert 1 <= dev["n_committed"][b] == dev["accept_len"][b] + 1 <= cfg.D + 1


def test_b64_round_stagewise():
    from eagle_draft_tree_expand_amd import round as dround
    cfg, inp, owts, wts = _shared("b64")
    T = 1.0
    rows = inp.iid_draft_rows()
    dr = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(inp)
    data.set_rows(rows)
    dr.step(wts, data, T)
    dev = dr.host()
    assert dev["status"] & ~0x8 == 0, hex(dev["status"])
    L = inp.prefix_len
    reqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 0, 17, 40, cfg.B - 1})
    print(f"[fullshape] b64 requests {reqs}, prefixes {[int(L[b]) for b in reqs]}", flush=True)
    flagged = _check_stages(dev, cfg, inp, owts, rows, T, reqs, "b64")
    assert flagged <= 1
    for b in range(cfg.B):
        assert 1 <= dev["n_committed"][b] == dev["accept_len"][b] + 1 <= cfg.D + 1
