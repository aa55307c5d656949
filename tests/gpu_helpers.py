"""Shared helpers of the GPU parity tests (inputs, oracle runs, comparisons)."""
import numpy as np

import synth
from oracle import accept as oaccept
from oracle import expand as oexpand
from oracle import lmhead as olm


def rel_err_rows(a, b):
    """max over rows of max|a - b| / max|b| (row = last axis flattened per leading index)."""
    a = np.asarray(a, np.float64).reshape(a.shape[0], -1)
    b = np.asarray(b, np.float64).reshape(b.shape[0], -1)
    den = np.maximum(np.abs(b).max(axis=1), 1e-30)
    return float((np.abs(a - b).max(axis=1) / den).max())


def tree_keys():
    return ("node_tok", "node_parent", "node_depth", "node_sib", "node_slot", "pool_tok", "pool_flat", "slot_src")


def compare_expand(dev, ora, k, label=""):
    """Bit-exact structure unless the oracle flags a near tie; values/q to 2e-6."""
    B = ora["node_tok"].shape[0]
    flagged = 0
    for b in range(B):
        t = ora["ties"][b]
        if t["children"] or t["frontier"] or t["rerank"]:
            flagged += 1
            continue
        for key in tree_keys():
            assert np.array_equal(dev[key][b], ora[key][b]), f"{label} b={b} {key}: {dev[key][b]} vs {ora[key][b]}"
        np.testing.assert_allclose(dev["node_value"][b], ora["node_value"][b], rtol=2e-6, atol=0)
        np.testing.assert_allclose(dev["pool_q"][b], ora["pool_q"][b], rtol=2e-6, atol=0)
        np.testing.assert_allclose(dev["slot_stats"][b][:, 0], ora["slot_stats"][b][:, 0], rtol=0, atol=0)
        np.testing.assert_allclose(dev["slot_stats"][b][:, 1], ora["slot_stats"][b][:, 1], rtol=1e-6)
    return flagged


def oracle_accept_inputs(cfg, rows, T, seed, inp, rng_logits=None, logits=None):
    """Oracle tree for rows + target logits (given, else N(0, 1) rows) and their stats."""
    ex = oexpand.expand_batch(rows, inp.roots, T, cfg.k, cfg.D, cfg.m, seed, 0)
    if logits is None:
        logits = rng_logits.standard_normal((cfg.B * cfg.N, cfg.V)).astype(np.float32)
    st, am = olm.row_stats(logits, T)
    return ex, logits, st, am


def oracle_accept(cfg, ex, logits, rows, T, U, am):
    res = []
    for b in range(cfg.B):
        tree = {key: ex[key][b] for key in ("node_tok", "node_parent", "node_slot", "pool_tok", "pool_flat")}
        res.append(oaccept.accept_request(tree, logits[b * cfg.N:(b + 1) * cfg.N], rows[b], T, cfg.k, cfg.D,
                                          U[b], am[b * cfg.N:(b + 1) * cfg.N]))
    return res


def compare_accept(dev, ora, label=""):
    flagged = 0
    for b, o in enumerate(ora):
        if o["ties"]:
            flagged += 1
            continue
        assert dev["n_committed"][b] == o["n_committed"], f"{label} b={b} n {dev['n_committed'][b]} vs {o['n_committed']}"
        assert dev["accept_len"][b] == o["accept_len"], f"{label} b={b}"
        assert np.array_equal(dev["accept_path"][b], o["accept_path"]), f"{label} b={b}"
        assert np.array_equal(dev["committed"][b], o["committed"]), \
            f"{label} b={b} committed {dev['committed'][b]} vs {o['committed']}"
    return flagged


def small_cfg(name, **kw):
    return synth.get_config(name).with_(**kw)
