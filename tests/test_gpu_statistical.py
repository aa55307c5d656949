"""Losslessness of the device walk, checked statistically and with no oracle:
with every request sharing one prefix, root token and draft rows, the first
committed token of every round must be distributed exactly as the target's
root distribution p (recursive speculative sampling commits tokens with the
target's distribution whatever the draft; EAGLE-1 notes, background A3 and
section 3.3).  For a near-uniform and a peaked target, 16384 independent walks (256 requests x 64 rounds, fresh
uniforms and Gumbel keys each round) on the tiny vocabulary of 256 tokens:
a chi-square test of the first-token histogram against p must not reject,
and the same histogram must reject the draft's own distribution q, which is
far from p (total variation about 0.7), so the test can tell the two apart."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
stats = pytest.importorskip("scipy.stats")


def _softmax64(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def _chisquare(counts, probs):
    """Chi-square p-value of counts against probabilities, the bins with an
    expected count below 5 pooled into one."""
    exp = probs * counts.sum()
    small = exp < 5.0
    c = np.append(counts[~small], counts[small].sum())
    e = np.append(exp[~small], exp[small].sum())
    if e[-1] == 0.0:
        c, e = c[:-1], e[:-1]
    return stats.chisquare(c, e).pvalue


# weight scale 1: near-uniform target rows (logit std ~0.05); 20: logit std ~1,
# a target distribution far from uniform
@pytest.mark.parametrize("wscale", [1.0, 20.0])
def test_first_committed_token_follows_target(wscale):
    from eagle_draft_tree_expand_amd import round as dround
    cfg = synth.get_config("tiny").with_(B=256)
    inp = synth.make_inputs(cfg)
    wts = dround.DeviceWeights(inp)
    wts.w.mul_(wscale)  # fp32 weights (tiny): no packed copy to redo
    data = dround.DeviceInputs(inp)
    rows = inp.iid_draft_rows()
    rows[:] = rows[0]  # every request drafts from request 0's rows
    data.set_rows(rows)
    for t in (data.k_prefix, data.v_prefix):
        t.copy_(t[0:1].expand_as(t).clone())
    data.prefix_len.fill_(int(inp.prefix_len[0]))
    data.roots.fill_(int(inp.roots[0]))
    dr = dround.DeviceRound(cfg)
    g = torch.Generator(device="cuda").manual_seed(20261202)
    counts = torch.zeros(cfg.V, dtype=torch.int64, device="cuda")
    rounds = 64
    for r in range(rounds):
        data.uniforms.copy_(torch.rand(data.uniforms.shape, generator=g, device="cuda"))
        dr.step(wts, data, 1.0, round_id=r)
        counts += torch.bincount(dr.acc["committed"][:, 0].long(), minlength=cfg.V)
        n = dr.acc["n_committed"]
        assert int(n.min()) >= 1 and int(n.max()) <= cfg.D + 1
    counts = counts.cpu().numpy()
    assert int(dr.status.item()) & 0x1 == 0
    # every request saw the same root row, so p is well defined
    z0 = dr.logits.view(cfg.B, cfg.N, cfg.V)[:, 0].cpu().numpy()
    assert (z0 == z0[0]).all()
    p = _softmax64(z0[0])
    q = _softmax64(rows[0, 0])
    total = int(counts.sum())
    assert total == cfg.B * rounds
    pv_p = _chisquare(counts, p)
    pv_q = _chisquare(counts, q)
    tv = 0.5 * np.abs(p - q).sum()
    print(f"scale {wscale}: {total} walks, 1/sum(p^2) = {1 / np.sum(p * p):.1f}; chi-square p-value against p "
          f"{pv_p:.3g}, against q {pv_q:.3g} (TV(p, q) = {tv:.3f})")
    assert tv > 0.5
    assert pv_p > 1e-4
    assert pv_q < 1e-12
