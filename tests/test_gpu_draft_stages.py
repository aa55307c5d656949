"""Staged parity of the draft head's kernels: each kernel checked on the values
the previous kernel wrote on the device (identical bf16 inputs on both sides).

After one eagle_draft_forward call the draft workspace holds every
intermediate of that depth (eagle_draft_workspace_layout gives their places).
From the device's own input to each step the oracle recomputes the step in
fp64 (the draft head of EAGLE-1 notes, section 3.1: FC over feature and
embedding, one decoder layer, the shared LM head):

* draft_in: x0 = [feature ; embedding of the token], bit for bit, and each
  slot's mask row = its parent's row plus itself;
* the fc, o and LM-head products: fp32 results against fp64 sums, 1e-5 of the
  row's largest value;
* draft_norm, draft_qkv, draft_silu and the last norm: bf16 outputs within one
  bf16 ulp of the fp64 value of the same formula (the device rounds an fp32
  value once), and equal to its bf16 rounding for at least 99% of entries;
* the draft attention: 2e-2 per row against the fp64 oracle on the slot mask.

At batch 64 the 640 frontier rows of depth 1 take the tiled GEMM, whose plain
products split the hidden dimension into uneven slices (fc: 5 slices of 12 or
13 chunks of 128; qkv: 3 of 10 or 11; down: 5 of 22 or 23); at batch 77 (770
rows) the qkv product takes 128-row tiles in 3 uneven slices with a ragged
last tile.  There 40 sampled rows (the first and the last included) and the
attention of 5 requests are checked.
"""
import numpy as np
import pytest

import synth
from oracle import attention as oattn
from synth.draft import make_draft_inputs

from gpu_helpers import rel_err_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bf16_close(dev, ref64, label, min_exact=0.99):
    """Within one bf16 ulp of the fp64 value, plus 1e-5 of the row's largest
    value for the fp32 accumulation of the device's products (entries near
    zero come from cancelling sums)."""
    dev = np.asarray(dev, np.float64)
    ref64 = np.asarray(ref64, np.float64)
    mag = np.abs(ref64)
    ulp = np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1e-30))) - 7)
    atol = 1e-5 * mag.max(axis=-1, keepdims=True)
    bad = np.abs(dev - ref64) > ulp + atol
    assert not bad.any(), f"{label}: {int(bad.sum())} entries beyond one bf16 ulp, e.g. {dev[bad][:4]} vs {ref64[bad][:4]}"
    exact = float(np.mean(dev == synth.bf16_round(ref64.astype(np.float32)).astype(np.float64)))
    assert exact >= min_exact, f"{label}: only {exact:.4f} equal to the bf16 rounding"
    return exact


def _rms(x):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)


class _Ws:
    """Typed views of the draft workspace."""

    def __init__(self, ws, lay):
        self.ws, self.lay = ws, lay

    def get(self, name, dtype, shape):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        off = self.lay[name]
        t = self.ws[off:off + n].view(dtype).view(*shape)
        return t.float().cpu().numpy() if dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("name,kw", [("mid_bf16", {}), ("8b", {}), ("b64", {}), ("b64", dict(B=77))])
def test_draft_kernels_staged(name, kw):
    from eagle_draft_tree_expand_amd import draft_head, ops
    from eagle_draft_tree_expand_amd import round as dround
    cfg = synth.get_config(name).with_(**kw)
    inp = synth.make_inputs(cfg)
    dinp = make_draft_inputs(cfg)
    wts = dround.DeviceWeights(inp)
    rnd = dround.DeviceRound(cfg)
    data = dround.DeviceInputs(inp)
    head = draft_head.DeviceDraftHead(cfg, dinp, wts)
    W = dinp.weights
    B, S, k, H, V = cfg.B, cfg.S, cfg.k, cfg.H, cfg.V
    Q, KV, I = cfg.hq * cfg.dh, cfg.hkv * cfg.dh, dinp.inter
    Wsl = (S + 63) // 64
    T = 1.0
    p = rnd.params(T, 0, data.seed)
    lay = ops.draft_workspace_layout(p, head.dims)
    ws = _Ws(head.ws, lay)
    bf = torch.bfloat16
    E = W["E"]
    Wlm = inp.w.astype(np.float64)
    rnd.status.zero_()
    for depth in (0, 1):
        print(f"[draft stages] {name} depth {depth}", flush=True)
        head.forward(p, depth, data.roots, data.prefix_len, rnd.tree, data.rows, rnd.status)
        torch.cuda.synchronize()
        kd = 1 if depth == 0 else k
        R = B * kd
        if R <= 64:
            samp = np.arange(R)
        else:
            pick = np.random.default_rng(3 + depth).choice(np.arange(1, R - 1), 38, replace=False)
            samp = np.unique(np.concatenate([[0, R - 1], pick]))
        idx = ws.get("idx", torch.int32, (R,))
        slots = idx - (np.arange(R) // kd) * S
        # draft_in: x0 = [feature ; E[token]] bit for bit
        x0 = ws.get("x0", bf, (R, 2 * H))
        slot_feat = ws.get("slot_feat", bf, (B, S, H))
        pool_tok = rnd.tree["pool_tok"].cpu().numpy().reshape(B, -1)
        slot_src = rnd.tree["slot_src"].cpu().numpy()
        masks = ws.get("slot_mask", torch.int64, (B, S, Wsl)).view(np.uint64)
        for r in samp:
            b, s = r // kd, int(slots[r])
            if depth == 0:
                tok, feat = int(inp.roots[b]), dinp.root_feat[b]
                par_mask = np.zeros(Wsl, np.uint64)
            else:
                e = int(slot_src[b, s])
                tok, feat = int(pool_tok[b, e]), slot_feat[b, e // k]
                par_mask = masks[b, e // k]
            assert np.array_equal(x0[r], np.concatenate([feat, E[tok]])), f"x0 row {r}"
            want = par_mask.copy()
            want[s // 64] |= np.uint64(1) << np.uint64(s % 64)
            assert np.array_equal(masks[b, s], want), f"mask of slot {s}"
        # fc product and the first norm
        u = ws.get("u", torch.float32, (R, H))
        assert rel_err_rows(u[samp], x0[samp].astype(np.float64) @ W["fc"].astype(np.float64).T) <= 1e-5
        n1 = ws.get("n1", bf, (R, H))
        _bf16_close(n1[samp], _rms(u[samp]), "n1 = rms(u)")
        # qkv product to bf16 q rows and slot k/v rows
        q = ws.get("q", bf, (R, Q))
        n1_64 = n1[samp].astype(np.float64)
        _bf16_close(q[samp], n1_64 @ W["q"].astype(np.float64).T, "q rows")
        sk = ws.get("slot_k", bf, (B * S, KV))
        sv = ws.get("slot_v", bf, (B * S, KV))
        _bf16_close(sk[idx[samp]], n1_64 @ W["k"].astype(np.float64).T, "k rows")
        _bf16_close(sv[idx[samp]], n1_64 @ W["v"].astype(np.float64).T, "v rows")
        # draft attention: frontier queries over the draft prefix and the slots their mask rows allow
        og = ws.get("attn", bf, (R, Q))
        scale = np.float32(1.0 / np.sqrt(cfg.dh))
        reqs = range(B) if R <= 64 else sorted(set((samp[:4] // kd).tolist()) | {B - 1})
        for b in reqs:
            qf = np.zeros((S, cfg.hq, cfg.dh), np.float32)
            rows_b = [r for r in range(R) if r // kd == b]
            for r in rows_b:
                qf[slots[r]] = q[r].reshape(cfg.hq, cfg.dh)
            mb = np.zeros((S, S), bool)
            for s in range(S):
                for j in range(S):
                    mb[s, j] = bool((int(masks[b, s, j // 64]) >> (j % 64)) & 1)
            L = min(int(inp.prefix_len[b]), head.cap)
            o64 = oattn.tree_attention(qf, dinp.k_prefix[b], dinp.v_prefix[b], L,
                                       sk[b * S:(b + 1) * S].reshape(S, cfg.hkv, cfg.dh),
                                       sv[b * S:(b + 1) * S].reshape(S, cfg.hkv, cfg.dh), mb, scale)
            got = np.stack([og[r] for r in rows_b]).reshape(-1, cfg.dh)
            ref = np.stack([o64[slots[r]] for r in rows_b]).reshape(-1, cfg.dh)
            assert rel_err_rows(got, ref) <= 2e-2, f"attention b={b}"
        # o product + residual, second norm
        h = ws.get("h", torch.float32, (R, H))
        assert rel_err_rows(h[samp], u[samp].astype(np.float64)
                            + og[samp].astype(np.float64) @ W["o"].astype(np.float64).T) <= 1e-5
        n2 = ws.get("n2", bf, (R, H))
        _bf16_close(n2[samp], _rms(h[samp]), "n2 = rms(h)")
        # gate/up product and silu
        n2_64 = n2[samp].astype(np.float64)
        g = n2_64 @ W["g"].astype(np.float64).T
        up = n2_64 @ W["u"].astype(np.float64).T
        m = ws.get("m", bf, (R, I))
        _bf16_close(m[samp], g / (1.0 + np.exp(-g)) * up, "m = silu(g) * u", min_exact=0.98)
        # down product + residual: the head output a, also the slot's feature
        a = ws.get("a", bf, (R, H))
        _bf16_close(a[samp], h[samp].astype(np.float64) + m[samp].astype(np.float64) @ W["d"].astype(np.float64).T,
                    "a")
        slot_feat = ws.get("slot_feat", bf, (B, S, H))
        for r in samp:
            assert np.array_equal(slot_feat[r // kd, slots[r]], a[r])
        # the shared LM head: the frontier's draft rows at their slots
        rows = data.rows
        zd = np.stack([rows[r // kd, int(slots[r])].cpu().numpy() for r in samp])
        assert rel_err_rows(zd, a[samp].astype(np.float64) @ Wlm.T) <= 1e-5
        assert int(rnd.status.item()) & ~0x8 == 0
        if depth == 0:
            ops.expand_depth(p, 0, data.rows, rnd.tree, rnd.ws, rnd.status)
