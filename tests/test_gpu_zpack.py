"""The z-packed LM-head weight (EAGLE_W_ZPACKED) against the packed one.

The z-packed form stores each bf16 weight's high byte as a 4-bit code where
its fragment allows it and keeps the rest raw; decoding restores every bit.
The streaming kernel that reads it accumulates in the same order as the packed
kernel (the same MFMA sequence per 16x16 output tile over the hidden
dimension, in chunk order), so logits, statistics and argmax must be equal bit
for bit, and the compact rows too.  Cases: the 8B head (61 rows, one 64-row
tile), a ragged vocabulary whose last 64-row group is half padding (mixed
zero rows force raw fragments), the 13B and 70B heads (vocabulary 32000: the
hidden split and the combine launch), several row tiles, and a weight with
planted extremes (zeros, subnormals, very large values, infinities) so that
both forms meet in one launch.  Also: the number of raw fragments on
N(0, 0.02) weights is a few percent, and row counts above the streaming
kernel's range are refused.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _heads(rows, H, V, T, w, x, compact=False):
    from eagle_draft_tree_expand_amd import ops
    dev = "cuda"
    wd = w.to(dev)
    xd = x.to(dev)
    wp = ops.pack_lmhead_weight(wd)
    wz, nraw = ops.zpack_lmhead_weight(wd)
    ws = ops.new_workspace(256 << 20, dev)  # stage area: tile records and hidden-split partials
    out = []
    for w_, layout in ((wp, True), (wz, "z")):
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        stats = torch.full((rows, 2), -1.0, device=dev)
        am = torch.full((rows,), -1, dtype=torch.int32, device=dev)
        if compact:
            z16 = torch.zeros((rows, V), dtype=torch.float16, device=dev)
            bm = torch.zeros((rows, (V + 127) // 128), device=dev)
            ops.lmhead_softmax_compact(rows, H, V, xd, w_, T, z16, bm, stats, am, ws, status=status, packed=layout)
            res = (z16, bm, stats, am)
        else:
            lg = torch.full((rows, V), -7.0, device=dev)
            ops.lmhead_softmax(rows, H, V, xd, w_, T, lg, stats, am, ws, status=status, packed=layout)
            res = (lg, stats, am)
        torch.cuda.synchronize()
        out.append(([r.cpu() for r in res], int(status.item())))
    return out, nraw, wz.numel(), wp.numel() * 2


def _same(a, b):
    """bitwise equality of two CPU tensors (NaN payloads included)."""
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    if a.dtype == torch.float16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("rows,H,V,T,compact", [
    (61, 4096, 128256, 1.0, False),   # the 8B head
    (61, 4096, 128256, 0.0, False),
    (61, 4096, 128256, 1.0, True),    # compact rows
    (7, 256, 1000, 0.7, False),       # ragged vocabulary: the last group is 40 rows + 24 padding rows
    (50, 5120, 32000, 1.0, False),    # 13B: hidden split + combine
    (48, 8192, 32000, 1.0, True),     # 70B, compact: hidden split + compact combine
    (130, 1024, 5003, 1.0, False),    # three row tiles, ragged vocabulary
])
def test_zpacked_head_equals_packed(rows, H, V, T, compact):
    rng = np.random.default_rng(rows * 7 + V)
    w = _bf16(0.02 * rng.standard_normal((V, H)))
    x = _bf16(rng.standard_normal((rows, H)))
    res, nraw, zbytes, pbytes = _heads(rows, H, V, T, w, x, compact)
    (a, sa), (b, sb) = res
    print(f"rows {rows} H {H} V {V} T {T} compact {compact}: raw fragments {nraw}, z-packed {zbytes} B, packed {pbytes} B")
    assert sa == sb
    for i, (p, q) in enumerate(zip(a, b)):
        assert _same(p, q), f"output {i} differs"
    nfrag = (V + 63) // 64 * (H // 8)
    assert nraw <= 0.2 * nfrag


def test_zpacked_planted_extremes():
    rows, H, V = 20, 512, 2048
    rng = np.random.default_rng(5)
    w = 0.02 * rng.standard_normal((V, H)).astype(np.float32)
    flat = w.reshape(-1)
    idx = rng.choice(flat.size, 400, replace=False)
    flat[idx[:100]] = 0.0
    flat[idx[100:150]] = -0.0
    flat[idx[150:200]] = 1e-39       # subnormal in fp32 and bf16
    flat[idx[200:250]] = 3e4
    flat[idx[250:300]] = -1e-30
    flat[idx[300:302]] = np.inf      # logits of the rows hitting it become non-finite
    wt = _bf16(w)
    x = _bf16(0.1 * rng.standard_normal((rows, H)))
    res, nraw, _, _ = _heads(rows, H, V, 1.0, wt, x)
    (a, sa), (b, sb) = res
    assert nraw > 0
    assert sa == sb
    for p, q in zip(a, b):
        assert _same(p, q)


def test_zpacked_rejects_gemm_rows():
    from eagle_draft_tree_expand_amd import ops
    from eagle_draft_tree_expand_amd._lib import EagleError
    rows, H, V = 193, 256, 1000
    w = torch.zeros((V, H), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((rows, H), dtype=torch.bfloat16, device="cuda")
    wz, _ = ops.zpack_lmhead_weight(w)
    ws = ops.new_workspace(64 << 20, "cuda")
    lg = torch.zeros((rows, V), device="cuda")
    stats = torch.zeros((rows, 2), device="cuda")
    am = torch.zeros((rows,), dtype=torch.int32, device="cuda")
    with pytest.raises(EagleError):
        ops.lmhead_softmax(rows, H, V, x, wz, 1.0, lg, stats, am, ws, packed="z")
