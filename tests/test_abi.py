"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host with the documented
codes before touching the device.

Every call below fails a host check (the fake pointers are never handed to a
kernel): a shape that is valid is shown valid by a later check failing, such as
a workspace that is too small or a null pointer, never by a call that could
reach a launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eagle.h")


@pytest.fixture(scope="module")
def lib():
    from eagle_draft_tree_expand_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from eagle_draft_tree_expand_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle_[a-z_]+)\s*\(", src)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("eagle_expand_tree", "eagle_build_tree_mask", "eagle_tree_attention", "eagle_lmhead_softmax",
              "eagle_verify_accept"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from eagle_draft_tree_expand_amd import _lib
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_error_strings(lib):
    assert lib.eagle_abi_version() >> 16 == 1
    assert lib.eagle_error_string(-4) == b"workspace too small"
    assert lib.eagle_error_string(0) == b"ok"


def _params(**kw):
    from eagle_draft_tree_expand_amd import ops
    d = dict(batch=1, vocab=1000, depth=3, topk=2, m=5, temperature=1.0)
    d.update(kw)
    return ops.tree_params(d["batch"], d["vocab"], d["depth"], d["topk"], d["m"], d["temperature"])


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(m=0), -2), (dict(m=11), -2), (dict(topk=17), -2), (dict(topk=0), -2), (dict(depth=0), -2),
    (dict(depth=17), -2), (dict(vocab=1), -2), (dict(temperature=-1.0), -2), (dict(batch=0), -2),
    (dict(temperature=float("nan")), -2),
])
def test_expand_rejects_bad_shapes(lib, kw, code):
    p = _params(**kw)
    args = [FAKE] * 16
    rc = lib.eagle_expand_tree(ctypes.byref(p), *args[:14], FAKE, 1 << 30, None, None)
    assert rc == code


def test_expand_null_align_workspace(lib):
    p = _params()
    ptrs = [FAKE] * 14
    assert lib.eagle_expand_tree(ctypes.byref(p), None, *ptrs[1:], FAKE, 1 << 30, None, None) == -1
    assert lib.eagle_expand_tree(ctypes.byref(p), FAKE + 4, *ptrs[1:], FAKE, 1 << 30, None, None) == -6
    assert lib.eagle_expand_tree(ctypes.byref(p), *ptrs, FAKE, 100, None, None) == -4
    assert lib.eagle_expand_tree(None, *ptrs, FAKE, 1 << 30, None, None) == -1


def test_workspace_size(lib):
    p = _params()
    n = lib.eagle_workspace_size(ctypes.byref(p), 4, 2, 128, 300, 512)
    assert n > 65536 and n % 256 == 0
    assert lib.eagle_workspace_size(ctypes.byref(_params(m=11)), 4, 2, 128, 300, 512) == 0
    assert lib.eagle_workspace_size(ctypes.byref(p), 4, 3, 128, 300, 512) == 0   # hq % hkv


def test_attention_rejects(lib):
    f = lib.eagle_tree_attention
    ok = (1, 5, 4, 2, 128, 100, 1)
    tail = [FAKE] * 7
    assert f(*ok, *tail, 0.1, FAKE, FAKE, 1000, None, None) == -4   # the shape passes; the workspace does not
    assert f(1, 5, 4, 3, 128, 100, 1, *tail, 0.1, FAKE, FAKE, 1 << 30, None, None) == -2
    assert f(1, 5, 4, 2, 96, 100, 1, *tail, 0.1, FAKE, FAKE, 1 << 30, None, None) == -3
    assert f(1, 5, 4, 2, 128, 100, 7, *tail, 0.1, FAKE, FAKE, 1 << 30, None, None) == -3
    assert f(1, 0, 4, 2, 128, 100, 1, *tail, 0.1, FAKE, FAKE, 1 << 30, None, None) == -2
    assert f(1, 257, 4, 2, 128, 100, 1, *tail, 0.1, FAKE, FAKE, 1 << 30, None, None) == -2
    assert f(*ok, None, *tail[1:], 0.1, FAKE, FAKE, 1 << 30, None, None) == -1
    assert f(*ok, FAKE + 2, *tail[1:], 0.1, FAKE, FAKE, 1 << 30, None, None) == -6
    assert f(*ok, *tail, float("inf"), FAKE, FAKE, 1 << 30, None, None) == -2
    assert f(*ok, *tail, 0.1, FAKE, FAKE, 1000, None, None) == -4


def test_lmhead_rejects(lib):
    f = lib.eagle_lmhead_softmax
    good = (FAKE, FAKE, 0, 1.0, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None, None)
    assert f(10, 100, 500, 1, *good) == -2                      # bf16 needs hidden % 128
    assert f(10, 128, 500, 2, *good) == -3                      # dtype
    assert f(0, 128, 500, 1, *good) == -2
    assert f(10, 128, 500, 1, None, *good[1:]) == -1
    assert f(10, 128, 500, 1, FAKE, FAKE, 0, -2.0, *good[4:]) == -2
    assert f(10, 128, 500, 1, FAKE, FAKE, 7, 1.0, *good[4:]) == -2    # layout
    assert f(10, 128, 500, 0, FAKE, FAKE, 1, 1.0, *good[4:]) == -3    # packed is bf16 only
    assert f(10, 128, 500, 1, *good[:-3], 10, None, None) == -4
    assert f(10, 20000, 500, 0, *good) == -2                    # fp32 row must fit LDS


def test_packed_weight_size_and_rejects(lib):
    assert lib.eagle_lmhead_packed_bytes(128256, 4096, 1) == ((128256 + 63) // 64) * 64 * 4096 * 2
    assert lib.eagle_lmhead_packed_bytes(100, 256, 1) == 128 * 256 * 2
    assert lib.eagle_lmhead_packed_bytes(100, 100, 1) == 0
    assert lib.eagle_lmhead_packed_bytes(100, 256, 0) == 0
    assert lib.eagle_lmhead_pack_weight(100, 256, 0, FAKE, FAKE, None) == -3
    assert lib.eagle_lmhead_pack_weight(100, 256, 1, None, FAKE, None) == -1
    assert lib.eagle_lmhead_pack_weight(100, 256, 1, FAKE, FAKE + 8, None) == -6


def test_zpacked_weight_size_and_rejects(lib):
    """The z-packed form (EAGLE_W_ZPACKED): its size, the pack call's host checks, and the LM head's
    refusal of the layout beyond the streaming kernel's rows or hidden size."""
    F = (128256 + 63) // 64 * (4096 // 8)            # fragments of the 8B head
    n = lib.eagle_lmhead_zpack_bytes(128256, 4096)
    slot = (F + 16 + 255) // 256 * 256
    raw = (slot + F * 768 + 16 + 255) // 256 * 256
    assert n == raw + F * 1024
    assert lib.eagle_lmhead_zpack_bytes(100, 100) == 0          # hidden % 128
    assert lib.eagle_lmhead_zpack_bytes(100, 16512) == 0        # hidden above 16384
    assert lib.eagle_lmhead_zpack_weight(100, 100, FAKE, FAKE, None, None) == -2
    assert lib.eagle_lmhead_zpack_weight(100, 256, None, FAKE, None, None) == -1
    assert lib.eagle_lmhead_zpack_weight(100, 256, FAKE, FAKE + 16, None, None) == -6   # w_z 256-aligned
    assert lib.eagle_lmhead_zpack_weight(100, 256, FAKE + 8, FAKE, None, None) == -6    # w 16-aligned
    assert lib.eagle_lmhead_zpack_weight(100, 256, FAKE, FAKE, FAKE + 2, None) == -6    # count word
    f = lib.eagle_lmhead_softmax
    tail = (1.0, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None, None)
    assert f(193, 128, 500, 1, FAKE, FAKE, 2, *tail) == -2      # z-packed: at most 192 rows
    assert f(10, 16512, 500, 1, FAKE, FAKE, 2, *tail) == -2     # ... and hidden <= 16384
    assert f(10, 128, 500, 0, FAKE, FAKE, 2, *tail) == -3       # ... bf16 only
    assert f(10, 128, 500, 1, FAKE, FAKE, 2, *tail[:-3], 10, None, None) == -4   # the shape passes
    g = lib.eagle_lmhead_softmax_compact
    ctail = (1.0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, None)
    assert g(193, 128, 500, FAKE, FAKE, 2, *ctail) == -2


def test_mask_gather_accept_reject(lib):
    assert lib.eagle_build_tree_mask(1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert lib.eagle_build_tree_mask(1, 300, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert lib.eagle_build_tree_mask(1, 5, None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.eagle_gather_rows(4, 8, 5, FAKE, 10, FAKE, FAKE, None, None) == -3
    assert lib.eagle_gather_rows(4, 0, 1, FAKE, 10, FAKE, FAKE, None, None) == -2
    assert lib.eagle_gather_rows(0, 8, 1, None, 10, None, None, None, None) == 0
    p = _params()
    args = [FAKE] * 16
    assert lib.eagle_verify_accept(ctypes.byref(_params(m=0)), *args, FAKE, 1 << 20, None, None) == -2
    args[0] = None
    assert lib.eagle_verify_accept(ctypes.byref(p), *args, FAKE, 1 << 20, None, None) == -1


def test_gather_multi_rejects(lib):
    elems = (ctypes.c_int32 * 3)(8, 4, 4)
    tabs = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    outs = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    a = [ctypes.addressof(elems), ctypes.addressof(tabs), ctypes.addressof(outs)]
    assert lib.eagle_gather_rows_multi(0, 4, 1, 10, FAKE, *a, None, None) == -2   # no table
    assert lib.eagle_gather_rows_multi(5, 4, 1, 10, FAKE, *a, None, None) == -2   # more than 4
    assert lib.eagle_gather_rows_multi(3, 4, 7, 10, FAKE, *a, None, None) == -3   # dtype
    assert lib.eagle_gather_rows_multi(3, 4, 1, 0, FAKE, *a, None, None) == -2    # empty table
    assert lib.eagle_gather_rows_multi(3, 4, 1, 10, None, *a, None, None) == -1   # no ids
    assert lib.eagle_gather_rows_multi(3, 4, 1, 10, FAKE, None, a[1], a[2], None, None) == -1
    outs[1] = None
    assert lib.eagle_gather_rows_multi(3, 4, 1, 10, FAKE, *a, None, None) == -1
    outs[1] = FAKE
    elems[2] = 0
    assert lib.eagle_gather_rows_multi(3, 4, 1, 10, FAKE, *a, None, None) == -2
    assert lib.eagle_gather_rows_multi(1, 0, 1, 10, None, *a, None, None) == 0    # nothing to do


def test_workspace_init_rejects(lib):
    assert lib.eagle_workspace_init(None, 1 << 20, None) == -1
    assert lib.eagle_workspace_init(FAKE, 100, None) == -4


def test_commit_rejects(lib):
    f = lib.eagle_commit_accepted
    ok = (2, 9, 2, 128, 100, 512, 4, 1)
    ptrs = [FAKE] * 9
    assert f(0, *ok[1:], *ptrs, None, None) == 0                          # empty batch
    assert f(2, 0, *ok[2:], *ptrs, None, None) == -2                      # no nodes
    assert f(2, 257, *ok[2:], *ptrs, None, None) == -2
    assert f(*ok[:6], 0, 1, *ptrs, None, None) == -2                      # depth
    assert f(*ok[:6], 17, 1, *ptrs, None, None) == -2
    assert f(*ok[:4], 0, *ok[5:], *ptrs, None, None) == -2                # no cache room at all
    assert f(*ok[:7], 5, *ptrs, None, None) == -3                         # dtype
    assert f(2, 9, 2, 12, 100, 512, 4, 1, *ptrs, None, None) == -6        # head_dim row not 16-byte units
    assert f(2, 9, 2, 128, 100, 501, 4, 0, *ptrs, None, None) == -6       # hidden row (fp32) ...
    assert f(2, 9, 2, 128, 100, 500, 4, 0, None, *ptrs[1:], None, None) == -1  # ... 500 fp32 is whole units
    assert f(2, 9, 2, 128, 100, 500, 4, 1, *ptrs, None, None) == -6       # 500 bf16 is not
    assert f(*ok, None, *ptrs[1:], None, None) == -1
    assert f(*ok, *ptrs[:8], None, None, None) == -1
    assert f(*ok, *ptrs[:2], FAKE + 8, *ptrs[3:], None, None) == -6
    assert f(*ok, *ptrs[:8], FAKE + 4, None, None) == -6


def test_warp_rejects(lib):
    f = lib.eagle_sampling_warp
    t = [FAKE, FAKE, FAKE, None, None]
    assert f(0, 100, 5, 0.9, 2, 1.0, *t) == 0                 # no rows: nothing to do
    assert f(3, 0, 5, 0.9, 2, 1.0, *t) == -2
    assert f(3, 100, -1, 0.9, 2, 1.0, *t) == -2
    assert f(3, 100, 5, 0.0, 2, 1.0, *t) == -2                # top_p in (0, 1]
    assert f(3, 100, 5, 1.5, 2, 1.0, *t) == -2
    assert f(3, 100, 5, float("nan"), 2, 1.0, *t) == -2
    assert f(3, 100, 5, 0.9, 0, 1.0, *t) == -2                # min_keep >= 1
    assert f(3, 100, 5, 0.9, 101, 1.0, *t) == -2
    assert f(3, 100, 5, 0.9, 6, 1.0, *t) == -2                # top_k below min_keep
    assert f(3, 100, 0, 0.9, 6, -1.0, *t) == -2
    assert f(3, 100, 0, 0.9, 6, 1.0, None, FAKE, FAKE, None, None) == -1


def test_draft_rejects(lib):
    from eagle_draft_tree_expand_amd import _lib as L
    p = L.TreeParams(2, 5003, 4, 3, 14, 1.0, 1, 0)
    dims = L.DraftDims(512, 4, 2, 128, 1408, 400)
    size = lib.eagle_draft_workspace_size(ctypes.byref(p), ctypes.byref(dims))
    assert size > 0 and size % 256 == 0
    assert lib.eagle_draft_workspace_size(ctypes.byref(p), None) == 0
    for bad in (L.DraftDims(500, 4, 2, 128, 1408, 400),      # hidden not a multiple of 128
                L.DraftDims(512, 4, 3, 128, 1408, 400),      # hq % hkv
                L.DraftDims(512, 4, 2, 96, 1408, 400),       # head_dim
                L.DraftDims(512, 4, 2, 128, 1400, 400),      # inter
                L.DraftDims(512, 4, 2, 128, 1408, 0)):       # no prefix cache
        assert lib.eagle_draft_workspace_size(ctypes.byref(p), ctypes.byref(bad)) == 0
    w = L.DraftWeights(*([FAKE] * 7))
    f = lib.eagle_draft_forward
    args = lambda depth, wts=w, ws=size, ptrs=None: (ctypes.byref(p), depth, ctypes.byref(dims), ctypes.byref(wts),  # noqa: E731
                                                     *(ptrs or [FAKE] * 7), FAKE, FAKE, ws, None, None)
    assert f(*args(-1)) == -2
    assert f(*args(4)) == -2                                               # depth < D
    assert f(*args(0, ws=size - 256)) == -4
    assert f(*args(0, wts=L.DraftWeights(*([FAKE] * 6 + [None])))) == -1
    assert f(*args(0, wts=L.DraftWeights(*([FAKE + 8] + [FAKE] * 6)))) == -6
    assert f(*args(0, wts=L.DraftWeights(*([FAKE] * 7 + [FAKE + 16])))) == -6   # z-packed head: 256-aligned
    assert f(*args(0, ws=size - 256, wts=L.DraftWeights(*([FAKE] * 8)))) == -4   # ... accepted otherwise
    assert f(*args(1, ptrs=[FAKE] * 5 + [None, FAKE])) == -1                # pool_tok needed below the root
    assert f(*args(0, ws=size - 256, ptrs=[FAKE] * 5 + [None, FAKE])) == -4  # ... but not at the root
    assert f(*args(0, ptrs=[None] + [FAKE] * 6)) == -1
    e = lib.eagle_expand_depth
    assert e(ctypes.byref(p), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, None) == -2
    assert e(ctypes.byref(p), 0, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, None) == -6
    assert e(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, None, None) == -4
    assert e(ctypes.byref(p), 0, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, None) == -1
    ew = lib.eagle_expand_depth_warped
    wargs = lambda prm=p, depth=0, tk=50, tp=0.9, z=FAKE, bnd=FAKE, ws=1 << 30: (  # noqa: E731
        ctypes.byref(prm), depth, tk, tp, z, bnd, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None, None)
    assert ew(*wargs(depth=4)) == -2
    assert ew(*wargs(prm=L.TreeParams(2, 5003, 4, 3, 14, 0.0, 1, 0))) == -2  # greedy: no warp
    assert ew(*wargs(tk=2)) == -2                                            # top_k below k
    assert ew(*wargs(tp=0.0)) == -2
    assert ew(*wargs(tp=1.5)) == -2
    assert ew(*wargs(bnd=None)) == -1
    assert ew(*wargs(z=FAKE + 4)) == -6
    assert ew(*wargs(ws=1024)) == -4
    g = lib.eagle_expand_finish
    assert g(ctypes.byref(p), *([FAKE] * 11), None, None, None) == -1
    bad_p = L.TreeParams(2, 5003, 4, 0, 14, 1.0, 1, 0)
    assert g(ctypes.byref(bad_p), *([FAKE] * 12), None, None) == -2


def test_static_tree_info_on_the_host(lib):
    """Shape bookkeeping is host-only (no device call): the static shape's slots, depth, largest
    child count and per-slot counts, and the rejection of invalid parent arrays."""
    import synth
    from eagle_draft_tree_expand_amd import _lib, ops
    from oracle import static_tree as ost
    par = synth.get_config("8b_static").static_parent
    info = ost.shape_info(par)
    S, D, kmax, slot_k = ops.static_tree_info(par)
    assert (S, D, kmax) == (info["S"], info["D"], info["kmax"])
    assert slot_k == [int(x) for x in info["slot_k"]]
    for bad in ([0, 0], [-1, 1], [-1, 0, 2], [-1, -1], [-1] + [0] * 17, [-1]):
        with pytest.raises(_lib.EagleError):
            ops.static_tree_info(bad)


def test_expand_static_rejects_mismatched_params(lib):
    import synth
    from eagle_draft_tree_expand_amd import ops
    par = synth.get_config("8b_static").static_parent
    arr = (ctypes.c_int32 * len(par))(*par)
    ptrs = [FAKE] * 14
    good = dict(batch=1, vocab=1000, depth=5, topk=4, m=len(par) - 1)
    for kw in (dict(topk=3), dict(depth=6), dict(m=len(par)), dict(vocab=3)):
        d = dict(good)
        d.update(kw)
        p = ops.tree_params(d["batch"], d["vocab"], d["depth"], d["topk"], d["m"], 1.0)
        assert lib.eagle_expand_static(ctypes.byref(p), len(par), arr, *ptrs, FAKE, 1 << 30, None, None) == -2
    p = ops.tree_params(1, 1000, 5, 4, len(par) - 1, 1.0)
    assert lib.eagle_expand_static(ctypes.byref(p), len(par), arr, *ptrs, FAKE, 100, None, None) == -4
    assert lib.eagle_static_workspace_size(ctypes.byref(p), len(par), arr, 0, 0, 0, 0, 0) > 0
