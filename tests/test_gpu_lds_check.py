"""The debug library (lib/libeagle_debug.so, built with EAGLE_LDS_CHECK): the
tree assembly and the acceptance walk check every LDS index that is computed
from data (layer ranks, slots, pool and flat indices, the walk's node) and
set EAGLE_STATUS_LDS_INDEX for one outside its array.  Whole rounds on
several shapes through the debug library must set no such bit and give the
release library's outputs bit for bit (a check that passes changes nothing)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LDS_INDEX = 0x100


def _round(cfg, T):
    from eagle_draft_tree_expand_amd import round as dround
    inp = synth.make_inputs(cfg)
    wts = dround.DeviceWeights(inp)
    data = dround.DeviceInputs(inp)
    data.set_rows(inp.iid_draft_rows())
    dr = dround.DeviceRound(cfg)
    dr.step(wts, data, T)
    return dr.host()


@pytest.mark.parametrize("name,kw,T", [
    ("tiny", {}, 1.0),
    ("mid_bf16", {}, 1.0),
    ("mid_bf16", {}, 0.0),
    ("mid_bf16", dict(k=16, D=5, m=70), 1.0),   # k > 11: the general layer step
    ("mid_static", dict(B=3), 1.0),
    ("8b", {}, 1.0),
])
def test_debug_library_lds_indices(name, kw, T):
    from eagle_draft_tree_expand_amd import _lib
    cfg = synth.get_config(name).with_(**kw)
    rel = _round(cfg, T)
    with _lib.using(_lib.DEBUG_LIB_PATH):
        dbg = _round(cfg, T)
    assert dbg["status"] & LDS_INDEX == 0, hex(dbg["status"])
    assert dbg["status"] == rel["status"]
    diff = [k for k in rel if k != "status" and np.asarray(rel[k]).tobytes() != np.asarray(dbg[k]).tobytes()]
    assert not diff, diff
