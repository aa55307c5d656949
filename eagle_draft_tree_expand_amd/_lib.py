"""ctypes binding of libeagle.so (the C ABI in include/eagle.h).

Argument marshalling only: every computation runs in the HIP kernels of the
library.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libeagle.so")
# the same library built with LDS index checks (build(debug=True))
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libeagle_debug.so")

EAGLE_OK = 0
ERRORS = {-1: "EAGLE_ERR_NULL", -2: "EAGLE_ERR_SHAPE", -3: "EAGLE_ERR_DTYPE",
          -4: "EAGLE_ERR_WORKSPACE", -5: "EAGLE_ERR_LAUNCH", -6: "EAGLE_ERR_ALIGN", -7: "EAGLE_ERR_TOO_LARGE"}
EAGLE_F32, EAGLE_BF16 = 0, 1
EAGLE_W_ROWMAJOR, EAGLE_W_PACKED, EAGLE_W_ZPACKED = 0, 1, 2
STATUS_BITS = {0x1: "TOKEN_RANGE", 0x2: "NONFINITE", 0x4: "ZERO_RESIDUAL", 0x8: "TOPK_RESCAN",
               0x10: "BAD_TREE", 0x20: "CAND_OVERFLOW", 0x40: "SYNC_TIMEOUT",
               0x80: "CACHE_FULL"}

# Every symbol include/eagle.h declares.
EXPORTS = ("eagle_workspace_size", "eagle_workspace_init", "eagle_expand_tree", "eagle_build_tree_mask",
           "eagle_tree_attention", "eagle_lmhead_softmax", "eagle_verify_accept", "eagle_gather_rows",
           "eagle_gather_rows_multi", "eagle_commit_accepted", "eagle_sampling_warp",
           "eagle_expand_tree_warped", "eagle_expand_tree_masked", "eagle_expand_tree_noalloc", "eagle_verify_accept_warped", "eagle_lmhead_packed_bytes",
           "eagle_lmhead_pack_weight", "eagle_lmhead_zpack_bytes", "eagle_lmhead_zpack_weight", "eagle_draft_workspace_size", "eagle_draft_workspace_layout",
           "eagle_draft_forward", "eagle_expand_depth", "eagle_expand_depth_warped",
           "eagle_expand_finish", "eagle_static_tree_info", "eagle_static_workspace_size", "eagle_expand_static",
           "eagle_verify_accept_static", "eagle_lmhead_softmax_compact", "eagle_verify_accept_compact",
           "eagle_error_string", "eagle_abi_version")


class TreeParams(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("vocab", c_int32), ("depth", c_int32), ("topk", c_int32),
                ("m", c_int32), ("temperature", c_float), ("seed", c_uint64), ("round_id", c_uint64)]


class DraftDims(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("hq", c_int32), ("hkv", c_int32), ("head_dim", c_int32), ("inter", c_int32),
                ("max_prefix", c_int32)]


class DraftWeights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("fc", c_void_p), ("qkv", c_void_p), ("o", c_void_p), ("gate_up", c_void_p),
                ("down", c_void_p), ("lm_head", c_void_p), ("lm_head_z", c_void_p)]


class EagleError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} returned {code} ({ERRORS.get(code, 'unknown')})")


_lib = None

_P = c_void_p
_SIGS = {
    "eagle_workspace_size": (c_size_t, [POINTER(TreeParams), c_int32, c_int32, c_int32, c_int32, c_int32]),
    "eagle_workspace_init": (c_int32, [_P, c_size_t, _P]),
    "eagle_expand_tree": (c_int32, [POINTER(TreeParams), _P, _P] + [_P] * 7 + [_P] * 5 + [_P, c_size_t, _P, _P]),
    "eagle_build_tree_mask": (c_int32, [c_int32, c_int32, _P, _P, _P, _P, _P, _P, _P]),
    "eagle_tree_attention": (c_int32, [c_int32] * 7 + [_P] * 4 + [_P, _P, _P, c_float, _P, _P, c_size_t, _P, _P]),
    "eagle_lmhead_softmax": (c_int32, [c_int32] * 4 + [_P, _P, c_int32, c_float, _P, _P, _P, _P, _P, c_size_t, _P,
                                                         _P]),
    "eagle_lmhead_packed_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "eagle_lmhead_pack_weight": (c_int32, [c_int32, c_int32, c_int32, _P, _P, _P]),
    "eagle_lmhead_zpack_bytes": (c_size_t, [c_int32, c_int32]),
    "eagle_lmhead_zpack_weight": (c_int32, [c_int32, c_int32, _P, _P, _P, _P]),
    "eagle_verify_accept": (c_int32, [POINTER(TreeParams)] + [_P] * 16 + [_P, c_size_t, _P, _P]),
    "eagle_gather_rows": (c_int32, [c_int32, c_int32, c_int32, _P, c_int32, _P, _P, _P, _P]),
    "eagle_gather_rows_multi": (c_int32, [c_int32, c_int32, c_int32, c_int32, _P, _P, _P, _P, _P, _P]),
    "eagle_commit_accepted": (c_int32, [c_int32] * 8 + [_P] * 9 + [_P, _P]),
    "eagle_expand_tree_warped": (c_int32, [POINTER(TreeParams), _P, _P, _P] + [_P] * 7 + [_P] * 5 +
                                 [_P, c_size_t, _P, _P]),
    "eagle_expand_tree_masked": (c_int32, [POINTER(TreeParams), _P, _P, _P] + [_P] * 7 + [_P] * 5 + [_P, _P] +
                                 [_P, c_size_t, _P, _P]),
    "eagle_expand_tree_noalloc": (c_int32, [POINTER(TreeParams), _P, _P] + [_P] * 7 + [_P] * 5 + [_P, _P]),
    "eagle_verify_accept_warped": (c_int32, [POINTER(TreeParams), _P, _P] + [_P] * 16 + [_P, c_size_t, _P, _P]),
    "eagle_sampling_warp": (c_int32, [c_int32, c_int32, c_int32, c_float, c_int32, c_float, _P, _P, _P, _P, _P]),
    "eagle_draft_workspace_size": (c_size_t, [POINTER(TreeParams), POINTER(DraftDims)]),
    "eagle_draft_workspace_layout": (c_int32, [POINTER(TreeParams), POINTER(DraftDims), POINTER(c_size_t), c_int32]),
    "eagle_draft_forward": (c_int32, [POINTER(TreeParams), c_int32, POINTER(DraftDims), POINTER(DraftWeights)] +
                            [_P] * 8 + [_P, c_size_t, _P, _P]),
    "eagle_expand_depth": (c_int32, [POINTER(TreeParams), c_int32] + [_P] * 5 + [_P, c_size_t, _P, _P]),
    "eagle_expand_depth_warped": (c_int32, [POINTER(TreeParams), c_int32, c_int32, c_float] + [_P] * 6 +
                                  [_P, c_size_t, _P, _P]),
    "eagle_expand_finish": (c_int32, [POINTER(TreeParams)] + [_P] * 12 + [_P, _P]),
    "eagle_static_tree_info": (c_int32, [c_int32, _P, _P, _P, _P, _P]),
    "eagle_static_workspace_size": (c_size_t, [POINTER(TreeParams), c_int32, _P] + [c_int32] * 5),
    "eagle_expand_static": (c_int32, [POINTER(TreeParams), c_int32, _P, _P, _P] + [_P] * 7 + [_P] * 5 +
                            [_P, c_size_t, _P, _P]),
    "eagle_verify_accept_static": (c_int32, [POINTER(TreeParams), c_int32] + [_P] * 16 + [_P, c_size_t, _P, _P]),
    "eagle_lmhead_softmax_compact": (c_int32, [c_int32] * 3 + [_P, _P, c_int32, c_float] + [_P] * 4 +
                                     [_P, c_size_t, _P, _P]),
    "eagle_verify_accept_compact": (c_int32, [POINTER(TreeParams), c_int32] + [_P] * 17 + [_P, c_size_t, _P, _P]),
    "eagle_error_string": (c_char_p, [c_int32]),
    "eagle_abi_version": (c_int32, []),
}


def load(path: str = LIB_PATH):
    """Load libeagle.so (cached).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libeagle.so not found at {path}; build it first "
                           "(python -m eagle_draft_tree_expand_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


@contextlib.contextmanager
def using(path: str):
    """Route every call of the binding to the library at `path` (another build,
    e.g. DEBUG_LIB_PATH) inside the block, and back to the previous one after
    it.  Not thread-safe: for tests."""
    global _lib
    prev = _lib
    _lib = None
    try:
        yield load(path)
    finally:
        _lib = prev


def check(fn_name: str, code: int):
    if code != EAGLE_OK:
        raise EagleError(fn_name, code)
