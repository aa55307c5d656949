"""MI355X-native EAGLE draft-tree round: C-ABI library (libeagle.so) + binding.

The product path is the HIP library under csrc/ (include/eagle.h is its ABI);
this package only builds it and marshals arguments to it.
"""
from ._lib import EagleError, LIB_PATH, TreeParams, load  # noqa: F401

__all__ = ["EagleError", "LIB_PATH", "TreeParams", "load"]
