"""MI355X (gfx950) engine for the Kimi Delta Attention fixed-size recurrent-state update.

The compute lives in the HIP library ``lib/libkda.so`` (C ABI in ``include/kda.h``); this
package is its Python binding. Importing it fails if the library has not been built.
"""
from ._abi import KDAError, lib  # noqa: F401  (raises ImportError if libkda.so is missing)
from .pool import IndexArray, KDAPool, chunk_for, prefix_hit  # noqa: F401
