"""Decode attention read directly from a low-rank-compressed KV cache on MI355X.

The compute path is liblrkv.so (hand-written HIP for gfx950, C ABI in
include/lrkv.h); this package is its ctypes binding. The library is loaded on
first use, and any call fails with an error if it has not been built
(python -m rank_compressed_kv_amd.build). There is no fallback path.
"""
from .api import *  # noqa: F401,F403
from .api import __all__  # noqa: F401
from ._lib import lib as load_library  # noqa: F401
