"""On-Demand Attention decode step for AMD Instinct MI355X (gfx950).

The compute path is liboda.so (HIP kernels behind the C ABI of
include/oda.h); this package binds it with ctypes (``_lib``) and drives one
decode step over torch-allocated device buffers (``step``).
"""
from ._lib import *  # noqa: F401,F403
from ._lib import EXPORTED, LIB_PATH, OdaError, lib  # noqa: F401
