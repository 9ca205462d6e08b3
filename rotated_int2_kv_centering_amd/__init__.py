"""Rotated INT2 KV-cache quantize-append and decode attention for MI355X (gfx950).

The compute path is libkvq.so (hand-written HIP kernels behind the C ABI of
include/kvq.h); ``kvq`` is its ctypes binding and ``KvqLayer`` a small
torch-side holder of one layer's cache buffers.
"""

from . import kvq  # noqa: F401
from .kvq import KvqError, load  # noqa: F401
