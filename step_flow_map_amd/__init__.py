"""FlashMap drafting step (one flow-map jump from Gaussian noise to a 16-token
draft, then greedy verification) for MI355X / gfx950.

The compute lives in libflashmap.so (HIP kernels behind the C ABI of
include/flashmap.h); this package is its ctypes binding.
"""
from .binding import *  # noqa: F401,F403
from .binding import Drafter, FlashMapError, lib, verify  # noqa: F401
