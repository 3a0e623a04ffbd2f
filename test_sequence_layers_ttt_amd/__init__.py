"""MI355X-native forward scan of a test-time-training (TTT) layer.

The compute lives in libttt_amd.so (HIP kernels for gfx950 behind the C ABI in
include/ttt.h); `ttt` is its Python binding and `inputs` the seeded synthetic
input generator.  The library is loaded on first use.
"""
from . import inputs, ttt  # noqa: F401

__all__ = ["inputs", "ttt"]
