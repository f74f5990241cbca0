"""MI355X-native Hadamard-rotated W4A4 Q4_0 matmul.

The compute lives in libw4a4.so (hand-written HIP for gfx950, C ABI in
include/w4a4.h); this package is its thin Python binding plus the seeded
synthetic-input generator.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "ops"]


def __getattr__(name):
    # the binding imports torch; load it only when asked for
    if name == "ops":
        from . import _lib
        return _lib
    raise AttributeError(name)
