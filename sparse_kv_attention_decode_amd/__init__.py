"""SFI (Slow-Fast Inference) decode hot path for MI355X (gfx950).

The kernels live in libsfi.so (csrc/*.hip, C ABI in include/sfi.h); `lib` is the thin
ctypes binding and `engine` drives one decode step over many layers on two HIP streams.
"""
from . import lib  # noqa: F401
